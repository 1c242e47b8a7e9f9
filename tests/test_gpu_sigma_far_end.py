"""Boundary-state mode with a last weight far from every codeword: the branch cost of s_n = sigma is hundreds to
thousands in log2 units, the largest value the backward pass starts from.

With s_n = sigma the posterior at the last step is the indicator of sigma, and every earlier step's backward message
carries theta_{n-1}(sigma) as a common offset (gist.science Technical Summary, Core Mechanism: the posterior of each
step under the Boltzmann path weights).  The kernels keep that offset out of the messages, so the next step's branch
terms keep their own precision.  These cases put it at 1e2..2e3: the soft codeword, ln Z, the weights' gradient and
the codebook gradient must still meet their one-ulp conditioning bars against the oracle, on the tuned k = 2 kernels
(several sequences per block at small L, one per block at L = 16) and on the general trellis."""
import numpy as np
import pytest
import torch

import cases
import differentiable_bcjr_amd as dba
import parity

pytestmark = pytest.mark.gpu

# (L, k, V, B, n): n counts weights (n / V steps)
CASES = [(6, 2, 1, 9, 8), (8, 2, 1, 5, 12), (12, 2, 1, 3, 10), (16, 2, 1, 2, 10), (9, 3, 1, 4, 6), (8, 4, 2, 3, 12)]
IDS = cases.ids(CASES)
FAR = 6.0   # the codebook has unit variance: (FAR - c)^2 / T is ~1e2..2e3 in log2 units at T = 0.1, 0.05


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _t(a, dev):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _inputs(L, k, V, B, n, seed):
    w, c, g, s = cases.vin(L, V, B, cases.sigma_n(L, k, n // V), seed, True)   # n // V steps
    w[:, -V:] = FAR   # the last step's weights
    return w, c, g, s


@pytest.mark.parametrize("L,k,V,B,n", CASES, ids=IDS)
def test_far_end_soft_and_grad(oracle_mod, dev, L, k, V, B, n):
    w, c, g, s = _inputs(L, k, V, B, n, 8800 + 13 * L + k + V)
    ok = True
    for T in (0.1, 0.05):
        print(f"far end L{L} k{k} V{V} B{B} n{w.shape[1]} T={T}:", flush=True)
        ws, lz = dba.soft_codeword(_t(w, dev), _t(c, dev), L, k, T, _t(s, dev), return_log_z=True)
        ok &= parity.soft_ok(oracle_mod, ws, lz, w, c, L, k, T, sigma=s, label="soft ")
        gr, ws2 = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T, _t(s, dev), return_w_soft=True)
        ok &= parity.grad_ok(oracle_mod, gr, ws2, w, c, g, L, k, T, sigma=s, label="grad ")
    assert ok


@pytest.mark.parametrize("L,k,V,B,n", CASES, ids=IDS)
def test_far_end_codebook_grad(oracle_mod, dev, L, k, V, B, n):
    w, c, g, s = _inputs(L, k, V, B, n, 8900 + 13 * L + k + V)
    ok = True
    for T in (0.1, 0.05):
        print(f"far end codebook grad L{L} k{k} V{V} B{B} n{w.shape[1]} T={T}:", flush=True)
        gc, gw, ws = dba.soft_codeword_grad_codebook(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T, _t(s, dev),
                                                     return_w_soft=True)
        ok &= parity.codebook_grad_ok(oracle_mod, gc, gw, ws, w, c, g, L, k, T, sigma=s)
    assert ok
