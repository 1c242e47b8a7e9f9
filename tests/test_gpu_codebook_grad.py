"""GPU parity of the codebook gradient dL/dc (bcjr_soft_codeword_grad_codebook, through the C-ABI) against the oracle.

dL/dc(v) = sum_b sum_u p(s_u = v) [g_u + (2/T)(w_u - c(v))(E[F | s_u = v] - E[F])] is a vector over the 2^L states,
summed over the batch.  Its entries span many orders of magnitude (states far from every weight have
vanishing posterior), so it is compared as a vector: ||x - ref||_2 / ||ref||_2 and max |x - ref| / max |ref|, each
within max(1e-5, kappa), kappa its one-ulp conditioning computed by the oracle (tests/parity.py).  The weights'
gradient and the soft codeword that the same call returns are held to the gradient op's bars.
"""
import numpy as np
import pytest
import torch

import differentiable_bcjr_amd as dba
import parity
import workloads
from differentiable_bcjr_amd import abi
from parity import norm_err
from test_gpu_parity import _inputs, _t

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


# (L, B, n): every geometry, ragged batches across the sequences-per-block packing of small L, n = 1 and 2
CASES = [(4, 16, 6), (4, 67, 5), (5, 7, 9), (6, 5, 33), (8, 16, 64), (8, 3, 1), (8, 2, 2), (9, 5, 17), (10, 9, 40),
         (12, 3, 20), (13, 2, 11), (14, 2, 12), (15, 2, 10), (16, 2, 8)]


@pytest.mark.parametrize("L,B,n", CASES)
@pytest.mark.parametrize("sigma", [False, True])
def test_codebook_grad_matches_oracle(oracle_mod, dev, L, B, n, sigma):
    if sigma and n < (L + 1) // 2:
        n = (L + 1) // 2 + 1   # every sigma reachable
    w, c, g, s = _inputs(L, B, n, 900 + 11 * L + n, sigma)
    ok = True
    for T in [1.0, 0.1, 0.05]:
        gc, gw, ws = dba.soft_codeword_grad_codebook(_t(w, dev), _t(c, dev), _t(g, dev), L, 2, T, _t(s, dev),
                                                     return_w_soft=True)
        print(f"L{L} B{B} n{n} T{T} sigma={sigma}:", flush=True)
        ok &= parity.codebook_grad_ok(oracle_mod, gc, gw, ws, w, c, g, L, 2, T, s)
    assert ok


@pytest.mark.parametrize("L", [6, 12, 16])
@pytest.mark.parametrize("sigma", [False, True])
def test_codebook_grad_optional_outputs_and_plain_gradient_agree(dev, L, sigma):
    """grad_w and w_soft are optional (sigma mode included, where the last step's weight gradient is set apart); when
    asked for they match what the gradient op returns."""
    B, n, T = 9, 30, 0.2
    w, c, g, s = _inputs(L, B, n, 77 + L, sigma)
    wt, ct, gt, st = _t(w, dev), _t(c, dev), _t(g, dev), _t(s, dev)
    only = dba.soft_codeword_grad_codebook(wt, ct, gt, L, 2, T, st, return_grad_w=False)
    gc, gw, ws = dba.soft_codeword_grad_codebook(wt, ct, gt, L, 2, T, st, return_w_soft=True)
    assert torch.equal(only, gc)
    pgw, pws = dba.soft_codeword_grad(wt, ct, gt, L, 2, T, st, return_w_soft=True)
    assert norm_err(gw.cpu().numpy(), pgw.cpu().numpy()) <= 1e-6
    assert norm_err(ws.cpu().numpy(), pws.cpu().numpy()) <= 1e-6


def test_codebook_grad_is_nan_without_an_admissible_path(dev):
    L, B, n = 8, 5, 2   # sigma mode needs n >= L/k steps
    w, c, g, s = _inputs(L, B, n, 5, True)
    s[:] = np.array([1, 2, 3, 200, 77], np.int32)
    gc, gw = dba.soft_codeword_grad_codebook(_t(w, dev), _t(c, dev), _t(g, dev), L, 2, 0.5, _t(s, dev))
    assert torch.isnan(gc).all() and torch.isnan(gw).all()


def test_codebook_grad_headline_rows(oracle_mod, dev):
    """The 2^16-state, 256-step workload: sampled rows of the 1024x1024 matrix at T = 0.1 and 1."""
    wl = workloads.WORKLOADS[2]
    c, w, g = wl.codebook(), wl.weights(), wl.upstream_grad()
    rows = wl.sample_rows(2)
    ok = True
    for T in [0.1, 1.0]:
        gc, gw = dba.soft_codeword_grad_codebook(_t(w[rows], dev), _t(c, dev), _t(g[rows], dev), wl.L, wl.k, T)
        print(f"headline rows {rows.tolist()} T{T}:", flush=True)
        ok &= parity.codebook_grad_ok(oracle_mod, gc, gw, None, w[rows], c, g[rows], wl.L, wl.k, T)
    assert ok


def test_codebook_grad_full_batch_properties(dev):
    """All 4096 sequences of the 1024x1024 matrix: determinism, additivity over the batch, and the exact identity
    sum_v dL/dc(v) + sum_u dL/dw_u = sum_t g_t (a common shift of codebook and weights leaves the measure alone)."""
    wl = workloads.WORKLOADS[2]
    c, w, g = wl.codebook(), wl.weights(), wl.upstream_grad()
    T = 0.1
    wt, ct, gt = _t(w, dev), _t(c, dev), _t(g, dev)
    gc, gw = dba.soft_codeword_grad_codebook(wt, ct, gt, wl.L, wl.k, T)
    gc2, gw2 = dba.soft_codeword_grad_codebook(wt, ct, gt, wl.L, wl.k, T)
    assert torch.equal(gc, gc2) and torch.equal(gw, gw2)
    h = w.shape[0] // 2
    ga = dba.soft_codeword_grad_codebook(wt[:h], ct, gt[:h], wl.L, wl.k, T, return_grad_w=False)
    gb = dba.soft_codeword_grad_codebook(wt[h:], ct, gt[h:], wl.L, wl.k, T, return_grad_w=False)
    x = gc.double().cpu().numpy()
    e_add = norm_err(x, (ga.double() + gb.double()).cpu().numpy())
    y = gw.double().cpu().numpy()
    lhs, rhs = x.sum() + y.sum(), g.astype(np.float64).sum()
    scale = np.abs(x).sum() + np.abs(y).sum() + abs(rhs)
    print(f"full batch: additivity {e_add:.2e}, shift identity {abs(lhs - rhs) / scale:.2e} of the summed magnitudes",
          flush=True)
    assert e_add <= 1e-6
    assert abs(lhs - rhs) <= 1e-6 * scale


def test_codebook_grad_graph_replays_match_eager(dev):
    L, B, n, T = 12, 40, 24, 0.2
    w, c, g, _ = _inputs(L, B, n, 91)
    wt, ct, gt = _t(w, dev), _t(c, dev), _t(g, dev)
    nbytes = abi.bcjr_workspace_bytes(abi.BCJR_OP_GRAD_CODEBOOK, B, n, L, 2)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    def call(gc, gw, stream):
        rc = abi.bcjr_soft_codeword_grad_codebook(wt.data_ptr(), ct.data_ptr(), B, n, L, 2, T, None, gt.data_ptr(),
                                                  gc.data_ptr(), gw.data_ptr(), None, ws.data_ptr(), nbytes,
                                                  stream.cuda_stream)
        assert rc == 0

    eager = (torch.empty(1 << L, device=dev), torch.empty(B, n, device=dev))
    call(*eager, torch.cuda.current_stream(dev))
    torch.cuda.synchronize()
    outs = (torch.empty(1 << L, device=dev), torch.empty(B, n, device=dev))
    side = torch.cuda.Stream(dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call(*outs, side)
    for rep in range(3):
        for o in outs:
            o.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a, b), f"replay {rep} differs from the eager call"


@pytest.mark.parametrize("sigma", [False, True])
def test_soft_quantize_codebook_autograd(oracle_mod, dev, sigma):
    """Autograd through soft_quantize with a trainable codebook: both gradients exact."""
    L, B, n, T = 10, 6, 24, 0.1
    w, c, g, s = _inputs(L, B, n, 62, sigma)
    wt = _t(w, dev).requires_grad_(True)
    ct = _t(c, dev).requires_grad_(True)
    (dba.soft_quantize(wt, ct, L, 2, T, _t(s, dev)) * _t(g, dev)).sum().backward()
    assert parity.codebook_grad_ok(oracle_mod, ct.grad, wt.grad, None, w, c, g, L, 2, T, s)
    c_only = _t(c, dev).requires_grad_(True)
    (dba.soft_quantize(_t(w, dev), c_only, L, 2, T, _t(s, dev)) * _t(g, dev)).sum().backward()
    assert torch.equal(c_only.grad, ct.grad)


def _random_cases(count=24, seed=4048):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for i in range(count):
        L = int(rng.integers(4, 17))
        n = int(rng.integers(1, 65)) if L <= 12 else int(rng.integers(1, 17))
        B = int(rng.integers(1, 41)) if L <= 12 else int(rng.integers(1, 4))
        T = float(rng.choice([1.0, 0.3, 0.1, 0.05]))
        sigma = bool(rng.integers(0, 2)) and n >= (L + 1) // 2
        cases.append((i, L, B, n, T, sigma))
    return cases


@pytest.mark.parametrize("i,L,B,n,T,sigma", _random_cases())
def test_codebook_grad_random_configuration(oracle_mod, dev, i, L, B, n, T, sigma):
    w, c, g, s = _inputs(L, B, n, 7000 + i, sigma)
    gc, gw = dba.soft_codeword_grad_codebook(_t(w, dev), _t(c, dev), _t(g, dev), L, 2, T, _t(s, dev))
    print(f"random {i}: L{L} B{B} n{n} T{T} sigma={sigma}:", flush=True)
    assert parity.codebook_grad_ok(oracle_mod, gc, gw, None, w, c, g, L, 2, T, s)
