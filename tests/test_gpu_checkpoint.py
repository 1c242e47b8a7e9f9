"""GPU parity of the soft codeword's checkpoint-and-recompute memory mode, through the C-ABI.

Given a workspace of bcjr_workspace_bytes_min (smaller than the full tape), bcjr_soft_codeword keeps every c-th forward
message row, c = ceil(sqrt(n)).  The backward pass rebuilds each segment's rows from its checkpoint, using the stored
per-step normalisers, before it consumes them.  Checked here:

* the soft codeword and ln Z against the oracle, within the general-trellis bars;
* bit-identity with the full-tape mode of the same kernel (every (k, V) other than k = 2, V = 1, where the full tape
  runs the tuned kernel instead).  The recomputed rows repeat the first pass's arithmetic, so the two modes agree
  bit for bit.

Cases cover n not a multiple of c, n = 1 and 2, n = 4096, sigma mode, and batches larger than the grid.
"""
import numpy as np
import pytest
import torch

import differentiable_bcjr_amd as dba
import workloads
from differentiable_bcjr_amd import abi
from test_gpu_general_trellis import _scale, _sigma_n, _vin, vsoft_tol
from test_gpu_parity import _t, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _soft(w, c, L, k, T, s, dev, checkpoint):
    return dba.soft_codeword(_t(w, dev), _t(c, dev), L, k, T, _t(s, dev), return_log_z=True, checkpoint=checkpoint)


# (L, k, V, B, n)
CASES = [(8, 2, 1, 5, 37), (8, 2, 1, 4, 40), (9, 3, 2, 3, 50), (6, 3, 1, 4, 1), (8, 1, 2, 4, 2), (12, 1, 1, 3, 100),
         (13, 4, 1, 2, 26), (16, 2, 1, 2, 40), (16, 3, 1, 2, 33), (16, 4, 2, 2, 20), (16, 1, 1, 1, 17)]


@pytest.mark.parametrize("L,k,V,B,n", CASES, ids=[f"L{c[0]}k{c[1]}V{c[2]}B{c[3]}n{c[4]}" for c in CASES])
@pytest.mark.parametrize("sigma", [False, True])
def test_checkpoint_mode_matches_oracle(oracle_mod, dev, L, k, V, B, n, sigma):
    if sigma:
        n = _sigma_n(L, k, n)
    w, c, _, s = _vin(L, V, B, n, 6100 + 31 * L + 7 * k + V + n, sigma)
    need_min = abi.bcjr_workspace_bytes_min(abi.BCJR_OP_SOFT, B, n, L, k, V)
    full = abi.bcjr_workspace_bytes_v(abi.BCJR_OP_SOFT, B, n, L, k, V)
    assert need_min <= full
    for T in [1.0, 0.1, 0.05]:
        ws, lz = _soft(w, c, L, k, T, s, dev, checkpoint=True)
        rws, rlz = oracle_mod.soft(w, c, L, k, T, sigma=s)
        e = rel_err(ws.cpu().numpy(), rws)
        el = float(np.max(np.abs(lz.cpu().numpy() - rlz) / np.maximum(np.abs(rlz), 1.0)))
        print(f"checkpoint L{L} k{k} V{V} B{B} n{n} sigma={sigma} T={T}: {e:.2e}, ln Z {el:.2e} "
              f"(workspace {need_min} of {full} bytes)", flush=True)
        assert e <= vsoft_tol(T, sigma, k, V) and el <= 1e-5
        if (k, V) != (2, 1):
            ws_t, lz_t = _soft(w, c, L, k, T, s, dev, checkpoint=False)
            assert torch.equal(ws, ws_t) and torch.equal(lz, lz_t)


@pytest.mark.parametrize("L,k,V,B,n", [(8, 3, 2, 4300, 9), (16, 2, 1, 270, 5)])
def test_checkpoint_mode_several_sequences_per_workgroup(oracle_mod, dev, L, k, V, B, n):
    w, c, _, _ = _vin(L, V, B, n, 6200 + L)
    T = 0.1
    ws, _ = _soft(w, c, L, k, T, None, dev, checkpoint=True)
    rws, _ = oracle_mod.soft(w, c, L, k, T)
    assert rel_err(ws.cpu().numpy(), rws) <= 1e-5 * _scale(k, V)


@pytest.mark.parametrize("L,k,V", [(10, 2, 1), (9, 3, 2)])
def test_checkpoint_mode_longest_sequences(oracle_mod, dev, L, k, V):
    """n = 4096: 65 checkpoints of 64-step segments instead of 4097 rows."""
    n, B, T = 4096, 2, 0.3
    w, c, _, _ = _vin(L, V, B, n, 6300 + L)
    ws, lz = _soft(w, c, L, k, T, None, dev, checkpoint=True)
    rws, rlz = oracle_mod.soft(w, c, L, k, T)
    assert rel_err(ws.cpu().numpy(), rws) <= 1e-5 * _scale(k, V)
    assert float(np.max(np.abs(lz.cpu().numpy() - rlz) / np.abs(rlz))) <= 1e-5


def test_checkpoint_mode_headline_workload_rows(oracle_mod, dev):
    """The 1024x1024 workload (L = 16, k = 2, n = 256) in the checkpoint mode: 33 message rows per in-flight sequence
    instead of 257; sampled rows against the oracle."""
    wl = workloads.WORKLOADS[2]
    c, w = wl.codebook(), wl.weights()
    T = 0.1
    ws, _ = dba.soft_codeword(_t(w, dev), _t(c, dev), wl.L, wl.k, T, return_log_z=True, checkpoint=True)
    rows = wl.sample_rows(3)
    rws, _ = oracle_mod.soft(w[rows], c, wl.L, wl.k, T)
    e = rel_err(ws.cpu().numpy()[rows], rws)
    print(f"checkpoint mode, {wl.name}: soft {e:.2e}", flush=True)
    assert e <= 1e-5
