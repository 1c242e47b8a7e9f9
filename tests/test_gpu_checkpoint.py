"""GPU parity of the checkpoint-and-recompute memory mode, through the C-ABI.

Given a workspace of bcjr_workspace_bytes_min (smaller than the full tape), the soft codeword and the two gradients
keep every c-th forward message row, c = ceil(sqrt(n)).  The gradients keep both of their forward messages (R~ and
Q^) this way.  The backward pass rebuilds each segment's rows from its checkpoint, using the stored per-step
normalisers (and Q input offsets), before it consumes them.  Checked here:

* the outputs against the oracle, within the conditioning bars of tests/parity.py; at the 1024x1024 workload on the
  64 stored rows of the full-size references;
* bit-identity with the full-tape mode of the same kernels, for every (k, V): each kernel family, the tuned k = 2
  one included, has its own checkpoint mode.  The recomputed rows repeat the first pass's arithmetic, so the two modes
  agree bit for bit.

Cases cover n not a multiple of c, n <= 3 (where checkpoints save nothing and the full tape runs), n = 4096,
sigma mode, and batches larger than the grid.
"""
import numpy as np
import pytest
import torch

import differentiable_bcjr_amd as dba
import cases
import parity
import workloads
from differentiable_bcjr_amd import abi
from cases import sigma_n as _sigma_n, vin as _vin
from test_gpu_parity import _golden_grad, _golden_soft, _t

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _soft(w, c, L, k, T, s, dev, checkpoint):
    return dba.soft_codeword(_t(w, dev), _t(c, dev), L, k, T, _t(s, dev), return_log_z=True, checkpoint=checkpoint)


# (L, k, V, B, n)
CASES = cases.CHECKPOINT


@pytest.mark.parametrize("L,k,V,B,n", CASES, ids=[f"L{c[0]}k{c[1]}V{c[2]}B{c[3]}n{c[4]}" for c in CASES])
@pytest.mark.parametrize("sigma", [False, True])
def test_checkpoint_mode_matches_oracle(oracle_mod, dev, L, k, V, B, n, sigma):
    if sigma:
        n = _sigma_n(L, k, n)
    w, c, _, s = _vin(L, V, B, n, 6100 + 31 * L + 7 * k + V + n, sigma)
    need_min = abi.bcjr_workspace_bytes_min(abi.BCJR_OP_SOFT, B, n, L, k, V)
    full = abi.bcjr_workspace_bytes_v(abi.BCJR_OP_SOFT, B, n, L, k, V)
    assert need_min <= full
    ok = True
    for T in [1.0, 0.1, 0.05]:
        ws, lz = _soft(w, c, L, k, T, s, dev, checkpoint=True)
        print(f"checkpoint L{L} k{k} V{V} B{B} n{n} sigma={sigma} T={T} (workspace {need_min} of {full} bytes):",
              flush=True)
        ok &= parity.soft_ok(oracle_mod, ws, lz, w, c, L, k, T, s)
        # every (k, V), the k = 2 kernel included, has a checkpoint mode of the kernel that runs its full tape
        ws_t, lz_t = _soft(w, c, L, k, T, s, dev, checkpoint=False)
        assert torch.equal(ws, ws_t) and torch.equal(lz, lz_t)
    assert ok


@pytest.mark.parametrize("L,k,V,B,n", cases.CHECKPOINT_SOFT_SEVERAL)
def test_checkpoint_mode_several_sequences_per_workgroup(oracle_mod, dev, L, k, V, B, n):
    w, c, _, _ = _vin(L, V, B, n, 6200 + L)
    T = 0.1
    ws, _ = _soft(w, c, L, k, T, None, dev, checkpoint=True)
    assert parity.soft_ok(oracle_mod, ws, None, w, c, L, k, T)


@pytest.mark.parametrize("L,k,V", [(10, 2, 1), (9, 3, 2)])
def test_checkpoint_mode_longest_sequences(oracle_mod, dev, L, k, V):
    """n = 4096: 65 checkpoints of 64-step segments instead of 4097 rows."""
    n, B, T = 4096, 2, 0.3
    w, c, _, _ = _vin(L, V, B, n, 6300 + L)
    ws, lz = _soft(w, c, L, k, T, None, dev, checkpoint=True)
    assert parity.soft_ok(oracle_mod, ws, lz, w, c, L, k, T)


def test_checkpoint_mode_headline_workload_rows(dev):
    """The 1024x1024 workload (L = 16, k = 2, n = 256) in the checkpoint mode: 33 message rows per in-flight sequence
    instead of 257; the 64 stored rows against the oracle's answers."""
    wl = workloads.WORKLOADS[2]
    G = parity.load_golden(2)
    c, w = wl.codebook(), wl.weights()
    T = 0.1
    ws, lz = dba.soft_codeword(_t(w, dev), _t(c, dev), wl.L, wl.k, T, return_log_z=True, checkpoint=True)
    print(f"checkpoint mode, {wl.name}:", flush=True)
    assert _golden_soft(G, ws, lz, T)
    ws_t, lz_t = dba.soft_codeword(_t(w, dev), _t(c, dev), wl.L, wl.k, T, return_log_z=True)
    assert torch.equal(ws, ws_t) and torch.equal(lz, lz_t)


# ------------------------------------------------------------------------------- the gradients' checkpoint mode

GRAD_CASES = CASES
GRAD_IDS = [f"L{c[0]}k{c[1]}V{c[2]}B{c[3]}n{c[4]}" for c in GRAD_CASES]


def _grad(w, c, g, L, k, T, s, dev, checkpoint):
    return dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T, _t(s, dev), return_w_soft=True,
                                  checkpoint=checkpoint)


def _gc(w, c, g, L, k, T, s, dev, checkpoint):
    return dba.soft_codeword_grad_codebook(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T, _t(s, dev),
                                           return_w_soft=True, checkpoint=checkpoint)


def _uses_checkpoints(op, B, n, L, k, V):
    return abi.bcjr_workspace_bytes_min(op, B, n, L, k, V) < abi.bcjr_workspace_bytes_v(op, B, n, L, k, V)


@pytest.mark.parametrize("L,k,V,B,n", GRAD_CASES, ids=GRAD_IDS)
@pytest.mark.parametrize("sigma", [False, True])
def test_grad_checkpoint_mode_matches_oracle(oracle_mod, dev, L, k, V, B, n, sigma):
    if sigma:
        n = _sigma_n(L, k, n)
    w, c, g, s = _vin(L, V, B, n, 6400 + 31 * L + 7 * k + V + n, sigma)
    # n <= 3: the 256-byte rounding leaves the checkpoint slot no smaller, and the full tape runs
    assert _uses_checkpoints(abi.BCJR_OP_GRAD, B, n, L, k, V) == (n > 3)
    assert _uses_checkpoints(abi.BCJR_OP_GRAD_CODEBOOK, B, n, L, k, V) == (n > 3)
    ok = True
    for T in [1.0, 0.1, 0.05]:
        gr, ws = _grad(w, c, g, L, k, T, s, dev, checkpoint=True)
        print(f"grad checkpoint L{L} k{k} V{V} B{B} n{n} sigma={sigma} T={T}:", flush=True)
        ok &= parity.grad_ok(oracle_mod, gr, ws, w, c, g, L, k, T, s)
        gr_t, ws_t = _grad(w, c, g, L, k, T, s, dev, checkpoint=False)
        assert torch.equal(gr, gr_t) and torch.equal(ws, ws_t)
    assert ok


@pytest.mark.parametrize("L,k,V,B,n", GRAD_CASES, ids=GRAD_IDS)
@pytest.mark.parametrize("sigma", [False, True])
def test_codebook_grad_checkpoint_mode_matches_oracle(oracle_mod, dev, L, k, V, B, n, sigma):
    if sigma:
        n = _sigma_n(L, k, n)
    w, c, g, s = _vin(L, V, B, n, 6500 + 31 * L + 7 * k + V + n, sigma)
    ok = True
    for T in [1.0, 0.1]:
        gc, gw, ws = _gc(w, c, g, L, k, T, s, dev, checkpoint=True)
        print(f"codebook grad checkpoint L{L} k{k} V{V} B{B} n{n} sigma={sigma} T={T}:", flush=True)
        ok &= parity.codebook_grad_ok(oracle_mod, gc, gw, ws, w, c, g, L, k, T, s)
        gc_t, gw_t, ws_t = _gc(w, c, g, L, k, T, s, dev, checkpoint=False)
        assert torch.equal(gc, gc_t) and torch.equal(gw, gw_t) and torch.equal(ws, ws_t)
    assert ok


@pytest.mark.parametrize("L,k,V,B,n", cases.CHECKPOINT_GRAD_SEVERAL)
def test_grad_checkpoint_mode_several_sequences_per_workgroup(oracle_mod, dev, L, k, V, B, n):
    """Each workgroup's slot, its checkpoint rows, offsets and saved messages, reused by the next sequence."""
    w, c, g, _ = _vin(L, V, B, n, 6600 + L + k)
    T = 0.1
    gr, _ = _grad(w, c, g, L, k, T, None, dev, checkpoint=True)
    ok = parity.grad_ok(oracle_mod, gr, None, w, c, g, L, k, T)
    gc, _, _ = _gc(w, c, g, L, k, T, None, dev, checkpoint=True)
    ok &= parity.codebook_grad_ok(oracle_mod, gc, None, None, w, c, g, L, k, T)
    assert ok


@pytest.mark.parametrize("L,k,V", [(10, 2, 1), (9, 3, 2)])
def test_grad_checkpoint_mode_longest_sequences(oracle_mod, dev, L, k, V):
    """n = 4096: 65 checkpoints of 64-step segments for each of the two forward messages."""
    n, B, T = 4096, 2, 0.3
    w, c, g, _ = _vin(L, V, B, n, 6700 + L)
    gr, ws = _grad(w, c, g, L, k, T, None, dev, checkpoint=True)
    assert parity.grad_ok(oracle_mod, gr, ws, w, c, g, L, k, T)


def test_grad_checkpoint_mode_headline_workload_rows(dev):
    """The 1024x1024 workload (L = 16, k = 2, n = 256) in the checkpoint mode: 33 rows of each forward message per
    in-flight sequence instead of 257; the 64 stored rows against the oracle's answers."""
    wl = workloads.WORKLOADS[2]
    G = parity.load_golden(2)
    c, w, g = wl.codebook(), wl.weights(), wl.upstream_grad()
    T = 0.1
    gr, ws = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), wl.L, wl.k, T, return_w_soft=True,
                                    checkpoint=True)
    assert bool(torch.isfinite(gr).all())
    print(f"grad checkpoint mode, {wl.name}:", flush=True)
    assert _golden_grad(G, gr, ws, g, c, T)
    gr_t, ws_t = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), wl.L, wl.k, T, return_w_soft=True)
    assert torch.equal(gr, gr_t) and torch.equal(ws, ws_t)


@pytest.mark.parametrize("L,k,V", [(9, 3, 2), (10, 2, 1)])
def test_soft_quantize_checkpoint_mode(oracle_mod, dev, L, k, V):
    """Autograd through soft_quantize with checkpoint=True: the forward, dL/dw and dL/dc with the smallest
    workspaces: bit-identical to the full-tape mode, and against the oracle."""
    B, n, T = 5, 40, 0.2
    w, c, g, _ = _vin(L, V, B, n, 6800 + L)
    outs = {}
    for ck in (False, True):
        wt = _t(w, dev).requires_grad_(True)
        ct = _t(c, dev).requires_grad_(True)
        out = dba.soft_quantize(wt, ct, L, k, T, checkpoint=ck)
        (out * _t(g, dev)).sum().backward()
        outs[ck] = (out.detach(), wt.grad, ct.grad)
    for a, b in zip(outs[False], outs[True]):
        assert torch.equal(a, b)
    ws, gw, gc = outs[True]
    assert parity.codebook_grad_ok(oracle_mod, gc, gw, ws, w, c, g, L, k, T)
