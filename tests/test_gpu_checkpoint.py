"""GPU parity of the checkpoint-and-recompute memory mode, through the C-ABI.

Given a workspace of bcjr_workspace_bytes_min (smaller than the full tape), the soft codeword and the two gradients
keep every c-th forward message row, c = ceil(sqrt(n)).  The gradients keep both of their forward messages (R~ and
Q^) this way.  The backward pass rebuilds each segment's rows from its checkpoint, using the stored per-step
normalisers (and Q input offsets), before it consumes them.  Checked here:

* the outputs against the oracle, within the general-trellis bars;
* bit-identity with the full-tape mode of the same kernels (every (k, V) other than k = 2, V = 1, where the full tape
  runs the tuned kernels instead).  The recomputed rows repeat the first pass's arithmetic, so the two modes agree
  bit for bit.

Cases cover n not a multiple of c, n <= 3 (where checkpoints save nothing and the full tape runs), n = 4096,
sigma mode, and batches larger than the grid.
"""
import numpy as np
import pytest
import torch

import differentiable_bcjr_amd as dba
import workloads
from differentiable_bcjr_amd import abi
from test_gpu_general_trellis import _max_err, _scale, _sigma_n, _vin, vgrad_norm_ok, vgrad_tol, vsoft_tol
from test_gpu_parity import GRAD_ELEM_TOL_LONG, TOL, _t, grad_err, norm_err, rel_err

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
    for T in [1.0, 0.1, 0.05]:
        gr, ws = _grad(w, c, g, L, k, T, s, dev, checkpoint=True)
        rgr, rws = oracle_mod.grad(w, c, g, L, k, T, sigma=s)
        e = grad_err(gr.cpu().numpy(), rgr, g, c, T)
        print(f"grad checkpoint L{L} k{k} V{V} B{B} n{n} sigma={sigma} T={T}: {e:.2e} "
              f"(normwise {norm_err(gr.cpu().numpy(), rgr):.2e})", flush=True)
        assert e <= vgrad_tol(T, sigma, k, V)
        assert vgrad_norm_ok(gr.cpu().numpy(), rgr, T, sigma, k, V)
        assert rel_err(ws.cpu().numpy(), rws) <= vsoft_tol(T, sigma, k, V)
        if (k, V) != (2, 1):
            gr_t, ws_t = _grad(w, c, g, L, k, T, s, dev, checkpoint=False)
            assert torch.equal(gr, gr_t) and torch.equal(ws, ws_t)


@pytest.mark.parametrize("L,k,V,B,n", GRAD_CASES, ids=GRAD_IDS)
@pytest.mark.parametrize("sigma", [False, True])
def test_codebook_grad_checkpoint_mode_matches_oracle(oracle_mod, dev, L, k, V, B, n, sigma):
    if sigma:
        n = _sigma_n(L, k, n)
    w, c, g, s = _vin(L, V, B, n, 6500 + 31 * L + 7 * k + V + n, sigma)
    f = _scale(k, V)
    for T in [1.0, 0.1]:
        gc, gw, ws = _gc(w, c, g, L, k, T, s, dev, checkpoint=True)
        rgc, rgw, rws = oracle_mod.grad_codebook(w, c, g, L, k, T, sigma=s)
        en, em = norm_err(gc.cpu().numpy(), rgc), _max_err(gc.cpu().numpy(), rgc)
        print(f"codebook grad checkpoint L{L} k{k} V{V} B{B} n{n} sigma={sigma} T={T}: {en:.2e} normwise, "
              f"{em:.2e} of max", flush=True)
        assert en <= (5e-5 if sigma else 1e-5) * f and em <= 5e-5 * f
        assert grad_err(gw.cpu().numpy(), rgw, g, c, T) <= vgrad_tol(T, sigma, k, V)
        assert rel_err(ws.cpu().numpy(), rws) <= vsoft_tol(T, sigma, k, V)
        if (k, V) != (2, 1):
            gc_t, gw_t, ws_t = _gc(w, c, g, L, k, T, s, dev, checkpoint=False)
            assert torch.equal(gc, gc_t) and torch.equal(gw, gw_t) and torch.equal(ws, ws_t)


@pytest.mark.parametrize("L,k,V,B,n", [(8, 3, 2, 4300, 9), (16, 2, 1, 270, 5), (8, 1, 1, 4200, 10)])
def test_grad_checkpoint_mode_several_sequences_per_workgroup(oracle_mod, dev, L, k, V, B, n):
    """Each workgroup's slot, its checkpoint rows, offsets and saved messages, reused by the next sequence."""
    w, c, g, _ = _vin(L, V, B, n, 6600 + L + k)
    T = 0.1
    gr, _ = _grad(w, c, g, L, k, T, None, dev, checkpoint=True)
    rgr, _ = oracle_mod.grad(w, c, g, L, k, T)
    assert grad_err(gr.cpu().numpy(), rgr, g, c, T) <= vgrad_tol(T, False, k, V)
    gc, _, _ = _gc(w, c, g, L, k, T, None, dev, checkpoint=True)
    rgc, _, _ = oracle_mod.grad_codebook(w, c, g, L, k, T)
    assert norm_err(gc.cpu().numpy(), rgc) <= 1e-5 * _scale(k, V)


@pytest.mark.parametrize("L,k,V", [(10, 2, 1), (9, 3, 2)])
def test_grad_checkpoint_mode_longest_sequences(oracle_mod, dev, L, k, V):
    """n = 4096: 65 checkpoints of 64-step segments for each of the two forward messages."""
    n, B, T = 4096, 2, 0.3
    w, c, g, _ = _vin(L, V, B, n, 6700 + L)
    gr, ws = _grad(w, c, g, L, k, T, None, dev, checkpoint=True)
    rgr, rws = oracle_mod.grad(w, c, g, L, k, T)
    assert norm_err(gr.cpu().numpy(), rgr) <= 1e-5 * _scale(k, V)
    assert rel_err(ws.cpu().numpy(), rws) <= 1e-5 * _scale(k, V)


def test_grad_checkpoint_mode_headline_workload_rows(oracle_mod, dev):
    """The 1024x1024 workload (L = 16, k = 2, n = 256) in the checkpoint mode: 33 rows of each forward message per
    in-flight sequence instead of 257; sampled rows against the oracle at the full-length bars of the k = 2 kernels."""
    wl = workloads.WORKLOADS[2]
    c, w, g = wl.codebook(), wl.weights(), wl.upstream_grad()
    T = 0.1
    gr = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), wl.L, wl.k, T, checkpoint=True).cpu().numpy()
    assert np.all(np.isfinite(gr))
    rows = wl.sample_rows(3)
    rgr, _ = oracle_mod.grad(w[rows], c, g[rows], wl.L, wl.k, T)
    e_n, e_e = norm_err(gr[rows], rgr), grad_err(gr[rows], rgr, g[rows], c, T)
    print(f"grad checkpoint mode, {wl.name}: {e_n:.2e} normwise, {e_e:.2e} elementwise", flush=True)
    assert e_n <= TOL and e_e <= GRAD_ELEM_TOL_LONG


@pytest.mark.parametrize("L,k,V", [(9, 3, 2), (10, 2, 1)])
def test_soft_quantize_checkpoint_mode(oracle_mod, dev, L, k, V):
    """Autograd through soft_quantize with checkpoint=True: the forward, dL/dw and dL/dc with the smallest
    workspaces.  Off the tuned trellis they are bit-identical to the full-tape mode; at k = 2, V = 1 they match the
    oracle (the two modes run different kernels there)."""
    B, n, T = 5, 40, 0.2
    w, c, g, _ = _vin(L, V, B, n, 6800 + L)
    outs = {}
    for ck in (False, True):
        wt = _t(w, dev).requires_grad_(True)
        ct = _t(c, dev).requires_grad_(True)
        out = dba.soft_quantize(wt, ct, L, k, T, checkpoint=ck)
        (out * _t(g, dev)).sum().backward()
        outs[ck] = (out.detach(), wt.grad, ct.grad)
    if (k, V) != (2, 1):
        for a, b in zip(outs[False], outs[True]):
            assert torch.equal(a, b)
    rgc, rgw, rws = oracle_mod.grad_codebook(w, c, g, L, k, T)
    ws, gw, gc = (x.cpu().numpy() for x in outs[True])
    assert rel_err(ws, rws) <= 1e-5 * _scale(k, V)
    assert norm_err(gw, rgw) <= 1e-5 * _scale(k, V)
    assert norm_err(gc, rgc) <= 1e-5 * _scale(k, V)
