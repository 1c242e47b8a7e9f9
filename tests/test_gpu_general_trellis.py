"""GPU parity of the general trellis kernels against the oracle, through the C-ABI.

The kernels cover k = 1..4 bits shifted in per step and V = 1 or 2 weights per step; k = 2 with V = 1 runs the tuned
kernels and is covered elsewhere.  Checked:

* the soft codeword and ln Z;
* the weights' gradient;
* the Viterbi hard code: states, codewords and float32 costs, bit-exact.

Cases span:

* L = 4..16, which covers both kernel forms: L = 16 (compile-time strides) and the run-time-L form, including
  sub-wave workgroups;
* ragged batches, n = 1, free and sigma boundaries;
* batches larger than the persistent grid, so that a workgroup decodes several sequences in turn.  This exercises the
  Viterbi traceback pipelined across sequences.

Bars.  They are the k = 2, V = 1 bars multiplied by V max(1, 2/k).  The same float32 recursion runs here, and its
error comes from the two sources the k = 2 derivation names, both of which grow with the trellis:

* The rounding of a state's log weight theta' = -|c - w|^2 log2(e) / T is proportional to its size.  With V components
  that log weight is a sum of V squared distances, V times larger on average.
* The recursion's per-step rounding adds up over the L/k steps of trellis memory, which is twice as long at k = 1 as at
  k = 2.

At k = 3 and 4 with V = 1 the bars are the k = 2 ones.  Measured maxima over these cases (with other seeds):

* soft codeword at T = 0.05: 1.6e-5 at L = 9, k = 1, V = 2 (free) and 1.5e-5 at L = 5, k = 1, V = 1 (sigma);
* gradient at T = 0.1: 1.6e-5 elementwise at L = 5, k = 2, V = 2 (free, 2.5e-6 normwise);
* every k >= 2, V = 1 case at T >= 0.1: within 1e-5.
"""
import numpy as np
import pytest
import torch

import differentiable_bcjr_amd as dba
import workloads
from test_gpu_parity import _t, grad_err, grad_tol, norm_err, rel_err, soft_tol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _vin(L, V, B, n, seed, sigma=False):
    """Codebook ([2^L] for V = 1, else [2^L, V], unit variance), weights and upstream gradient [B, n V], sigma [B]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    c = rng.standard_normal((1 << L, V))
    c = (c / c.std()).astype(np.float32)
    if V == 1:
        c = c[:, 0].copy()
    w = rng.standard_normal((B, n * V)).astype(np.float32)
    g = rng.standard_normal((B, n * V)).astype(np.float32)
    s = rng.integers(0, 1 << L, size=B).astype(np.int32) if sigma else None
    return w, c, g, s


# (L, k, V, B, n steps)
CASES = [(4, 1, 1, 16, 6), (4, 1, 2, 7, 5), (5, 1, 1, 5, 8), (5, 2, 2, 9, 9), (6, 3, 1, 5, 4), (6, 3, 2, 3, 7),
         (7, 3, 1, 4, 9), (8, 1, 1, 6, 33), (8, 4, 1, 4, 5), (8, 4, 2, 3, 6), (9, 1, 2, 5, 17), (9, 3, 2, 4, 12),
         (10, 4, 1, 3, 10), (11, 1, 1, 2, 20), (12, 3, 1, 2, 16), (12, 4, 2, 2, 9), (13, 1, 2, 2, 7), (14, 3, 2, 2, 6),
         (15, 1, 1, 2, 6), (16, 1, 1, 2, 4), (16, 1, 2, 1, 4), (16, 2, 2, 2, 5), (16, 3, 1, 2, 5), (16, 3, 2, 2, 4),
         (16, 4, 1, 2, 4), (16, 4, 2, 2, 5)]
IDS = [f"L{L}k{k}V{V}B{B}n{n}" for L, k, V, B, n in CASES]


def _scale(k, V):
    """How much the float32 error grows over the k = 2, V = 1 trellis: a state's log weight is a sum of V squared
    distances, and the recursion's rounding adds up over L/k steps of trellis memory."""
    return V * (2 if k == 1 else 1)


def vsoft_tol(T, sigma, k, V):
    return soft_tol(T, sigma) * _scale(k, V)


def vgrad_tol(T, sigma, k, V):
    return grad_tol(T, sigma) * _scale(k, V)


def vgrad_norm_ok(x, ref, T, sigma, k, V):
    return sigma or T >= 0.1 or norm_err(x, ref) <= 1e-5 * _scale(k, V)


def _sigma_n(L, k, n):
    """Enough steps for every sigma to be reachable: the constraint needs at least L/k steps."""
    return max(n, -(-L // k) + 1)


@pytest.mark.parametrize("L,k,V,B,n", CASES, ids=IDS)
@pytest.mark.parametrize("sigma", [False, True])
def test_soft_codeword_matches_oracle(oracle_mod, dev, L, k, V, B, n, sigma):
    if sigma:
        n = _sigma_n(L, k, n)
    w, c, _, s = _vin(L, V, B, n, 7000 + 31 * L + 7 * k + V + n, sigma)
    for T in [1.0, 0.1, 0.05]:
        got, lz = dba.soft_codeword(_t(w, dev), _t(c, dev), L, k, T, _t(s, dev), return_log_z=True)
        ref, rlz = oracle_mod.soft(w, c, L, k, T, sigma=s)
        e = rel_err(got.cpu().numpy(), ref)
        el = float(np.max(np.abs(lz.cpu().numpy() - rlz) / np.maximum(np.abs(rlz), 1.0)))
        print(f"soft L{L} k{k} V{V} B{B} n{n} sigma={sigma} T={T}: {e:.2e}, ln Z {el:.2e}", flush=True)
        assert e <= vsoft_tol(T, sigma, k, V)
        assert el <= 1e-5


@pytest.mark.parametrize("L,k,V,B,n", CASES, ids=IDS)
@pytest.mark.parametrize("sigma", [False, True])
def test_grad_matches_oracle(oracle_mod, dev, L, k, V, B, n, sigma):
    if sigma:
        n = _sigma_n(L, k, n)
    w, c, g, s = _vin(L, V, B, n, 7100 + 31 * L + 7 * k + V + n, sigma)
    for T in [1.0, 0.1, 0.05]:
        gr, ws = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T, _t(s, dev), return_w_soft=True)
        rgr, rws = oracle_mod.grad(w, c, g, L, k, T, sigma=s)
        e = grad_err(gr.cpu().numpy(), rgr, g, c, T)
        print(f"grad L{L} k{k} V{V} B{B} n{n} sigma={sigma} T={T}: {e:.2e} "
              f"(normwise {norm_err(gr.cpu().numpy(), rgr):.2e})", flush=True)
        assert e <= vgrad_tol(T, sigma, k, V)
        assert vgrad_norm_ok(gr.cpu().numpy(), rgr, T, sigma, k, V)
        assert rel_err(ws.cpu().numpy(), rws) <= vsoft_tol(T, sigma, k, V)


@pytest.mark.parametrize("L,k,V,B,n", CASES, ids=IDS)
@pytest.mark.parametrize("sigma", [False, True])
def test_viterbi_matches_oracle_bit_exact(oracle_mod, dev, L, k, V, B, n, sigma):
    if sigma:
        n = _sigma_n(L, k, n)
    w, c, _, s = _vin(L, V, B, n, 7200 + 31 * L + 7 * k + V + n, sigma)
    st, wh, cost = (x.cpu().numpy() for x in dba.viterbi_hard_code(_t(w, dev), _t(c, dev), L, k, _t(s, dev)))
    rst, rwh, rcost = oracle_mod.viterbi(w, c, L, k, sigma=s)
    np.testing.assert_array_equal(st, rst)
    np.testing.assert_array_equal(wh.view(np.uint32), rwh.view(np.uint32))
    np.testing.assert_array_equal(cost.view(np.uint32), rcost.view(np.uint32))


def test_gradient_k1_at_L16_keeps_q_in_the_workspace(oracle_mod, dev):
    """k = 1 at L = 16: the two 128 KiB messages exceed LDS, so the gradients keep Q^ in a workspace buffer.  Both
    gradients, with and without checkpoints, against the oracle."""
    L, k, B, n, T = 16, 1, 2, 7, 0.3
    for V in (1, 2):
        w, c, g, _ = _vin(L, V, B, n, 7090 + V)
        rgc, rgw, _ = oracle_mod.grad_codebook(w, c, g, L, k, T)
        for ck in (False, True):
            gr = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T, checkpoint=ck).cpu().numpy()
            assert grad_err(gr, rgw, g, c, T) <= vgrad_tol(T, False, k, V)
            gc = dba.soft_codeword_grad_codebook(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T, return_grad_w=False,
                                                 checkpoint=ck).cpu().numpy()
            assert norm_err(gc, rgc) <= 1e-5 * _scale(k, V)


# ------------------------------------------------------------------------ batches larger than the persistent grid


@pytest.mark.parametrize("L,k,V,B,n", [(8, 1, 2, 4600, 5), (9, 3, 1, 4200, 4), (16, 3, 1, 260, 3),
                                       (16, 4, 2, 258, 3)])
def test_several_sequences_per_workgroup(oracle_mod, dev, L, k, V, B, n):
    """More sequences than the grid has workgroups (4096 at L <= 11, 256 at L = 16): every workgroup reuses its slot
    and LDS, and Viterbi traces one sequence back while it decodes the next."""
    w, c, g, _ = _vin(L, V, B, n, 7300 + L + k + V)
    T = 0.1
    ws = dba.soft_codeword(_t(w, dev), _t(c, dev), L, k, T).cpu().numpy()
    rws, _ = oracle_mod.soft(w, c, L, k, T)
    assert rel_err(ws, rws) <= vsoft_tol(T, False, k, V)
    gr = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T).cpu().numpy()
    rgr, _ = oracle_mod.grad(w, c, g, L, k, T)
    assert grad_err(gr, rgr, g, c, T) <= vgrad_tol(T, False, k, V)
    st, wh, cost = (x.cpu().numpy() for x in dba.viterbi_hard_code(_t(w, dev), _t(c, dev), L, k))
    rst, rwh, rcost = oracle_mod.viterbi(w, c, L, k)
    np.testing.assert_array_equal(st, rst)
    np.testing.assert_array_equal(wh.view(np.uint32), rwh.view(np.uint32))
    np.testing.assert_array_equal(cost.view(np.uint32), rcost.view(np.uint32))


# ------------------------------------------------------------------------------------------------- edge cases


@pytest.mark.parametrize("L,k,V", [(8, 1, 1), (9, 3, 2), (16, 4, 2)])
def test_one_step(oracle_mod, dev, L, k, V):
    w, c, g, _ = _vin(L, V, 3, 1, 7400 + L)
    T = 0.3
    ws, lz = dba.soft_codeword(_t(w, dev), _t(c, dev), L, k, T, return_log_z=True)
    rws, rlz = oracle_mod.soft(w, c, L, k, T)
    assert rel_err(ws.cpu().numpy(), rws) <= 1e-5
    assert np.max(np.abs(lz.cpu().numpy() - rlz) / np.maximum(np.abs(rlz), 1.0)) <= 1e-5
    gr = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T).cpu().numpy()
    rgr, _ = oracle_mod.grad(w, c, g, L, k, T)
    assert grad_err(gr, rgr, g, c, T) <= 1e-5
    st, _, cost = (x.cpu().numpy() for x in dba.viterbi_hard_code(_t(w, dev), _t(c, dev), L, k))
    rst, _, rcost = oracle_mod.viterbi(w, c, L, k)
    np.testing.assert_array_equal(st, rst)
    np.testing.assert_array_equal(cost.view(np.uint32), rcost.view(np.uint32))


@pytest.mark.parametrize("L,k,V", [(8, 1, 2), (12, 3, 1), (16, 4, 2)])
def test_sigma_without_a_path(oracle_mod, dev, L, k, V):
    """n < L/k: most sigmas have no admissible path; their outputs are NaN, ln Z = -inf and the Viterbi cost +inf,
    as in the oracle, while sigmas that do have one match it."""
    n = max(1, L // k - 2)
    B = 6
    w, c, g, s = _vin(L, V, B, n, 7500 + L, sigma=True)
    T = 0.5
    ws, lz = dba.soft_codeword(_t(w, dev), _t(c, dev), L, k, T, _t(s, dev), return_log_z=True)
    rws, rlz = oracle_mod.soft(w, c, L, k, T, sigma=s)
    ws, lz = ws.cpu().numpy(), lz.cpu().numpy()
    dead = ~np.isfinite(rlz)
    assert dead.any()
    assert np.all(np.isnan(ws[dead])) and np.all(lz[dead] == -np.inf)
    if (~dead).any():
        assert rel_err(ws[~dead], rws[~dead]) <= 3e-5
    gr = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T, _t(s, dev)).cpu().numpy()
    assert np.all(np.isnan(gr[dead]))
    _, _, cost = dba.viterbi_hard_code(_t(w, dev), _t(c, dev), L, k, _t(s, dev))
    assert np.all(cost.cpu().numpy()[dead] == np.inf)


def test_silent_second_component_matches_the_scalar_trellis(dev):
    """V = 2 with the second codebook column and every second weight at 0 runs the general kernels on the scalar
    trellis: the first components agree with the k = 2 tuned kernels within the parity bar, the second is 0, and
    Viterbi is bit-identical (adding 0 * 0 changes no float32 sum)."""
    L, k, B, n, T = 12, 2, 5, 24, 0.2
    w1, c1, g1, _ = _vin(L, 1, B, n, 7600)
    c2 = np.stack([c1, np.zeros_like(c1)], axis=1)
    w2 = np.stack([w1, np.zeros_like(w1)], axis=2).reshape(B, 2 * n)
    g2 = np.stack([g1, np.zeros_like(g1)], axis=2).reshape(B, 2 * n)
    a = dba.soft_codeword(_t(w1, dev), _t(c1, dev), L, k, T).cpu().numpy()
    b = dba.soft_codeword(_t(w2, dev), _t(c2, dev), L, k, T).cpu().numpy()
    assert rel_err(b[:, 0::2], a) <= 2e-5 and np.all(b[:, 1::2] == 0.0)
    ga = dba.soft_codeword_grad(_t(w1, dev), _t(c1, dev), _t(g1, dev), L, k, T).cpu().numpy()
    gb = dba.soft_codeword_grad(_t(w2, dev), _t(c2, dev), _t(g2, dev), L, k, T).cpu().numpy()
    assert norm_err(gb[:, 0::2], ga) <= 2e-5
    assert np.max(np.abs(gb[:, 1::2])) == 0.0
    sa = [x.cpu().numpy() for x in dba.viterbi_hard_code(_t(w1, dev), _t(c1, dev), L, k)]
    sb = [x.cpu().numpy() for x in dba.viterbi_hard_code(_t(w2, dev), _t(c2, dev), L, k)]
    np.testing.assert_array_equal(sa[0], sb[0])
    np.testing.assert_array_equal(sa[2].view(np.uint32), sb[2].view(np.uint32))


# ------------------------------------------------------------------- the 1024x1024 workload at other bit rates


@pytest.mark.parametrize("name", ["k3", "k4v2"])
def test_trellis_variant_workload_rows(oracle_mod, dev, name):
    """The whole 4096-sequence batch through all three operations; sampled rows against the oracle."""
    wl = workloads.TRELLIS_VARIANTS[name]
    c, w, g = wl.codebook(), wl.weights(), wl.upstream_grad()
    T = wl.temps[0]
    ct, wt, gt = _t(c, dev), _t(w, dev), _t(g, dev)
    ws = dba.soft_codeword(wt, ct, wl.L, wl.k, T).cpu().numpy()
    gr = dba.soft_codeword_grad(wt, ct, gt, wl.L, wl.k, T).cpu().numpy()
    st, wh, cost = (x.cpu().numpy() for x in dba.viterbi_hard_code(wt, ct, wl.L, wl.k))
    assert np.all(np.isfinite(ws)) and np.all(np.isfinite(gr))
    rows = wl.sample_rows(3)
    rws, _ = oracle_mod.soft(w[rows], c, wl.L, wl.k, T)
    rgr, _ = oracle_mod.grad(w[rows], c, g[rows], wl.L, wl.k, T)
    rst, rwh, rcost = oracle_mod.viterbi(w[rows], c, wl.L, wl.k)
    e_s, e_g = rel_err(ws[rows], rws), norm_err(gr[rows], rgr)
    e_ge = grad_err(gr[rows], rgr, g[rows], c, T)
    print(f"{wl.name}: soft {e_s:.2e}, grad {e_g:.2e} normwise, {e_ge:.2e} elementwise", flush=True)
    f = _scale(wl.k, wl.V)
    assert e_s <= 1e-5 * f
    assert e_g <= 1e-5 * f and e_ge <= 5e-5 * f   # the full-length bars of the k = 2 kernels, scaled as above
    np.testing.assert_array_equal(st[rows], rst)
    np.testing.assert_array_equal(wh[rows].view(np.uint32), rwh.view(np.uint32))
    np.testing.assert_array_equal(cost[rows].view(np.uint32), rcost.view(np.uint32))


# ------------------------------------------------------------------------------------ codebook gradient (row f1)
# dL/dc [2^L] or [2^L, V], summed over the batch, compared as a vector like the k = 2 codebook gradient: normwise
# 1e-5 free and 5e-5 sigma, 5e-5 of the largest entry elementwise, scaled as the other bars here.

GC_CASES = CASES
GC_IDS = IDS


def _max_err(x, ref):
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


@pytest.mark.parametrize("L,k,V,B,n", GC_CASES, ids=GC_IDS)
@pytest.mark.parametrize("sigma", [False, True])
def test_codebook_grad_matches_oracle(oracle_mod, dev, L, k, V, B, n, sigma):
    if sigma:
        n = _sigma_n(L, k, n)
    w, c, g, s = _vin(L, V, B, n, 7700 + 31 * L + 7 * k + V + n, sigma)
    f = _scale(k, V)
    for T in [1.0, 0.1, 0.05]:
        gc, gw, ws = dba.soft_codeword_grad_codebook(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T, _t(s, dev),
                                                     return_w_soft=True)
        rgc, rgw, rws = oracle_mod.grad_codebook(w, c, g, L, k, T, sigma=s)
        assert gc.shape == c.shape
        en, em = norm_err(gc.cpu().numpy(), rgc), _max_err(gc.cpu().numpy(), rgc)
        eg = grad_err(gw.cpu().numpy(), rgw, g, c, T)
        print(f"codebook grad L{L} k{k} V{V} B{B} n{n} sigma={sigma} T={T}: {en:.2e} normwise, {em:.2e} of max; "
              f"weights' grad {eg:.2e}", flush=True)
        assert en <= (5e-5 if sigma else 1e-5) * f and em <= 5e-5 * f
        assert eg <= vgrad_tol(T, sigma, k, V) and vgrad_norm_ok(gw.cpu().numpy(), rgw, T, sigma, k, V)
        assert rel_err(ws.cpu().numpy(), rws) <= vsoft_tol(T, sigma, k, V)


@pytest.mark.parametrize("L,k,V", [(9, 3, 2), (12, 1, 1), (16, 4, 2)])
def test_codebook_grad_translation_identity(dev, L, k, V):
    """Shifting component v of every codebook entry and of every weight by the same amount leaves every energy
    unchanged and shifts that component of the soft codeword by it, so per component
    sum_s dL/dc(s, v) + sum_u dL/dw(u, v) = sum_t g(t, v).  The codebook-only call (no dL/dw requested) agrees with
    the full one bit for bit."""
    B, n, T = 40, 24, 0.1
    w, c, g, _ = _vin(L, V, B, n, 7800 + L)
    wt, ct, gt = _t(w, dev), _t(c, dev), _t(g, dev)
    gc, gw = dba.soft_codeword_grad_codebook(wt, ct, gt, L, k, T)
    only = dba.soft_codeword_grad_codebook(wt, ct, gt, L, k, T, return_grad_w=False)
    assert torch.equal(only, gc)
    gc2 = gc.double().cpu().numpy().reshape(1 << L, V)
    gw2 = gw.double().cpu().numpy().reshape(B, n, V)
    g2 = g.astype(np.float64).reshape(B, n, V)
    lhs = gc2.sum(axis=0) + gw2.sum(axis=(0, 1))
    rhs = g2.sum(axis=(0, 1))
    scale_ = np.abs(gc2).sum(axis=0) + np.abs(gw2).sum(axis=(0, 1)) + np.abs(g2).sum(axis=(0, 1))
    assert np.all(np.abs(lhs - rhs) <= 1e-6 * scale_)


@pytest.mark.parametrize("L,k,V", [(8, 1, 2), (12, 3, 1)])
def test_codebook_grad_nan_when_no_path(dev, L, k, V):
    n = max(1, L // k - 2)
    w, c, g, s = _vin(L, V, 5, n, 7900 + L, sigma=True)
    gc = dba.soft_codeword_grad_codebook(_t(w, dev), _t(c, dev), _t(g, dev), L, k, 0.5, _t(s, dev),
                                         return_grad_w=False)
    assert torch.isnan(gc).all()


def test_soft_quantize_trains_the_codebook_at_other_bit_rates(oracle_mod, dev):
    """Autograd through soft_quantize with a trainable [2^L, 2] codebook at k = 3: both gradients match the oracle."""
    L, k, V, B, n, T = 9, 3, 2, 6, 14, 0.2
    w, c, g, _ = _vin(L, V, B, n, 8000)
    wt = _t(w, dev).requires_grad_(True)
    ct = _t(c, dev).requires_grad_(True)
    (dba.soft_quantize(wt, ct, L, k, T) * _t(g, dev)).sum().backward()
    rgc, rgw, _ = oracle_mod.grad_codebook(w, c, g, L, k, T)
    assert norm_err(ct.grad.cpu().numpy(), rgc) <= 1e-5 * _scale(k, V)
    assert norm_err(wt.grad.cpu().numpy(), rgw) <= 1e-5 * _scale(k, V)


@pytest.mark.parametrize("name", ["k3", "k4v2"])
def test_codebook_grad_variant_workload_rows(oracle_mod, dev, name):
    """The codebook gradient of three sampled rows of the 1024x1024 variant workloads, as one batch, against the
    oracle on the same rows."""
    wl = workloads.TRELLIS_VARIANTS[name]
    c = wl.codebook()
    rows = wl.sample_rows(3)
    w, g = wl.weights()[rows], wl.upstream_grad()[rows]
    T = wl.temps[0]
    gc = dba.soft_codeword_grad_codebook(_t(w, dev), _t(c, dev), _t(g, dev), wl.L, wl.k, T,
                                         return_grad_w=False).cpu().numpy()
    rgc, _, _ = oracle_mod.grad_codebook(w, c, g, wl.L, wl.k, T)
    en = norm_err(gc, rgc)
    print(f"{wl.name} codebook grad, 3 rows: {en:.2e} normwise, {_max_err(gc, rgc):.2e} of max", flush=True)
    assert en <= 1e-5 * _scale(wl.k, wl.V)


# ------------------------------------------------------------------------------------ seeded random configurations


def _random_cases(count=30, seed=4242):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for i in range(count):
        k = int(rng.integers(1, 5))
        V = int(rng.integers(1, 3))
        if (k, V) == (2, 1):
            V = 2
        L = int(rng.integers(max(4, 2 * k), 17))
        sigma = bool(rng.integers(0, 2))
        n = int(rng.integers(1, 40)) if L <= 12 else int(rng.integers(1, 8))
        if sigma:
            n = _sigma_n(L, k, n)
        B = int(rng.integers(1, 30)) if L <= 12 else int(rng.integers(1, 4))
        T = float(rng.choice([1.0, 0.3, 0.1]))
        cases.append((i, L, k, V, B, n, sigma, T))
    return cases


def _ulp(a, rng):
    """a moved by one float32 ulp, up or down at random, element by element."""
    d = np.where(rng.integers(0, 2, a.shape) == 1, np.float32(np.inf), np.float32(-np.inf)).astype(np.float32)
    return np.nextafter(a, d)


def grad_ulp_sensitivity(oracle_mod, w, c, g, L, k, T, s, trials=4, seed=0):
    """The exact gradient, and how far it moves (grad_err) when w and c move by one float32 ulp: the conditioning of
    the problem at float32 resolution.  Rounding the inputs alone moves the answer that far, so no float32 evaluation
    can be held closer.  Computed by the oracle alone."""
    ref, _ = oracle_mod.grad(w, c, g, L, k, T, sigma=s)
    rng = np.random.Generator(np.random.PCG64(seed))
    worst = 0.0
    for _ in range(trials):
        moved, _ = oracle_mod.grad(_ulp(w, rng), _ulp(c, rng), g, L, k, T, sigma=s)
        worst = max(worst, grad_err(moved, ref, g, c, T))
    return ref, worst


@pytest.mark.parametrize("i,L,k,V,B,n,sigma,T", _random_cases())
def test_general_trellis_random_configuration(oracle_mod, dev, i, L, k, V, B, n, sigma, T):
    """Random shapes: the gradient bar is the larger of the derived one and the one-ulp sensitivity above, since some
    draws are ill-conditioned at float32 resolution (e.g. L = 6, k = 2, V = 2, T = 0.1: one-ulp input moves shift the
    exact gradient by 4.7e-5)."""
    w, c, g, s = _vin(L, V, B, n, 9900 + i, sigma)
    ws = dba.soft_codeword(_t(w, dev), _t(c, dev), L, k, T, _t(s, dev)).cpu().numpy()
    rws, _ = oracle_mod.soft(w, c, L, k, T, sigma=s)
    assert rel_err(ws, rws) <= vsoft_tol(T, sigma, k, V)
    gr = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T, _t(s, dev)).cpu().numpy()
    rgr, sens = grad_ulp_sensitivity(oracle_mod, w, c, g, L, k, T, s)
    e = grad_err(gr, rgr, g, c, T)
    print(f"random {i}: L{L} k{k} V{V} B{B} n{n} sigma={sigma} T={T}: grad {e:.2e} "
          f"(one-ulp sensitivity {sens:.2e})", flush=True)
    assert e <= max(vgrad_tol(T, sigma, k, V), sens)
    st, wh, cost = (x.cpu().numpy() for x in dba.viterbi_hard_code(_t(w, dev), _t(c, dev), L, k, _t(s, dev)))
    rst, rwh, rcost = oracle_mod.viterbi(w, c, L, k, sigma=s)
    np.testing.assert_array_equal(st, rst)
    np.testing.assert_array_equal(cost.view(np.uint32), rcost.view(np.uint32))


@pytest.mark.parametrize("L,k,V,B,n", [(9, 3, 2, 4200, 3), (8, 1, 1, 4400, 4), (16, 4, 2, 300, 2)])
def test_codebook_grad_several_sequences_per_slot(oracle_mod, dev, L, k, V, B, n):
    """More sequences than the grid has workgroups: each slot's accumulator sums several sequences before the
    reduction over slots."""
    w, c, g, _ = _vin(L, V, B, n, 8100 + L + k)
    T = 0.2
    gc = dba.soft_codeword_grad_codebook(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T, return_grad_w=False)
    rgc, _, _ = oracle_mod.grad_codebook(w, c, g, L, k, T)
    assert norm_err(gc.cpu().numpy(), rgc) <= 1e-5 * _scale(k, V)


@pytest.mark.parametrize("L,k,V", [(10, 3, 2), (8, 1, 1), (12, 4, 1)])
def test_longest_sequences(oracle_mod, dev, L, k, V):
    """n = 4096 steps, the largest the boundary accepts (the workspace offsets of the longest tapes)."""
    n, B, T = 4096, 2, 0.3
    w, c, g, _ = _vin(L, V, B, n, 8200 + L)
    ws = dba.soft_codeword(_t(w, dev), _t(c, dev), L, k, T).cpu().numpy()
    rws, _ = oracle_mod.soft(w, c, L, k, T)
    assert rel_err(ws, rws) <= 1e-5 * _scale(k, V)
    gr = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T).cpu().numpy()
    rgr, _ = oracle_mod.grad(w, c, g, L, k, T)
    assert norm_err(gr, rgr) <= 1e-5 * _scale(k, V)
    st, _, cost = (x.cpu().numpy() for x in dba.viterbi_hard_code(_t(w, dev), _t(c, dev), L, k))
    rst, _, rcost = oracle_mod.viterbi(w, c, L, k)
    np.testing.assert_array_equal(st, rst)
    np.testing.assert_array_equal(cost.view(np.uint32), rcost.view(np.uint32))


@pytest.mark.parametrize("L,k,V,B,n,sigma", [(12, 3, 2, 8301, 3, False), (12, 4, 2, 8195, 2, True),
                                             (13, 2, 2, 1027, 5, False), (12, 1, 2, 9, 1, False)])
def test_viterbi_paired_sequences(oracle_mod, dev, L, k, V, B, n, sigma):
    """V = 2 at L >= 12 decodes two sequences per workgroup (they share each codebook row read): odd batches (a
    missing second sequence), more pairs than the grid holds (several rounds per workgroup and both back-pointer
    parities), sigma mode, n = 1.  Bit-exact against the oracle."""
    if sigma:
        n = _sigma_n(L, k, n)
    w, c, _, s = _vin(L, V, B, n, 8400 + L + k + n, sigma)
    st, wh, cost = (x.cpu().numpy() for x in dba.viterbi_hard_code(_t(w, dev), _t(c, dev), L, k, _t(s, dev)))
    rst, rwh, rcost = oracle_mod.viterbi(w, c, L, k, sigma=s)
    np.testing.assert_array_equal(st, rst)
    np.testing.assert_array_equal(wh.view(np.uint32), rwh.view(np.uint32))
    np.testing.assert_array_equal(cost.view(np.uint32), rcost.view(np.uint32))
