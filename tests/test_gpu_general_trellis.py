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

Bars: max(1e-5, kappa) for every quantity, kappa being the case's one-ulp conditioning computed by the oracle alone
(tests/parity.py); Viterbi bit-exact.  The same float32 recursion runs here as at k = 2, with its error growing with
the trellis (a state's log weight sums V squared distances, and the recursion's rounding adds up over L/k steps of
trellis memory), and the conditioning of the exact answer grows the same way: one-ulp moves of V inputs per step
reach the log weights, over the same L/k steps.
"""
import numpy as np
import pytest
import torch

import differentiable_bcjr_amd as dba
import parity
import cases
import workloads
from parity import norm_err
from test_gpu_parity import _t

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


_vin = cases.vin
_sigma_n = cases.sigma_n
CASES = cases.GENERAL
IDS = cases.ids(CASES)


@pytest.mark.parametrize("L,k,V,B,n", CASES, ids=IDS)
@pytest.mark.parametrize("sigma", [False, True])
def test_soft_codeword_matches_oracle(oracle_mod, dev, L, k, V, B, n, sigma):
    if sigma:
        n = _sigma_n(L, k, n)
    w, c, _, s = _vin(L, V, B, n, 7000 + 31 * L + 7 * k + V + n, sigma)
    ok = True
    for T in [1.0, 0.1, 0.05]:
        got, lz = dba.soft_codeword(_t(w, dev), _t(c, dev), L, k, T, _t(s, dev), return_log_z=True)
        print(f"soft L{L} k{k} V{V} B{B} n{n} sigma={sigma} T={T}:", flush=True)
        ok &= parity.soft_ok(oracle_mod, got, lz, w, c, L, k, T, s)
    assert ok


@pytest.mark.parametrize("L,k,V,B,n", CASES, ids=IDS)
@pytest.mark.parametrize("sigma", [False, True])
def test_grad_matches_oracle(oracle_mod, dev, L, k, V, B, n, sigma):
    if sigma:
        n = _sigma_n(L, k, n)
    w, c, g, s = _vin(L, V, B, n, 7100 + 31 * L + 7 * k + V + n, sigma)
    ok = True
    for T in [1.0, 0.1, 0.05]:
        gr, ws = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T, _t(s, dev), return_w_soft=True)
        print(f"grad L{L} k{k} V{V} B{B} n{n} sigma={sigma} T={T}:", flush=True)
        ok &= parity.grad_ok(oracle_mod, gr, ws, w, c, g, L, k, T, s)
    assert ok


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
    ok = True
    for V in (1, 2):
        w, c, g, _ = _vin(L, V, B, n, 7090 + V)
        for ck in (False, True):
            print(f"k = 1, L = 16, V = {V}, checkpoint={ck}:", flush=True)
            gr = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T, checkpoint=ck)
            ok &= parity.grad_ok(oracle_mod, gr, None, w, c, g, L, k, T)
            gc = dba.soft_codeword_grad_codebook(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T, return_grad_w=False,
                                                 checkpoint=ck)
            ok &= parity.codebook_grad_ok(oracle_mod, gc, None, None, w, c, g, L, k, T)
    assert ok


# ------------------------------------------------------------------------ batches larger than the persistent grid


@pytest.mark.parametrize("L,k,V,B,n", cases.GENERAL_SEVERAL)
@pytest.mark.parametrize("ck", [False, True], ids=["full-tape", "checkpoint"])
def test_several_sequences_per_workgroup(oracle_mod, dev, L, k, V, B, n, ck):
    """More sequences than the grid has workgroups (4096 at L <= 11, 256 at L = 16): every workgroup reuses its slot
    and LDS (at k = 1, L = 16 the gradient's Q^ message buffer in the slot too), and Viterbi traces one sequence back
    while it decodes the next; in both memory modes."""
    w, c, g, _ = _vin(L, V, B, n, 7300 + L + k + V)
    T = 0.1
    print(f"L{L} k{k} V{V} B{B} n{n} checkpoint={ck}:", flush=True)
    ws = dba.soft_codeword(_t(w, dev), _t(c, dev), L, k, T, checkpoint=ck)
    ok = parity.soft_ok(oracle_mod, ws, None, w, c, L, k, T)
    gr = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T, checkpoint=ck)
    ok &= parity.grad_ok(oracle_mod, gr, None, w, c, g, L, k, T)
    assert ok
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
    ok = parity.soft_ok(oracle_mod, ws, lz, w, c, L, k, T)
    gr = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T)
    ok &= parity.grad_ok(oracle_mod, gr, None, w, c, g, L, k, T)
    assert ok
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
        live = np.flatnonzero(~dead)
        assert parity.soft_ok(oracle_mod, ws, None, w, c, L, k, T, s, rows=live)
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
    # two float32 evaluations of one quantity, each within the 1e-5 bar of the scalar trellis's exact answer
    assert parity.rel_err(b[:, 0::2], a) <= 2 * parity.TOL and np.all(b[:, 1::2] == 0.0)
    ga = dba.soft_codeword_grad(_t(w1, dev), _t(c1, dev), _t(g1, dev), L, k, T).cpu().numpy()
    gb = dba.soft_codeword_grad(_t(w2, dev), _t(c2, dev), _t(g2, dev), L, k, T).cpu().numpy()
    assert norm_err(gb[:, 0::2], ga) <= 2 * parity.TOL
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
    print(f"{wl.name}, rows {rows.tolist()}:", flush=True)
    ok = parity.soft_ok(oracle_mod, ws, None, w, c, wl.L, wl.k, T, rows=rows)
    ok &= parity.grad_ok(oracle_mod, gr, None, w, c, g, wl.L, wl.k, T, rows=rows)
    assert ok
    rst, rwh, rcost = oracle_mod.viterbi(w[rows], c, wl.L, wl.k)
    np.testing.assert_array_equal(st[rows], rst)
    np.testing.assert_array_equal(wh[rows].view(np.uint32), rwh.view(np.uint32))
    np.testing.assert_array_equal(cost[rows].view(np.uint32), rcost.view(np.uint32))


# ------------------------------------------------------------------------------------ codebook gradient (row f1)
# dL/dc [2^L] or [2^L, V], summed over the batch, compared as a vector (normwise and against its largest entry) like
# the k = 2 codebook gradient, within the conditioning bars.

GC_CASES = CASES
GC_IDS = IDS


@pytest.mark.parametrize("L,k,V,B,n", GC_CASES, ids=GC_IDS)
@pytest.mark.parametrize("sigma", [False, True])
def test_codebook_grad_matches_oracle(oracle_mod, dev, L, k, V, B, n, sigma):
    if sigma:
        n = _sigma_n(L, k, n)
    w, c, g, s = _vin(L, V, B, n, 7700 + 31 * L + 7 * k + V + n, sigma)
    ok = True
    for T in [1.0, 0.1, 0.05]:
        gc, gw, ws = dba.soft_codeword_grad_codebook(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T, _t(s, dev),
                                                     return_w_soft=True)
        print(f"codebook grad L{L} k{k} V{V} B{B} n{n} sigma={sigma} T={T}:", flush=True)
        ok &= parity.codebook_grad_ok(oracle_mod, gc, gw, ws, w, c, g, L, k, T, s)
    assert ok


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
    assert parity.codebook_grad_ok(oracle_mod, ct.grad, wt.grad, None, w, c, g, L, k, T)


@pytest.mark.parametrize("name", ["k3", "k4v2"])
def test_codebook_grad_variant_workload_rows(oracle_mod, dev, name):
    """The codebook gradient of three sampled rows of the 1024x1024 variant workloads, as one batch, against the
    oracle on the same rows."""
    wl = workloads.TRELLIS_VARIANTS[name]
    c = wl.codebook()
    rows = wl.sample_rows(3)
    w, g = wl.weights()[rows], wl.upstream_grad()[rows]
    T = wl.temps[0]
    gc = dba.soft_codeword_grad_codebook(_t(w, dev), _t(c, dev), _t(g, dev), wl.L, wl.k, T, return_grad_w=False)
    print(f"{wl.name} codebook grad, rows {rows.tolist()}:", flush=True)
    assert parity.codebook_grad_ok(oracle_mod, gc, None, None, w, c, g, wl.L, wl.k, T)


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


@pytest.mark.parametrize("i,L,k,V,B,n,sigma,T", _random_cases())
def test_general_trellis_random_configuration(oracle_mod, dev, i, L, k, V, B, n, sigma, T):
    """Random shapes, some of them ill-conditioned at float32 resolution (e.g. L = 6, k = 2, V = 2, T = 0.1: one-ulp
    input moves shift the exact gradient by 4.7e-5), which the conditioning bars follow."""
    w, c, g, s = _vin(L, V, B, n, 9900 + i, sigma)
    print(f"random {i}: L{L} k{k} V{V} B{B} n{n} sigma={sigma} T={T}:", flush=True)
    ws = dba.soft_codeword(_t(w, dev), _t(c, dev), L, k, T, _t(s, dev))
    ok = parity.soft_ok(oracle_mod, ws, None, w, c, L, k, T, s)
    gr = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T, _t(s, dev))
    ok &= parity.grad_ok(oracle_mod, gr, None, w, c, g, L, k, T, s)
    assert ok
    st, wh, cost = (x.cpu().numpy() for x in dba.viterbi_hard_code(_t(w, dev), _t(c, dev), L, k, _t(s, dev)))
    rst, rwh, rcost = oracle_mod.viterbi(w, c, L, k, sigma=s)
    np.testing.assert_array_equal(st, rst)
    np.testing.assert_array_equal(cost.view(np.uint32), rcost.view(np.uint32))


@pytest.mark.parametrize("L,k,V,B,n", cases.GENERAL_GC_SEVERAL)
@pytest.mark.parametrize("ck", [False, True], ids=["full-tape", "checkpoint"])
def test_codebook_grad_several_sequences_per_slot(oracle_mod, dev, L, k, V, B, n, ck):
    """More sequences than the grid has workgroups: each slot's accumulator sums several sequences before the
    reduction over slots (at k = 1, L = 16 each slot's Q^ message buffer serves them in turn), in both memory
    modes."""
    w, c, g, _ = _vin(L, V, B, n, 8100 + L + k)
    T = 0.2
    print(f"L{L} k{k} V{V} B{B} n{n} checkpoint={ck}:", flush=True)
    gc = dba.soft_codeword_grad_codebook(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T, return_grad_w=False,
                                         checkpoint=ck)
    assert parity.codebook_grad_ok(oracle_mod, gc, None, None, w, c, g, L, k, T)


@pytest.mark.parametrize("L,k,V", cases.GENERAL_LONGEST)
def test_longest_sequences(oracle_mod, dev, L, k, V):
    """n = 4096 steps, the largest the boundary accepts (the workspace offsets of the longest tapes)."""
    n, B, T = 4096, 2, 0.3
    w, c, g, _ = _vin(L, V, B, n, 8200 + L)
    ws = dba.soft_codeword(_t(w, dev), _t(c, dev), L, k, T)
    ok = parity.soft_ok(oracle_mod, ws, None, w, c, L, k, T)
    gr = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T)
    ok &= parity.grad_ok(oracle_mod, gr, None, w, c, g, L, k, T)
    assert ok
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
