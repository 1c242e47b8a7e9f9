"""GPU parity of the tail-biting entry points (through the C-ABI) against the oracle.

viterbi_tail_biting: bit-exact states, codewords, float32 costs and chosen start states, for the exact choice (every
sigma decoded, L <= 10) and rotate-and-decode.  soft_codeword_tail_biting and soft_codeword_grad_tail_biting: the soft
codeword, ln Z and the weights' gradient under the tail-biting measure (every s_0 = s_n path, L <= 10)."""
import numpy as np
import pytest
import torch

import cases
import differentiable_bcjr_amd as dba
import workloads
from test_gpu_parity import _inputs, _t

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _same(got, ref):
    st, wh, cost, sig = (x.cpu().numpy() for x in got)
    rst, rwh, rcost, rsig = ref
    np.testing.assert_array_equal(sig, rsig)
    np.testing.assert_array_equal(st, rst)
    np.testing.assert_array_equal(wh.view(np.uint32), rwh.view(np.uint32))
    np.testing.assert_array_equal(cost.view(np.uint32), rcost.view(np.uint32))


# (L, B, n): sequences per block > 1 below L = 10, ragged batches, n = 1, n below L/k (some start states unreachable)
EXACT = [(4, 16, 6), (4, 67, 5), (5, 9, 1), (6, 5, 2), (6, 7, 33), (8, 16, 64), (8, 3, 3), (9, 5, 17), (10, 4, 40)]
ROTATE = EXACT + [(12, 3, 20), (13, 2, 11), (14, 2, 12), (15, 2, 10), (16, 2, 8), (16, 3, 31)]


@pytest.mark.parametrize("L,B,n", EXACT)
def test_tail_biting_exact_matches_oracle(oracle_mod, dev, L, B, n):
    w, c, _, _ = _inputs(L, B, n, 1200 + 13 * L + n)
    got = dba.viterbi_tail_biting(_t(w, dev), _t(c, dev), L, 2, "exact")
    _same(got, oracle_mod.viterbi_tail_biting(w, c, L, 2, oracle_mod.TB_EXACT))


@pytest.mark.parametrize("L,B,n", ROTATE)
def test_tail_biting_rotate_matches_oracle(oracle_mod, dev, L, B, n):
    w, c, _, _ = _inputs(L, B, n, 1300 + 13 * L + n)
    got = dba.viterbi_tail_biting(_t(w, dev), _t(c, dev), L, 2, "rotate")
    _same(got, oracle_mod.viterbi_tail_biting(w, c, L, 2, oracle_mod.TB_ROTATE))


def test_tail_biting_exact_ties_take_the_smallest_sigma(oracle_mod, dev):
    """An all-equal codebook makes every path cost the same: sigma 0 and the all-zero path."""
    L, B, n = 6, 3, 9
    w, _, _, _ = _inputs(L, B, n, 5)
    c = np.full(1 << L, 0.25, np.float32)
    st, _, cost, sig = (x.cpu().numpy() for x in dba.viterbi_tail_biting(_t(w, dev), _t(c, dev), L, 2, "exact"))
    assert (sig == 0).all() and (st == 0).all()
    _same(dba.viterbi_tail_biting(_t(w, dev), _t(c, dev), L, 2, "exact"),
          oracle_mod.viterbi_tail_biting(w, c, L, 2, oracle_mod.TB_EXACT))


def test_tail_biting_cycles_and_exact_is_best(dev):
    L, B, n = 8, 64, 48
    w, c, _, _ = _inputs(L, B, n, 77)
    ex = [x.cpu().numpy() for x in dba.viterbi_tail_biting(_t(w, dev), _t(c, dev), L, 2, "exact")]
    ro = [x.cpu().numpy() for x in dba.viterbi_tail_biting(_t(w, dev), _t(c, dev), L, 2, "rotate")]
    mask = (1 << (L - 2)) - 1
    for st, _, cost, sig in (ex, ro):
        assert np.array_equal(st[:, -1], sig) and np.array_equal(st[:, 0] >> 2, sig & mask)
        assert np.array_equal(st[:, 1:] >> 2, st[:, :-1] & mask)
    assert np.all(ro[2] >= ex[2])
    print(f"rotate-and-decode found the exact tail-biting optimum for {np.mean(ro[2] == ex[2]):.3f} of {B} "
          f"sequences (L = {L}, n = {n})", flush=True)


def test_tail_biting_rotate_low_temperature_workload_rows(oracle_mod, dev):
    """The 2048x2048 workload (16384 sequences of 256 weights, L = 16): the whole batch decoded, sampled rows checked."""
    wl = workloads.WORKLOADS[4]
    c, w = wl.codebook(), wl.weights()
    got = [x.cpu().numpy() for x in dba.viterbi_tail_biting(_t(w, dev), _t(c, dev), wl.L, wl.k, "rotate")]
    rows = wl.sample_rows(3)
    ref = oracle_mod.viterbi_tail_biting(w[rows], c, wl.L, wl.k, oracle_mod.TB_ROTATE)
    _same([torch.from_numpy(g[rows]) for g in got], ref)


def _random_cases(count=24, seed=5150):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for i in range(count):
        mode = "exact" if rng.integers(0, 2) else "rotate"
        L = int(rng.integers(4, 11)) if mode == "exact" else int(rng.integers(4, 17))
        n = int(rng.integers(1, 65)) if L <= 12 else int(rng.integers(1, 33))
        B = int(rng.integers(1, 41)) if L <= 12 else int(rng.integers(1, 5))
        cases.append((i, mode, L, B, n))
    return cases


@pytest.mark.parametrize("i,mode,L,B,n", _random_cases())
def test_tail_biting_random_configuration(oracle_mod, dev, i, mode, L, B, n):
    w, c, _, _ = _inputs(L, B, n, 8000 + i)
    got = dba.viterbi_tail_biting(_t(w, dev), _t(c, dev), L, 2, mode)
    _same(got, oracle_mod.viterbi_tail_biting(w, c, L, 2, oracle_mod.TB_EXACT if mode == "exact" else
                                              oracle_mod.TB_ROTATE))


# ---------------------------------------------------------------- soft codeword and gradient under the measure
# Bars: max(1e-5, kappa) per quantity, kappa its one-ulp conditioning under the measure (tests/parity.py).

MEASURE = cases.TAIL_BITING_MEASURE


@pytest.mark.parametrize("L,B,n", MEASURE)
def test_soft_tail_biting_matches_oracle(oracle_mod, dev, L, B, n):
    import parity

    w, c, g, _ = _inputs(L, B, n, 1400 + 7 * L + n)
    ok = True
    for T in [1.0, 0.1, 0.05]:
        ws, lz = dba.soft_codeword_tail_biting(_t(w, dev), _t(c, dev), L, 2, T, return_log_z=True)
        gr, ws2 = dba.soft_codeword_grad_tail_biting(_t(w, dev), _t(c, dev), _t(g, dev), L, 2, T, return_w_soft=True)
        print(f"tail-biting measure L{L} B{B} n{n} T{T}:", flush=True)
        ok &= parity.tail_biting_ok(oracle_mod, ws, lz, gr, ws2, w, c, g, L, 2, T)
    assert ok


def test_soft_tail_biting_is_the_sigma_mixture(dev):
    """ln Z under the measure is the log-sum over sigma of the sigma-mode ln Z (GPU path against itself)."""
    L, B, n, T = 6, 4, 20, 0.3
    w, c, _, _ = _inputs(L, B, n, 99)
    _, lz = dba.soft_codeword_tail_biting(_t(w, dev), _t(c, dev), L, 2, T, return_log_z=True)
    S = 1 << L
    sig = torch.arange(S, dtype=torch.int32, device=dev).repeat(B)
    _, lz_s = dba.soft_codeword(_t(np.repeat(w, S, axis=0), dev), _t(c, dev), L, 2, T, sig, return_log_z=True)
    ref = torch.logsumexp(lz_s.double().view(B, S), dim=1)
    assert float((lz.double() - ref).abs().max()) <= 1e-5 * float(ref.abs().max())
