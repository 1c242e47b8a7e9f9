"""GPU parity of the tail-biting entry points on the general trellis (k = 1, 3, 4, and V = 2 weights per step at any
k, including k = 2), through the C-ABI, against the oracle.

viterbi_tail_biting: bit-exact states, codewords, float32 costs and chosen start states, for the exact choice (every
sigma decoded, L <= 10) and for rotate-and-decode (the rows rotated by n/2 trellis steps, any L).  The soft codeword,
ln Z and the weights' gradient under the tail-biting measure (L <= 10) are held to max(1e-5, kappa), kappa their
one-ulp conditioning under the measure (tests/parity.py)."""
import numpy as np
import pytest
import torch

import cases
import differentiable_bcjr_amd as dba
import parity
from cases import vin as _vin
from test_gpu_parity import _t

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


def _ids(cases):
    return [f"L{c[0]}k{c[1]}V{c[2]}B{c[3]}n{c[4]}" for c in cases]


# (L, k, V, B, n steps): n = 1, n below L/k (some start states unreachable), batches beyond the persistent grid
EXACT = [(4, 1, 1, 9, 6), (4, 1, 2, 5, 5), (6, 3, 1, 7, 4), (6, 3, 2, 3, 1), (8, 4, 1, 4, 2), (8, 4, 2, 3, 9),
         (8, 2, 2, 5, 12), (9, 1, 1, 3, 17), (10, 3, 2, 3, 20), (10, 4, 1, 5, 33)]
ROTATE = EXACT + [(12, 1, 2, 3, 14), (13, 4, 2, 2, 11), (16, 3, 1, 2, 12), (16, 4, 2, 3, 10), (16, 2, 2, 2, 7),
                  (15, 1, 1, 2, 9)]


@pytest.mark.parametrize("L,k,V,B,n", EXACT, ids=_ids(EXACT))
def test_general_tail_biting_exact_matches_oracle(oracle_mod, dev, L, k, V, B, n):
    w, c, _, _ = _vin(L, V, B, n, 2100 + 31 * L + 7 * k + V + n)
    print(f"exact tail-biting L{L} k{k} V{V} B{B} n{n}", flush=True)
    got = dba.viterbi_tail_biting(_t(w, dev), _t(c, dev), L, k, "exact")
    _same(got, oracle_mod.viterbi_tail_biting(w, c, L, k, oracle_mod.TB_EXACT))


@pytest.mark.parametrize("L,k,V,B,n", ROTATE, ids=_ids(ROTATE))
def test_general_tail_biting_rotate_matches_oracle(oracle_mod, dev, L, k, V, B, n):
    w, c, _, _ = _vin(L, V, B, n, 2200 + 31 * L + 7 * k + V + n)
    print(f"rotate tail-biting L{L} k{k} V{V} B{B} n{n}", flush=True)
    got = dba.viterbi_tail_biting(_t(w, dev), _t(c, dev), L, k, "rotate")
    _same(got, oracle_mod.viterbi_tail_biting(w, c, L, k, oracle_mod.TB_ROTATE))


@pytest.mark.parametrize("L,k,V", [(8, 1, 2), (9, 3, 1), (8, 4, 2)])
def test_general_tail_biting_cycles_and_exact_is_best(dev, L, k, V):
    B, n = 40, 30
    w, c, _, _ = _vin(L, V, B, n, 2300 + L + k)
    ex = [x.cpu().numpy() for x in dba.viterbi_tail_biting(_t(w, dev), _t(c, dev), L, k, "exact")]
    ro = [x.cpu().numpy() for x in dba.viterbi_tail_biting(_t(w, dev), _t(c, dev), L, k, "rotate")]
    mask = (1 << (L - k)) - 1
    for st, wh, cost, sig in (ex, ro):
        assert np.array_equal(st[:, -1], sig) and np.array_equal(st[:, 0] >> k, sig & mask)
        assert np.array_equal(st[:, 1:] >> k, st[:, :-1] & mask)
        np.testing.assert_array_equal(wh, c[st].reshape(B, -1))
    assert np.all(ro[2] >= ex[2])


def _random_cases(count=20, seed=6262):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for i in range(count):
        mode = "exact" if rng.integers(0, 2) else "rotate"
        k = int(rng.integers(1, 5))
        V = int(rng.integers(1, 3))
        if (k, V) == (2, 1):
            V = 2
        L = int(rng.integers(max(4, 2 * k), 11)) if mode == "exact" else int(rng.integers(max(4, 2 * k), 17))
        n = int(rng.integers(1, 40)) if L <= 12 else int(rng.integers(1, 12))
        B = int(rng.integers(1, 12)) if L <= 12 else int(rng.integers(1, 4))
        cases.append((i, mode, L, k, V, B, n))
    return cases


@pytest.mark.parametrize("i,mode,L,k,V,B,n", _random_cases())
def test_general_tail_biting_random_configuration(oracle_mod, dev, i, mode, L, k, V, B, n):
    w, c, _, _ = _vin(L, V, B, n, 9300 + i)
    print(f"random {i}: {mode} L{L} k{k} V{V} B{B} n{n}", flush=True)
    got = dba.viterbi_tail_biting(_t(w, dev), _t(c, dev), L, k, mode)
    _same(got, oracle_mod.viterbi_tail_biting(w, c, L, k, oracle_mod.TB_EXACT if mode == "exact" else
                                              oracle_mod.TB_ROTATE))


# ---------------------------------------------------------------- soft codeword and gradient under the measure

MEASURE = cases.TAIL_BITING_MEASURE_GENERAL


@pytest.mark.parametrize("L,k,V,B,n", MEASURE, ids=_ids(MEASURE))
def test_general_soft_tail_biting_matches_oracle(oracle_mod, dev, L, k, V, B, n):
    w, c, g, _ = _vin(L, V, B, n, 2400 + 31 * L + 7 * k + V + n)
    ok = True
    for T in [1.0, 0.1]:
        ws, lz = dba.soft_codeword_tail_biting(_t(w, dev), _t(c, dev), L, k, T, return_log_z=True)
        gr, ws2 = dba.soft_codeword_grad_tail_biting(_t(w, dev), _t(c, dev), _t(g, dev), L, k, T, return_w_soft=True)
        print(f"tail-biting measure L{L} k{k} V{V} B{B} n{n} T{T}:", flush=True)
        ok &= parity.tail_biting_ok(oracle_mod, ws, lz, gr, ws2, w, c, g, L, k, T)
    assert ok


def test_general_soft_tail_biting_is_the_sigma_mixture(dev):
    """ln Z under the measure is the log-sum over sigma of the sigma-mode ln Z (GPU path against itself), k = 3,
    V = 2."""
    L, k, V, B, n, T = 6, 3, 2, 4, 20, 0.3
    w, c, _, _ = _vin(L, V, B, n, 99)
    _, lz = dba.soft_codeword_tail_biting(_t(w, dev), _t(c, dev), L, k, T, return_log_z=True)
    S = 1 << L
    sig = torch.arange(S, dtype=torch.int32, device=dev).repeat(B)
    _, lz_s = dba.soft_codeword(_t(np.repeat(w, S, axis=0), dev), _t(c, dev), L, k, T, sig, return_log_z=True)
    ref = torch.logsumexp(lz_s.double().view(B, S), dim=1)
    assert float((lz.double() - ref).abs().max()) <= 1e-5 * float(ref.abs().max())
