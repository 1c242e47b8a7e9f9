"""Pins for the CPU oracle: it is checked against brute force, the Ising transfer-matrix identity, the free
energy, the T -> 0 and T -> infinity limits, symmetries and finite differences -- never against itself.

Sources: soft codeword = Boltzmann expectation of c(s_t) and exact differentiability (gist.science Technical
Summary, "Core Mechanism"); transfer-matrix equality and the T -> 0 limit (arXiv abstract).
"""
import numpy as np
import pytest

import pins
import workloads

TRELLISES = [(4, 2, 6), (5, 2, 5), (6, 2, 4), (4, 1, 8), (6, 3, 3)]


def _inputs(L, n, seed, B=3):
    rng = np.random.Generator(np.random.PCG64(seed))
    c = rng.standard_normal(1 << L).astype(np.float32)
    w = rng.standard_normal((B, n)).astype(np.float32)
    g = rng.standard_normal((B, n)).astype(np.float32)
    return w, c, g


# ---------------------------------------------------------------------------------------------- P1 brute force


@pytest.mark.parametrize("L,k,n", TRELLISES)
@pytest.mark.parametrize("T", [1.0, 0.3, 0.05])
def test_soft_matches_brute_force_free(oracle_mod, L, k, n, T):
    w, c, _ = _inputs(L, n, 11 * L + k + n)
    ws, lz, dev = oracle_mod.soft(w, c, L, k, T, with_check=True)
    paths = pins.free_paths(L, k, n)
    for b in range(w.shape[0]):
        ref, lnz, _ = pins.brute_soft(paths, w[b], c, T)
        np.testing.assert_allclose(ws[b], ref, rtol=0, atol=1e-12)
        assert abs(lz[b] - lnz) <= 1e-12 * max(1.0, abs(lnz))
    assert dev.max() < 1e-10


@pytest.mark.parametrize("L,k,n", TRELLISES)
def test_soft_matches_brute_force_sigma(oracle_mod, L, k, n):
    T = 0.4
    w, c, _ = _inputs(L, n, 7 * L + k)
    sig = np.array([0, (1 << L) - 1, 5 % (1 << L)], np.int32)
    ws, lz = oracle_mod.soft(w, c, L, k, T, sigma=sig)
    for b in range(w.shape[0]):
        paths = pins.sigma_paths(L, k, n, int(sig[b]))
        assert paths.shape[0] > 0
        ref, lnz, _ = pins.brute_soft(paths, w[b], c, T)
        np.testing.assert_allclose(ws[b], ref, rtol=0, atol=1e-12)
        assert abs(lz[b] - lnz) <= 1e-12 * max(1.0, abs(lnz))


def test_sigma_is_masked_to_L_bits(oracle_mod):
    L, k, n = 4, 2, 6
    w, c, _ = _inputs(L, n, 3)
    sig = np.array([3, 7, 9], np.int32)
    a, _ = oracle_mod.soft(w, c, L, k, 0.5, sigma=sig)
    b, _ = oracle_mod.soft(w, c, L, k, 0.5, sigma=sig + (1 << L) * np.array([1, 5, 2], np.int32))
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("L,k,n", TRELLISES)
@pytest.mark.parametrize("T", [1.0, 0.2])
def test_grad_matches_brute_force_jacobian(oracle_mod, L, k, n, T):
    w, c, g = _inputs(L, n, 5 * L + 3 * k + n)
    gr, ws = oracle_mod.grad(w, c, g, L, k, T)
    paths = pins.free_paths(L, k, n)
    for b in range(w.shape[0]):
        J = pins.brute_jacobian(paths, w[b], c, T)
        ref = J @ g[b].astype(np.float64)
        np.testing.assert_allclose(gr[b], ref, rtol=0, atol=1e-11 * max(1.0, np.abs(ref).max()))
        soft_ref, _, _ = pins.brute_soft(paths, w[b], c, T)
        np.testing.assert_allclose(ws[b], soft_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,k,n", [(4, 2, 6), (5, 2, 5), (4, 1, 8)])
def test_grad_matches_brute_force_sigma(oracle_mod, L, k, n):
    T = 0.7
    w, c, g = _inputs(L, n, 99 + L)
    sig = np.array([1, 6, (1 << L) - 2], np.int32)
    gr, _ = oracle_mod.grad(w, c, g, L, k, T, sigma=sig)
    for b in range(w.shape[0]):
        paths = pins.sigma_paths(L, k, n, int(sig[b]))
        J = pins.brute_jacobian(paths, w[b], c, T)
        ref = J @ g[b].astype(np.float64)
        np.testing.assert_allclose(gr[b], ref, rtol=0, atol=1e-11 * max(1.0, np.abs(ref).max()))


def test_brute_jacobian_is_the_derivative():
    """The covariance form of J used above equals finite differences of the brute-force soft codeword."""
    L, k, n, T = 4, 2, 5, 0.6
    w, c, _ = _inputs(L, n, 1234, B=1)
    paths = pins.free_paths(L, k, n)
    J = pins.brute_jacobian(paths, w[0], c, T)
    h = 1e-4
    w0 = w[0].astype(np.float64)
    for u in range(n):
        e = np.zeros(n)
        e[u] = h
        fp, _, _ = pins.brute_soft(paths, w0 + e, c, T)
        fm, _, _ = pins.brute_soft(paths, w0 - e, c, T)
        np.testing.assert_allclose((fp - fm) / (2 * h), J[:, u], rtol=0, atol=1e-6)


@pytest.mark.parametrize("L,k,n", TRELLISES)
def test_viterbi_matches_brute_force(oracle_mod, L, k, n):
    w, c, _ = _inputs(L, n, 17 * L + n, B=6)
    st, wh, cost = oracle_mod.viterbi(w, c, L, k)
    paths = pins.free_paths(L, k, n)
    for b in range(w.shape[0]):
        acc, argset = pins.brute_viterbi_fp32(paths, w[b], c)
        assert cost[b] == acc[argset[0]]                      # bit-exact fp32 cost
        if len(argset) == 1:
            np.testing.assert_array_equal(st[b], paths[argset[0]])
        else:
            assert any(np.array_equal(st[b], paths[i]) for i in argset)
        np.testing.assert_array_equal(wh[b], c[st[b]])


@pytest.mark.parametrize("L,k,n", [(4, 2, 6), (5, 2, 5), (6, 3, 3)])
def test_viterbi_sigma_matches_brute_force(oracle_mod, L, k, n):
    w, c, _ = _inputs(L, n, 3 * L + n, B=4)
    sig = np.array([0, 3, (1 << L) - 1, 10 % (1 << L)], np.int32)
    st, _, cost = oracle_mod.viterbi(w, c, L, k, sigma=sig)
    for b in range(w.shape[0]):
        paths = pins.sigma_paths(L, k, n, int(sig[b]))
        acc, argset = pins.brute_viterbi_fp32(paths, w[b], c)
        assert cost[b] == acc[argset[0]]
        assert any(np.array_equal(st[b], paths[i]) for i in argset)
        assert st[b, -1] == sig[b]


def test_viterbi_ties_take_smallest_predecessor_and_end_state(oracle_mod):
    """All-equal codebook: every path costs the same, so the tie rules alone pick the path (all zeros)."""
    L, k, n = 6, 2, 9
    c = np.full(1 << L, 0.25, np.float32)
    w = np.linspace(-1, 1, 2 * n, dtype=np.float32).reshape(2, n)
    st, _, _ = oracle_mod.viterbi(w, c, L, k)
    np.testing.assert_array_equal(st, 0)


# ------------------------------------------------------------------------------------------ P2 transfer matrix


@pytest.mark.parametrize("L,k,n,T", [(8, 2, 12, 0.5), (6, 2, 20, 0.1), (8, 1, 10, 1.0), (7, 2, 9, 2.0)])
def test_log_z_equals_ising_transfer_product(oracle_mod, L, k, n, T):
    w, c, _ = _inputs(L, n, 500 + L + n)
    _, lz = oracle_mod.soft(w, c, L, k, T)
    sig = np.array([1, 77 % (1 << L), (1 << L) - 1], np.int32)
    _, lzs = oracle_mod.soft(w, c, L, k, T, sigma=sig)
    for b in range(w.shape[0]):
        ref = pins.transfer_lnz_free(w[b].astype(np.float64), c, T, L, k)
        assert abs(lz[b] - ref) <= 1e-10 * max(1.0, abs(ref))
        refs = pins.transfer_lnz_sigma(w[b].astype(np.float64), c, T, L, k, int(sig[b]))
        assert abs(lzs[b] - refs) <= 1e-10 * max(1.0, abs(refs))


def test_tail_biting_partition_sums_sigma_partitions(oracle_mod):
    """Z_tb = trace of the transfer product = sum over sigma of Z_sigma."""
    L, k, n, T = 6, 2, 8, 0.5
    w, c, _ = _inputs(L, n, 42, B=1)
    sig = np.arange(1 << L, dtype=np.int32)
    wb = np.repeat(w, 1 << L, axis=0)
    _, lzs = oracle_mod.soft(wb, c, L, k, T, sigma=sig)
    M, ls = pins.transfer_product_log(w[0].astype(np.float64), c, T, L, k)
    ref = np.log(np.trace(M)) + ls
    m = lzs.max()
    got = m + np.log(np.exp(lzs - m).sum())
    assert abs(got - ref) <= 1e-10 * max(1.0, abs(ref))


# --------------------------------------------------------------------------------------------- P3 free energy


@pytest.mark.parametrize("sigma", [None, 37])
def test_soft_codeword_is_free_energy_derivative(oracle_mod, sigma):
    """w_soft_t = w_t + (T/2) d ln Z / d w_t, with ln Z from the transfer product and Richardson differences."""
    L, k, n, T = 8, 2, 10, 0.5
    w, c, _ = _inputs(L, n, 777, B=1)
    sg = None if sigma is None else np.array([sigma], np.int32)
    ws, _ = oracle_mod.soft(w, c, L, k, T, sigma=sg)
    w0 = w[0].astype(np.float64)

    def lnz(x):
        if sigma is None:
            return pins.transfer_lnz_free(x, c, T, L, k)
        return pins.transfer_lnz_sigma(x, c, T, L, k, sigma)

    h = 2e-3
    for t in range(n):
        e = np.zeros(n)
        e[t] = 1.0
        d1 = (lnz(w0 + h * e) - lnz(w0 - h * e)) / (2 * h)
        d2 = (lnz(w0 + 0.5 * h * e) - lnz(w0 - 0.5 * h * e)) / h
        deriv = (4 * d2 - d1) / 3
        assert abs(w0[t] + 0.5 * T * deriv - ws[0, t]) < 1e-8


# --------------------------------------------------------------------------------------------- P4 T -> 0


def test_low_temperature_recovers_viterbi_brute(oracle_mod):
    L, k, n = 5, 2, 6
    w, c, _ = _inputs(L, n, 2024, B=4)
    paths = pins.free_paths(L, k, n)
    st, _, _ = oracle_mod.viterbi(w, c, L, k)
    for b in range(w.shape[0]):
        E = pins.path_energies(paths, w[b], c)
        order = np.argsort(E)
        gap = E[order[1]] - E[order[0]]
        assert gap > 1e-6
        T = gap / 60.0
        ws, lz = oracle_mod.soft(w[b:b + 1], c, L, k, T)
        np.testing.assert_allclose(ws[0], c[paths[order[0]]], atol=1e-20 + 2 * np.abs(c).max() * 1e-20 + 1e-12)
        np.testing.assert_array_equal(st[b], paths[order[0]])
        assert abs(-T * lz[0] - E[order[0]]) <= T * np.log(paths.shape[0]) + 1e-12


def test_free_energy_bracket_and_convergence_L8(oracle_mod):
    """E* - T ln|P| <= -T ln Z <= E* at every T, with E* from a dense fp64 min-plus product."""
    L, k, n = 8, 2, 24
    w, c, _ = _inputs(L, n, 31337, B=2)
    A = pins.shift_matrix(L, k)
    for b in range(w.shape[0]):
        # dense min-plus over the window-overlap matrix
        v = (w[b, 0].astype(np.float64) - c.astype(np.float64)) ** 2
        inf_mask = np.where(A > 0, 0.0, np.inf)
        for t in range(1, n):
            e = (float(w[b, t]) - c.astype(np.float64)) ** 2
            v = (v[:, None] + inf_mask).min(axis=0) + e
        e_star = v.min()
        logP = L * np.log(2) + k * (n - 1) * np.log(2)
        for T in [1.0, 0.1, 0.01, 1e-3]:
            _, lz = oracle_mod.soft(w[b:b + 1], c, L, k, T)
            F = -T * lz[0]
            assert e_star - T * logP - 1e-9 <= F <= e_star + 1e-9
        st, _, cost = oracle_mod.viterbi(w[b:b + 1], c, L, k)
        e_path = ((w[b].astype(np.float64) - c.astype(np.float64)[st[0]]) ** 2).sum()
        assert abs(e_path - e_star) <= 1e-5 * e_star
        assert abs(float(cost[0]) - e_star) <= 1e-5 * e_star
        ws, _ = oracle_mod.soft(w[b:b + 1], c, L, k, 1e-6)
        assert np.mean(np.abs(ws[0] - c[st[0]])) < 1e-3


# --------------------------------------------------------------------------------------------- P5 T -> infinity


def test_high_temperature_limit_first_order(oracle_mod):
    L, k, n = 8, 2, 12
    w, c, g = _inputs(L, n, 4242, B=1)
    T = 1e6
    ws, _ = oracle_mod.soft(w, c, L, k, T)
    c64 = c.astype(np.float64)
    cbar = c64.mean()
    expect = np.zeros(n)
    for t in range(n):
        for u in range(n):
            f = (float(w[0, u]) - c64) ** 2
            if u >= t:
                expect[t] -= pins.uniform_lag_cov(L, k, u - t, c64, f)
            else:
                expect[t] -= pins.uniform_lag_cov(L, k, t - u, f, c64)
    np.testing.assert_allclose(T * (ws[0] - cbar), expect, rtol=1e-4, atol=1e-6)
    # gradient: (T/2) grad_u -> sum_t g_t Cov_unif(c(s_t), c(s_u))
    gr, _ = oracle_mod.grad(w, c, g, L, k, T)
    ref = np.zeros(n)
    for u in range(n):
        for t in range(n):
            lag = abs(t - u)
            ref[u] += float(g[0, t]) * pins.uniform_lag_cov(L, k, lag, c64, c64)
    np.testing.assert_allclose(0.5 * T * gr[0], ref, rtol=1e-4, atol=1e-6)


# --------------------------------------------------------------------------------------------- P6 invariants


def test_soft_codeword_within_codebook_range(oracle_mod):
    L, k, n = 8, 2, 40
    w, c, _ = _inputs(L, n, 8, B=4)
    for T in [10.0, 1.0, 0.01]:
        ws, _ = oracle_mod.soft(w * 3, c, L, k, T)
        lo, hi = float(c.min()), float(c.max())
        # fp64 rounding of exp(alpha + beta - ln Z) with |ln Z| ~ 1e4 at T = 0.01 allows ~1e-12 relative slack
        assert ws.min() >= lo - 1e-9 and ws.max() <= hi + 1e-9


def test_shift_and_scale_covariance(oracle_mod):
    L, k, n, T = 8, 2, 16, 0.3
    w, c, _ = _inputs(L, n, 9, B=2)
    w, c = pins.dyadic(w), pins.dyadic(c)
    ws, _ = oracle_mod.soft(w, c, L, k, T)
    ws2, _ = oracle_mod.soft(w + np.float32(0.5), c + np.float32(0.5), L, k, T)
    np.testing.assert_allclose(ws2, ws + 0.5, atol=1e-12)
    ws3, _ = oracle_mod.soft(2 * w, 2 * c, L, k, 4 * T)
    np.testing.assert_allclose(ws3, 2 * ws, atol=1e-12)


def test_time_reversal_with_symbol_reversed_codebook(oracle_mod):
    """Reversing time maps the left-shift trellis onto itself once the symbols of each state are reversed."""
    for L, k in [(8, 2), (6, 2), (6, 3)]:
        n, T = 14, 0.4
        w, c, g = _inputs(L, n, 60 + L + k, B=2)
        rho = pins.symbol_reverse(L, k)
        cr = c[rho]
        ws, lz = oracle_mod.soft(w, c, L, k, T)
        wr, lzr = oracle_mod.soft(w[:, ::-1], cr, L, k, T)
        np.testing.assert_allclose(wr[:, ::-1], ws, atol=1e-12)
        np.testing.assert_allclose(lzr, lz, rtol=1e-13)
        gr, _ = oracle_mod.grad(w, c, g, L, k, T)
        grr, _ = oracle_mod.grad(w[:, ::-1], cr, g[:, ::-1], L, k, T)
        np.testing.assert_allclose(grr[:, ::-1], gr, atol=1e-10)


# --------------------------------------------------------------------------------------------- P7 gradient


@pytest.mark.parametrize("T,sigma", [(0.5, None), (0.1, None), (0.5, 19)])
def test_grad_is_directional_derivative(oracle_mod, T, sigma):
    L, k, n = 8, 2, 12
    w, c, g = _inputs(L, n, 321, B=1)
    w = pins.dyadic(w, 12)
    sg = None if sigma is None else np.array([sigma], np.int32)
    gr, _ = oracle_mod.grad(w, c, g, L, k, T, sigma=sg)
    rng = np.random.Generator(np.random.PCG64(5))
    for _ in range(3):
        v = rng.integers(-1, 2, size=(1, n)).astype(np.float32)
        h = 2.0 ** -8

        def f(eps):
            ws, _ = oracle_mod.soft(w + np.float32(eps) * v, c, L, k, T, sigma=sg)
            return float(ws[0] @ g[0].astype(np.float64))

        d1 = (f(h) - f(-h)) / (2 * h)
        d2 = (f(h / 2) - f(-h / 2)) / h
        deriv = (4 * d2 - d1) / 3
        expect = float(gr[0] @ v[0].astype(np.float64))
        assert abs(deriv - expect) <= 1e-6 * max(1.0, abs(expect))


def test_jacobian_symmetric_and_psd(oracle_mod):
    L, k, n, T = 8, 2, 20, 0.2
    w, c, g = _inputs(L, n, 77, B=2)
    h = np.random.Generator(np.random.PCG64(1)).standard_normal(w.shape).astype(np.float32)
    jg, _ = oracle_mod.grad(w, c, g, L, k, T)
    jh, _ = oracle_mod.grad(w, c, h, L, k, T)
    for b in range(w.shape[0]):
        a = float(h[b].astype(np.float64) @ jg[b])
        bb = float(g[b].astype(np.float64) @ jh[b])
        assert abs(a - bb) <= 1e-10 * max(1.0, abs(a))
        assert float(g[b].astype(np.float64) @ jg[b]) >= -1e-12


# --------------------------------------------------------------------------------------------- workloads


def test_tiny_workload_sigma_and_free_self_consistent(oracle_mod):
    wl = workloads.WORKLOADS[1]
    c = wl.codebook()
    w = wl.weights()
    for T in wl.temps:
        ws, lz, dev = oracle_mod.soft(w, c, wl.L, wl.k, T, with_check=True)
        assert np.isfinite(ws).all() and np.isfinite(lz).all()
        assert dev.max() < 1e-8 * max(1.0, np.abs(lz).max())


# ------------------------------------------------------------------------------ P9 gradient in the codebook values


@pytest.mark.parametrize("L,k,n", TRELLISES)
@pytest.mark.parametrize("T", [1.0, 0.2])
def test_codebook_grad_matches_brute_force(oracle_mod, L, k, n, T):
    w, c, g = _inputs(L, n, 13 * L + 7 * k + n)
    gc, gw, ws = oracle_mod.grad_codebook(w, c, g, L, k, T, per_sequence=True)
    paths = pins.free_paths(L, k, n)
    for b in range(w.shape[0]):
        ref = g[b].astype(np.float64) @ pins.brute_codebook_jacobian(paths, w[b], c, T)
        np.testing.assert_allclose(gc[b], ref, rtol=0, atol=1e-11 * max(1.0, np.abs(ref).max()))
        Jw = pins.brute_jacobian(paths, w[b], c, T)
        np.testing.assert_allclose(gw[b], Jw @ g[b].astype(np.float64), rtol=0, atol=1e-11 * max(1.0, np.abs(gw[b]).max()))
    total, _, _ = oracle_mod.grad_codebook(w, c, g, L, k, T)
    np.testing.assert_allclose(total, gc.sum(axis=0), rtol=0, atol=1e-13 * max(1.0, np.abs(total).max()))


@pytest.mark.parametrize("L,k,n", [(4, 2, 6), (5, 2, 5), (4, 1, 8)])
def test_codebook_grad_matches_brute_force_sigma(oracle_mod, L, k, n):
    T = 0.6
    w, c, g = _inputs(L, n, 321 + L)
    sig = np.array([2, 9, (1 << L) - 3], np.int32)
    gc, _, _ = oracle_mod.grad_codebook(w, c, g, L, k, T, sigma=sig, per_sequence=True)
    for b in range(w.shape[0]):
        paths = pins.sigma_paths(L, k, n, int(sig[b]))
        ref = g[b].astype(np.float64) @ pins.brute_codebook_jacobian(paths, w[b], c, T)
        np.testing.assert_allclose(gc[b], ref, rtol=0, atol=1e-11 * max(1.0, np.abs(ref).max()))


def test_brute_codebook_jacobian_is_the_derivative():
    """The covariance form of the codebook Jacobian equals finite differences of the brute-force soft codeword."""
    L, k, n, T = 4, 2, 5, 0.7
    w, c, _ = _inputs(L, n, 4321, B=1)
    paths = pins.free_paths(L, k, n)
    K = pins.brute_codebook_jacobian(paths, w[0], c, T)
    h = 1e-4
    c0 = c.astype(np.float64)
    for v in range(1 << L):
        e = np.zeros(1 << L)
        e[v] = h
        fp, _, _ = pins.brute_soft(paths, w[0], c0 + e, T)
        fm, _, _ = pins.brute_soft(paths, w[0], c0 - e, T)
        np.testing.assert_allclose((fp - fm) / (2 * h), K[:, v], rtol=0, atol=1e-6)


@pytest.mark.parametrize("sigma", [None, 77])
def test_codebook_and_weight_grads_sum_to_upstream_total(oracle_mod, sigma):
    """Moving every codebook value and every weight by the same amount leaves the path measure alone and moves each
    w_soft_t by that amount, so sum_v dL/dc(v) + sum_u dL/dw_u = sum_t g_t exactly."""
    L, k, n, T = 8, 2, 40, 0.3
    w, c, g = _inputs(L, n, 555, B=3)
    sig = None if sigma is None else np.full(3, sigma, np.int32)
    gc, gw, _ = oracle_mod.grad_codebook(w, c, g, L, k, T, sigma=sig, per_sequence=True)
    for b in range(3):
        lhs = gc[b].sum() + gw[b].sum()
        rhs = g[b].astype(np.float64).sum()
        assert abs(lhs - rhs) <= 1e-10 * (np.abs(gc[b]).sum() + np.abs(gw[b]).sum() + np.abs(rhs))


def test_codebook_grad_low_temperature_is_viterbi_histogram(oracle_mod):
    """T -> 0: the measure sits on the best path s*, the covariance term dies as exp(-gap/T)/T, and dL/dc(v) tends to
    sum_t g_t [s*_t = v]."""
    L, k, n = 5, 2, 6
    w, c, g = _inputs(L, n, 777, B=3)
    paths = pins.free_paths(L, k, n)
    for b in range(3):
        E = pins.path_energies(paths, w[b], c)
        order = np.argsort(E)
        T = (E[order[1]] - E[order[0]]) / 60.0
        gc, _, _ = oracle_mod.grad_codebook(w[b:b + 1], c, g[b:b + 1], L, k, T)
        ref = np.zeros(1 << L)
        np.add.at(ref, paths[order[0]], g[b].astype(np.float64))
        np.testing.assert_allclose(gc, ref, rtol=0, atol=1e-9 * max(1.0, np.abs(ref).max()))


def test_codebook_grad_nan_when_no_path(oracle_mod):
    L, k, n = 6, 2, 2   # sigma mode needs n >= L/k
    w, c, g = _inputs(L, n, 9, B=2)
    gc, gw, _ = oracle_mod.grad_codebook(w, c, g, L, k, 0.5, sigma=np.array([5, 40], np.int32), per_sequence=True)
    assert np.isnan(gc).all() and np.isnan(gw).all()


# ------------------------------------------------------------------------------ P10 tail-biting with chosen sigma


def _brute_tail_biting(L, k, n, w, c):
    """(minimum fp32 cost over every tail-biting path, the smallest sigma attaining it, per-sigma argmin path sets)."""
    best, arg, sets = np.float32(np.inf), -1, {}
    for sig in range(1 << L):
        paths = pins.sigma_paths(L, k, n, sig)
        if paths.shape[0] == 0:
            continue
        acc, idx = pins.brute_viterbi_fp32(paths, w, c)
        sets[sig] = paths[idx]
        if acc.min() < best:
            best, arg = acc.min(), sig
    return best, arg, sets


@pytest.mark.parametrize("L,k,n", [(4, 2, 5), (4, 2, 7), (5, 2, 6), (4, 1, 7)])
def test_tail_biting_exact_matches_brute_force(oracle_mod, L, k, n):
    w, c, _ = _inputs(L, n, 808 + L + n, B=4)
    st, wh, cost, sig = oracle_mod.viterbi_tail_biting(w, c, L, k, oracle_mod.TB_EXACT)
    for b in range(w.shape[0]):
        best, arg, sets = _brute_tail_biting(L, k, n, w[b], c)
        assert cost[b] == best and sig[b] == arg
        assert any(np.array_equal(st[b], p) for p in sets[arg])
        np.testing.assert_array_equal(wh[b], c[st[b]])


def test_tail_biting_rotate_matches_brute_force_composition(oracle_mod):
    """The heuristic's steps redone by brute force: free minimum on the rotated weights, its state at the original
    last weight as sigma, then the sigma-constrained minimum."""
    L, k, n = 5, 2, 8
    w, c, _ = _inputs(L, n, 4242, B=5)
    st, _, cost, sig = oracle_mod.viterbi_tail_biting(w, c, L, k, oracle_mod.TB_ROTATE)
    free = pins.free_paths(L, k, n)
    r = n // 2
    for b in range(w.shape[0]):
        acc, idx = pins.brute_viterbi_fp32(free, np.roll(w[b], -r), c)
        assert sig[b] in {int(free[i][n - 1 - r]) for i in idx}
        acc2, idx2 = pins.brute_viterbi_fp32(pins.sigma_paths(L, k, n, int(sig[b])), w[b], c)
        assert cost[b] == acc2.min()


@pytest.mark.parametrize("mode", [0, 1])
def test_tail_biting_paths_close_the_cycle_and_exact_is_best(oracle_mod, mode):
    L, k, n = 8, 2, 40
    w, c, _ = _inputs(L, n, 99, B=6)
    st, _, cost, sig = oracle_mod.viterbi_tail_biting(w, c, L, k, mode)
    mask = (1 << (L - k)) - 1
    assert np.array_equal(st[:, -1], sig)                       # s_n = sigma
    assert np.array_equal(st[:, 0] >> k, sig & mask)            # s_1 is a successor of s_0 = sigma
    assert np.array_equal(st[:, 1:] >> k, st[:, :-1] & mask)    # every step is a trellis transition
    _, _, cost_exact, _ = oracle_mod.viterbi_tail_biting(w, c, L, k, 0)
    assert np.all(cost >= cost_exact)


# ------------------------------------------------------------------ P11 soft codeword under the tail-biting measure


def _tail_biting_paths(L, k, n):
    return np.concatenate([pins.sigma_paths(L, k, n, s) for s in range(1 << L)], axis=0)


@pytest.mark.parametrize("L,k,n", [(4, 2, 5), (4, 2, 7), (5, 2, 6), (4, 1, 7)])
@pytest.mark.parametrize("T", [1.0, 0.3])
def test_soft_tail_biting_matches_brute_force(oracle_mod, L, k, n, T):
    w, c, g = _inputs(L, n, 1717 + L + n)
    paths = _tail_biting_paths(L, k, n)
    ws, lz = oracle_mod.soft_tail_biting(w, c, L, k, T)
    gr, ws2 = oracle_mod.grad_tail_biting(w, c, g, L, k, T)
    for b in range(w.shape[0]):
        ref, lnz, _ = pins.brute_soft(paths, w[b], c, T)
        np.testing.assert_allclose(ws[b], ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(ws2[b], ref, rtol=0, atol=1e-12)
        assert abs(lz[b] - lnz) <= 1e-12 * max(1.0, abs(lnz))
        gref = pins.brute_jacobian(paths, w[b], c, T) @ g[b].astype(np.float64)
        np.testing.assert_allclose(gr[b], gref, rtol=0, atol=1e-11 * max(1.0, np.abs(gref).max()))


def test_soft_tail_biting_some_sigmas_unreachable(oracle_mod):
    """n below L/k: only the sigmas that can close the cycle carry weight."""
    L, k, n, T = 6, 2, 2, 0.5
    w, c, g = _inputs(L, n, 31, B=2)
    paths = _tail_biting_paths(L, k, n)
    ws, lz = oracle_mod.soft_tail_biting(w, c, L, k, T)
    gr, _ = oracle_mod.grad_tail_biting(w, c, g, L, k, T)
    for b in range(2):
        ref, lnz, _ = pins.brute_soft(paths, w[b], c, T)
        np.testing.assert_allclose(ws[b], ref, rtol=0, atol=1e-12)
        gref = pins.brute_jacobian(paths, w[b], c, T) @ g[b].astype(np.float64)
        np.testing.assert_allclose(gr[b], gref, rtol=0, atol=1e-11 * max(1.0, np.abs(gref).max()))


# ----------------------------------------------------------- P12 vector trellis (V weights per step) and k = 4
# A codebook [2^L, V] emits V weights per step; the path energy sums the squared distance over the components.

VEC_TRELLISES = [(4, 2, 5, 2), (4, 1, 6, 2), (6, 3, 3, 2), (4, 2, 4, 3), (8, 4, 2, 2)]


def _vec_inputs(L, n, V, seed, B=3):
    rng = np.random.Generator(np.random.PCG64(seed))
    c = rng.standard_normal((1 << L, V)).astype(np.float32)
    w = rng.standard_normal((B, n * V)).astype(np.float32)
    g = rng.standard_normal((B, n * V)).astype(np.float32)
    return w, c, g


@pytest.mark.parametrize("L,k,n,V", VEC_TRELLISES)
@pytest.mark.parametrize("T", [1.0, 0.3, 0.05])
def test_vector_soft_matches_brute_force(oracle_mod, L, k, n, V, T):
    w, c, _ = _vec_inputs(L, n, V, 31 * L + 7 * k + V)
    ws, lz, dev = oracle_mod.soft(w, c, L, k, T, with_check=True)
    assert ws.shape == w.shape
    paths = pins.free_paths(L, k, n)
    for b in range(w.shape[0]):
        ref, lnz, _ = pins.brute_soft(paths, w[b], c, T)
        np.testing.assert_allclose(ws[b], ref, rtol=0, atol=1e-12)
        assert abs(lz[b] - lnz) <= 1e-12 * max(1.0, abs(lnz))
    assert dev.max() < 1e-10
    sig = np.array([0, (1 << L) - 1, 5], np.int32)
    ws, lz = oracle_mod.soft(w, c, L, k, T, sigma=sig)
    for b in range(w.shape[0]):
        ref, lnz, _ = pins.brute_soft(pins.sigma_paths(L, k, n, int(sig[b])), w[b], c, T)
        np.testing.assert_allclose(ws[b], ref, rtol=0, atol=1e-12)
        assert abs(lz[b] - lnz) <= 1e-12 * max(1.0, abs(lnz))


@pytest.mark.parametrize("L,k,n,V", VEC_TRELLISES)
@pytest.mark.parametrize("sigma", [False, True])
def test_vector_grads_match_brute_force(oracle_mod, L, k, n, V, sigma):
    T = 0.5
    w, c, g = _vec_inputs(L, n, V, 7 * L + 3 * k + V + 1)
    sig = np.array([1, 6, (1 << L) - 2], np.int32) if sigma else None
    gc, gw, ws = oracle_mod.grad_codebook(w, c, g, L, k, T, sigma=sig, per_sequence=True)
    assert gc.shape == (w.shape[0], 1 << L, V) and gw.shape == w.shape
    for b in range(w.shape[0]):
        paths = pins.sigma_paths(L, k, n, int(sig[b])) if sigma else pins.free_paths(L, k, n)
        J = pins.brute_jacobian(paths, w[b], c, T)
        ref = J @ g[b].astype(np.float64)
        np.testing.assert_allclose(gw[b], ref, rtol=0, atol=1e-11 * max(1.0, np.abs(ref).max()))
        K = pins.brute_codebook_jacobian(paths, w[b], c, T)
        refc = (g[b].astype(np.float64) @ K).reshape(1 << L, V)
        np.testing.assert_allclose(gc[b], refc, rtol=0, atol=1e-11 * max(1.0, np.abs(refc).max()))
    gr, _ = oracle_mod.grad(w, c, g, L, k, T, sigma=sig)
    np.testing.assert_array_equal(gr, gw)


def test_vector_brute_jacobians_are_derivatives():
    """The covariance forms used above equal central differences of the brute-force soft codeword (V = 2)."""
    L, k, n, V, T = 4, 2, 3, 2, 0.6
    w, c, _ = _vec_inputs(L, n, V, 77, B=1)
    paths = pins.free_paths(L, k, n)
    w0, c0 = w[0].astype(np.float64), c.astype(np.float64)
    J = pins.brute_jacobian(paths, w0, c0, T)
    K = pins.brute_codebook_jacobian(paths, w0, c0, T)
    h = 1e-4
    for u in range(n * V):
        e = np.zeros(n * V)
        e[u] = h
        fp, _, _ = pins.brute_soft(paths, w0 + e, c0, T)
        fm, _, _ = pins.brute_soft(paths, w0 - e, c0, T)
        np.testing.assert_allclose((fp - fm) / (2 * h), J[:, u], rtol=0, atol=1e-6)
    for j in range(0, (1 << L) * V, 5):
        e = np.zeros((1 << L) * V)
        e[j] = h
        fp, _, _ = pins.brute_soft(paths, w0, c0 + e.reshape(c0.shape), T)
        fm, _, _ = pins.brute_soft(paths, w0, c0 - e.reshape(c0.shape), T)
        np.testing.assert_allclose((fp - fm) / (2 * h), K[:, j], rtol=0, atol=1e-6)


@pytest.mark.parametrize("L,k,n,V", VEC_TRELLISES)
def test_vector_viterbi_matches_brute_force(oracle_mod, L, k, n, V):
    w, c, _ = _vec_inputs(L, n, V, 5 * L + n + V, B=6)
    st, wh, cost = oracle_mod.viterbi(w, c, L, k)
    assert st.shape == (w.shape[0], n) and wh.shape == w.shape
    paths = pins.free_paths(L, k, n)
    for b in range(w.shape[0]):
        acc, argset = pins.brute_viterbi_fp32(paths, w[b], c)
        assert cost[b] == acc[argset[0]]
        assert any(np.array_equal(st[b], paths[i]) for i in argset)
        np.testing.assert_array_equal(wh[b], c[st[b]].reshape(-1))
    sig = np.array([0, 3, (1 << L) - 1, 10 % (1 << L), 1, 2], np.int32)
    st, _, cost = oracle_mod.viterbi(w, c, L, k, sigma=sig)
    for b in range(w.shape[0]):
        acc, argset = pins.brute_viterbi_fp32(pins.sigma_paths(L, k, n, int(sig[b])), w[b], c)
        assert cost[b] == acc[argset[0]] and st[b, -1] == sig[b]


@pytest.mark.parametrize("L,k,n,V,T", [(6, 2, 8, 2, 0.5), (8, 4, 5, 2, 0.3), (6, 1, 10, 3, 1.0)])
def test_vector_log_z_equals_ising_transfer_product(oracle_mod, L, k, n, V, T):
    w, c, _ = _vec_inputs(L, n, V, 900 + L + V)
    _, lz = oracle_mod.soft(w, c, L, k, T)
    sig = np.array([1, 21, (1 << L) - 1], np.int32)
    _, lzs = oracle_mod.soft(w, c, L, k, T, sigma=sig)
    for b in range(w.shape[0]):
        ref = pins.transfer_lnz_free(w[b].astype(np.float64), c, T, L, k)
        assert abs(lz[b] - ref) <= 1e-10 * max(1.0, abs(ref))
        refs = pins.transfer_lnz_sigma(w[b].astype(np.float64), c, T, L, k, int(sig[b]))
        assert abs(lzs[b] - refs) <= 1e-10 * max(1.0, abs(refs))


def test_vector_trellis_with_a_silent_component_is_the_scalar_trellis(oracle_mod):
    """V = 2 with the second codebook column and the second weight of every step at 0 is the V = 1 trellis on the
    first column: same ln Z, same first component, a zero second component, the same Viterbi path and cost."""
    L, k, n, T = 8, 2, 24, 0.2
    w1, c1, g1 = _inputs(L, n, 4242)
    c2 = np.stack([c1, np.zeros_like(c1)], axis=1)
    w2 = np.stack([w1, np.zeros_like(w1)], axis=2).reshape(w1.shape[0], 2 * n)
    g2 = np.stack([g1, np.zeros_like(g1)], axis=2).reshape(w1.shape[0], 2 * n)
    a, la = oracle_mod.soft(w1, c1, L, k, T)
    b, lb = oracle_mod.soft(w2, c2, L, k, T)
    np.testing.assert_array_equal(b[:, 0::2], a)
    np.testing.assert_array_equal(b[:, 1::2], 0.0)
    np.testing.assert_array_equal(lb, la)
    ga, _ = oracle_mod.grad(w1, c1, g1, L, k, T)
    gb, _ = oracle_mod.grad(w2, c2, g2, L, k, T)
    np.testing.assert_allclose(gb[:, 0::2], ga, rtol=0, atol=1e-12 * np.abs(ga).max())
    np.testing.assert_array_equal(gb[:, 1::2], 0.0)
    sa, _, ca = oracle_mod.viterbi(w1, c1, L, k)
    sb, _, cb = oracle_mod.viterbi(w2, c2, L, k)
    np.testing.assert_array_equal(sa, sb)
    np.testing.assert_array_equal(ca, cb)


# ------------------------------------------- P13 tail-biting on the general trellis (k = 1, 3, 4; V weights per step)
# The P10 and P11 pins again, on trellises other than k = 2, V = 1: every quantity by enumerating the paths with
# s_0 = s_n.

TB_TRELLISES = [(4, 1, 6, 1), (6, 3, 4, 1), (8, 4, 3, 1), (4, 2, 5, 2), (4, 1, 5, 2), (6, 3, 3, 2), (8, 4, 2, 2),
                (4, 2, 4, 3)]
TB_IDS = [f"L{L}k{k}n{n}V{V}" for L, k, n, V in TB_TRELLISES]


@pytest.mark.parametrize("L,k,n,V", TB_TRELLISES, ids=TB_IDS)
def test_vector_tail_biting_exact_matches_brute_force(oracle_mod, L, k, n, V):
    w, c, _ = _vec_inputs(L, n, V, 1300 + 31 * L + 7 * k + V)
    st, wh, cost, sig = oracle_mod.viterbi_tail_biting(w, c, L, k, oracle_mod.TB_EXACT)
    for b in range(w.shape[0]):
        best, arg, sets = _brute_tail_biting(L, k, n, w[b], c)
        assert cost[b] == best and sig[b] == arg
        assert any(np.array_equal(st[b], p) for p in sets[arg])
        np.testing.assert_array_equal(wh[b], c[st[b]].reshape(-1))


@pytest.mark.parametrize("L,k,n,V", [(4, 1, 7, 2), (6, 3, 4, 1), (8, 4, 3, 2)], ids=["L4k1V2", "L6k3V1", "L8k4V2"])
def test_vector_tail_biting_rotate_matches_brute_force_composition(oracle_mod, L, k, n, V):
    """Rotation by n // 2 trellis steps (n // 2 * V weights), then the sigma-constrained minimum, by brute force."""
    w, c, _ = _vec_inputs(L, n, V, 1400 + L + k, B=4)
    st, _, cost, sig = oracle_mod.viterbi_tail_biting(w, c, L, k, oracle_mod.TB_ROTATE)
    free = pins.free_paths(L, k, n)
    r = n // 2
    for b in range(w.shape[0]):
        acc, idx = pins.brute_viterbi_fp32(free, np.roll(w[b], -r * V), c)
        assert sig[b] in {int(free[i][n - 1 - r]) for i in idx}
        acc2, _ = pins.brute_viterbi_fp32(pins.sigma_paths(L, k, n, int(sig[b])), w[b], c)
        assert cost[b] == acc2.min()


@pytest.mark.parametrize("L,k,n,V", TB_TRELLISES, ids=TB_IDS)
@pytest.mark.parametrize("T", [1.0, 0.3])
def test_vector_soft_tail_biting_matches_brute_force(oracle_mod, L, k, n, V, T):
    w, c, g = _vec_inputs(L, n, V, 1500 + 31 * L + 7 * k + V)
    paths = _tail_biting_paths(L, k, n)
    ws, lz = oracle_mod.soft_tail_biting(w, c, L, k, T)
    gr, ws2 = oracle_mod.grad_tail_biting(w, c, g, L, k, T)
    for b in range(w.shape[0]):
        ref, lnz, _ = pins.brute_soft(paths, w[b], c, T)
        np.testing.assert_allclose(ws[b], ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(ws2[b], ref, rtol=0, atol=1e-12)
        assert abs(lz[b] - lnz) <= 1e-12 * max(1.0, abs(lnz))
        gref = pins.brute_jacobian(paths, w[b], c, T) @ g[b].astype(np.float64)
        np.testing.assert_allclose(gr[b], gref, rtol=0, atol=1e-11 * max(1.0, np.abs(gref).max()))
