"""GPU parity: the HIP path, called through the C-ABI, against the CPU oracle on the same seeded inputs.

Bars (tests/parity.py):
* Viterbi states, codewords and float32 path costs: bit-exact.
* Soft codeword, ln Z, gradient (elementwise and as a vector): max(1e-5, kappa), kappa being the case's one-ulp
  conditioning, which the oracle alone computes by moving every float32 weight and codebook value by one ulp.  A
  well-conditioned case is held to the benchmark spec's 1e-5; one whose exact answer itself moves by more than that when
  its inputs move by one float32 ulp is held to that movement, the resolution float32 inputs carry.
* Full-size workloads: the whole batch runs on the GPU in the launch configuration the benchmark times, and 64 sampled
  rows (rows 0 and B - 1 among them) are compared with stored oracle answers and kappas
  (tests/golden/make_full_size.py).
* Below T = 0.01 the soft codeword is also checked for convergence to the Viterbi code.
"""
import numpy as np
import pytest
import torch

import cases
import differentiable_bcjr_amd as dba
import parity
import workloads
from differentiable_bcjr_amd import abi
from parity import check, grad_norm_rows, grad_rows, lz_rows, rel_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


_inputs = cases.inputs


def _t(a, dev):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)


SMALL = [(4, 16, 6), (5, 7, 9), (6, 5, 33), (8, 16, 64), (8, 3, 1), (8, 2, 2), (9, 5, 17), (10, 9, 40), (12, 3, 20),
         (13, 2, 11), (14, 2, 12), (15, 2, 10), (16, 2, 8)]
TEMPS = [1.0, 0.1, 0.01]
GRAD_TEMPS = [1.0, 0.1, 0.05, 0.01]


@pytest.mark.parametrize("L,B,n", SMALL)
@pytest.mark.parametrize("sigma", [False, True])
def test_soft_codeword_matches_oracle(oracle_mod, dev, L, B, n, sigma):
    if sigma and n < (L + 1) // 2:
        n = (L + 1) // 2 + 1   # the sigma constraint needs at least L/k steps to be satisfiable for every sigma
    w, c, _, s = _inputs(L, B, n, 100 + 7 * L + n, sigma)
    ok = True
    for T in TEMPS:
        got, lz = dba.soft_codeword(_t(w, dev), _t(c, dev), L, 2, T, _t(s, dev), return_log_z=True)
        ref, rlz, k_ws, k_lz = parity.soft_reference(oracle_mod, w, c, L, 2, T, sigma=s)
        print(f"soft L={L} B={B} n={n} T={T} sigma={sigma}:", flush=True)
        ok &= check("w_soft", rel_rows(got.cpu().numpy(), ref), k_ws)
        ok &= check("ln Z", lz_rows(lz.cpu().numpy(), rlz), k_lz)
    assert ok


@pytest.mark.parametrize("L,B,n", SMALL)
@pytest.mark.parametrize("sigma", [False, True])
def test_gradient_matches_oracle(oracle_mod, dev, L, B, n, sigma):
    if sigma and n < (L + 1) // 2 + 2:
        n = (L + 1) // 2 + 2   # a unique path (n = L/k) has an exactly zero gradient, checked separately
    B = max(B, 4)             # the error floor is the batch rms: keep some sequences whose posterior is not frozen
    w, c, g, s = _inputs(L, B, n, 200 + 5 * L + n, sigma)
    ok = True
    for T in GRAD_TEMPS:
        got, ws = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), L, 2, T, _t(s, dev),
                                         return_w_soft=True)
        print(f"grad L={L} B={B} n={n} T={T} sigma={sigma}:", flush=True)
        ok &= parity.grad_ok(oracle_mod, got, ws, w, c, g, L, 2, T, s)
    assert ok


@pytest.mark.parametrize("L,B,n", SMALL)
@pytest.mark.parametrize("sigma", [False, True])
def test_viterbi_bit_exact(oracle_mod, dev, L, B, n, sigma):
    if sigma and n < (L + 1) // 2:
        n = (L + 1) // 2 + 1
    w, c, _, s = _inputs(L, B, n, 300 + 3 * L + n, sigma)
    st, wh, cost = dba.viterbi_hard_code(_t(w, dev), _t(c, dev), L, 2, _t(s, dev))
    rst, rwh, rcost = oracle_mod.viterbi(w, c, L, 2, sigma=s)
    print(f"viterbi L={L} B={B} n={n} sigma={sigma}", flush=True)
    np.testing.assert_array_equal(st.cpu().numpy(), rst)
    np.testing.assert_array_equal(cost.cpu().numpy().view(np.uint32), rcost.view(np.uint32))
    np.testing.assert_array_equal(wh.cpu().numpy(), rwh)


def test_viterbi_ties_follow_the_documented_rule(oracle_mod, dev):
    """All-equal codebook: every path ties, so the smallest-index rules alone fix the path (all zeros)."""
    for L in (6, 16):
        c = np.full(1 << L, 0.25, np.float32)
        w = np.linspace(-1, 1, 3 * 9, dtype=np.float32).reshape(3, 9)
        st, _, _ = dba.viterbi_hard_code(_t(w, dev), _t(c, dev), L)
        assert (st.cpu().numpy() == 0).all()


@pytest.mark.parametrize("L", [6, 8, 16])
def test_unique_sigma_path_has_zero_gradient(oracle_mod, dev, L):
    """n = L/k with s_0 = s_n = sigma leaves exactly one path: w_soft is its codeword sequence, the gradient is 0."""
    n = L // 2
    w, c, g, s = _inputs(L, 3, n, 77, True)
    for T in (1.0, 0.01):
        gr, ws = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), L, 2, T, _t(s, dev),
                                        return_w_soft=True)
        st, _, _ = oracle_mod.viterbi(w, c, L, 2, sigma=s)
        np.testing.assert_allclose(ws.cpu().numpy(), c[st], rtol=0, atol=1e-6)
        assert float(gr.abs().max()) <= 1e-6 * (2.0 / T)


def test_unsatisfiable_sigma_gives_nan_and_inf(dev):
    L, n = 8, 2   # 2 steps cannot bring a generic sigma back to itself
    w, c, g, _ = _inputs(L, 2, n, 9)
    s = np.array([0b10110001, 0b01001110], np.int32)
    ws, lz = dba.soft_codeword(_t(w, dev), _t(c, dev), L, 2, 0.5, _t(s, dev), return_log_z=True)
    assert torch.isnan(ws).all() and torch.isinf(lz).all() and (lz < 0).all()
    gr = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), L, 2, 0.5, _t(s, dev))
    assert torch.isnan(gr).all()
    _, _, cost = dba.viterbi_hard_code(_t(w, dev), _t(c, dev), L, 2, _t(s, dev))
    assert torch.isinf(cost).all()


def test_outputs_are_deterministic(dev):
    L, B, n = 16, 300, 32
    w, c, g, _ = _inputs(L, B, n, 11)
    a = dba.soft_codeword(_t(w, dev), _t(c, dev), L, 2, 0.1)
    b = dba.soft_codeword(_t(w, dev), _t(c, dev), L, 2, 0.1)
    assert torch.equal(a, b)
    ga = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), L, 2, 0.1)
    gb = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), L, 2, 0.1)
    assert torch.equal(ga, gb)


def test_raw_abi_call_on_a_stream(oracle_mod, dev):
    """The C entry point itself, with a caller-owned workspace on a non-default stream."""
    L, B, n, T = 8, 6, 20, 0.3
    w, c, _, _ = _inputs(L, B, n, 5)
    wt, ct = _t(w, dev), _t(c, dev)
    out = torch.empty_like(wt)
    need = abi.bcjr_workspace_bytes(abi.BCJR_OP_SOFT, B, n, L, 2)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    st = torch.cuda.Stream(dev)
    with torch.cuda.stream(st):
        rc = abi.bcjr_soft_codeword(wt.data_ptr(), ct.data_ptr(), B, n, L, 2, T, None, out.data_ptr(), None,
                                    ws.data_ptr(), need, st.cuda_stream)
    assert rc == abi.BCJR_OK
    st.synchronize()
    ref, _, k_ws, _ = parity.soft_reference(oracle_mod, w, c, L, 2, T)
    assert check("w_soft", rel_rows(out.cpu().numpy(), ref), k_ws)


# ------------------------------------------------------------------------------------------------------------------
# full-size workloads, in the launch configuration the benchmark times; sampled rows against the oracle


# The full-size gates: every sampled row as a vector (normwise) within max(1e-5, its random kappa), and rows 0 and
# B - 1 element by element within max(1e-5, their kappa), the larger of the first-order and the random estimates
# (the first-order one is stored for those two rows only).  The 64 rows' elementwise errors against the random
# estimate alone are printed as well, as a report.

FO = [0, -1]   # positions of rows 0 and B - 1 in the stored sample


def _golden_soft(G, got, lz, T, sigma=False):
    """A stored soft-codeword entry against the GPU's answers on its rows."""
    key = parity.golden_key("soft", T, sigma)
    rows = G["rows"]
    x, ref = got.cpu().numpy()[rows], G[key + "/w_soft"]
    ok = check(f"{key} w_soft normwise, {len(rows)} rows", parity.rel_norm_rows(x, ref), G[key + "/kappa_w_soft_norm"])
    k_fo = np.maximum(G[key + "/kappa_w_soft"][FO], G[key + "/fo_kappa_w_soft"])
    ok &= check(f"{key} w_soft, rows 0 and B-1", rel_rows(x[FO], ref[FO]), k_fo)
    check(f"{key} w_soft, {len(rows)} rows against the random kappa (report)", rel_rows(x, ref),
          G[key + "/kappa_w_soft"])
    if lz is not None:
        ok &= check(f"{key} ln Z", lz_rows(lz.cpu().numpy()[rows], G[key + "/log_z"]), G[key + "/kappa_log_z"])
    return ok


def _golden_grad(G, gr, ws, g, c, T, sigma=False):
    """A stored gradient entry (gradient elementwise and as a vector, and the pass's soft codeword) against the
    GPU's answers on its rows."""
    key = parity.golden_key("grad", T, sigma)
    rows = G["rows"]
    T = parity.t32(T)
    floor = float(G[key + "/grad_floor"])
    got, ref, gs = gr.cpu().numpy()[rows], G[key + "/grad"], g[rows]
    ok = check(f"{key} grad normwise, {len(rows)} rows", grad_norm_rows(got, ref, gs, c, T, floor),
               G[key + "/kappa_grad_norm"])
    k_fo = np.maximum(G[key + "/kappa_grad"][FO], G[key + "/fo_kappa_grad"])
    ok &= check(f"{key} grad, rows 0 and B-1", grad_rows(got[FO], ref[FO], gs[FO], c, T, floor), k_fo)
    check(f"{key} grad, {len(rows)} rows against the random kappa (report)", grad_rows(got, ref, gs, c, T, floor),
          G[key + "/kappa_grad"])
    if ws is not None:
        x, rws = ws.cpu().numpy()[rows], G[key + "/w_soft"]
        k_fo = np.maximum(G[key + "/kappa_w_soft"][FO], G[key + "/fo_kappa_w_soft"])
        ok &= check(f"{key} w_soft, rows 0 and B-1", rel_rows(x[FO], rws[FO]), k_fo)
    return ok


def _viterbi_rows(oracle_mod, st, wh, cost, w, c, wl, rows, sig=None):
    rst, rwh, rcost = oracle_mod.viterbi(w[rows], c, wl.L, wl.k, sigma=None if sig is None else sig[rows])
    np.testing.assert_array_equal(st.cpu().numpy()[rows], rst)
    if wh is not None:
        np.testing.assert_array_equal(wh.cpu().numpy()[rows].view(np.uint32), rwh.view(np.uint32))
    np.testing.assert_array_equal(cost.cpu().numpy()[rows].view(np.uint32), rcost.view(np.uint32))
    return rst


def test_headline_workload_sampled(dev):
    """4096 sequences x 256 weights, 2^16-state trellis (a 1024x1024 matrix): the benchmark's workload."""
    wl = workloads.WORKLOADS[2]
    G = parity.load_golden(2)
    wt, ct = _t(wl.weights(), dev), _t(wl.codebook(), dev)
    ok = True
    for T in wl.temps:
        got, lz = dba.soft_codeword(wt, ct, wl.L, wl.k, T, return_log_z=True)
        print(f"headline T={T}, {len(G['rows'])} rows:", flush=True)
        ok &= _golden_soft(G, got, lz, T)
    assert ok


def test_headline_workload_gradient_and_viterbi_sampled(oracle_mod, dev):
    """The benchmark's step on the same workload: gradient at T = 0.1 and the Viterbi code."""
    wl = workloads.WORKLOADS[2]
    G = parity.load_golden(2)
    c, w, g = wl.codebook(), wl.weights(), wl.upstream_grad()
    T = 0.1
    wt, ct = _t(w, dev), _t(c, dev)
    gr, ws = dba.soft_codeword_grad(wt, ct, _t(g, dev), wl.L, wl.k, T, return_w_soft=True)
    print(f"headline grad, {len(G['rows'])} rows:", flush=True)
    assert _golden_grad(G, gr, ws, g, c, T)
    st, wh, cost = dba.viterbi_hard_code(wt, ct, wl.L, wl.k)
    _viterbi_rows(oracle_mod, st, wh, cost, w, c, wl, G["rows"])


# ------------------------------------------------------------------------------------------------------------------
# shape edges: the longest sequences, one sequence, batches that leave a block partly idle or make blocks loop


@pytest.mark.parametrize("sigma", [False, True])
def test_longest_sequences(oracle_mod, dev, sigma):
    """n = 4096, the largest the boundary accepts, on a 2^10-state trellis."""
    L, B, n, T = 10, 2, 4096, 0.1
    w, c, g, s = _inputs(L, B, n, 77, sigma)
    wt, ct, st_ = _t(w, dev), _t(c, dev), _t(s, dev)
    got, lz = dba.soft_codeword(wt, ct, L, 2, T, st_, return_log_z=True)
    ref, rlz, k_ws, k_lz = parity.soft_reference(oracle_mod, w, c, L, 2, T, sigma=s)
    print(f"n=4096 sigma={sigma}:", flush=True)
    ok = check("w_soft", rel_rows(got.cpu().numpy(), ref), k_ws)
    ok &= check("ln Z", lz_rows(lz.cpu().numpy(), rlz), k_lz)
    gr = dba.soft_codeword_grad(wt, ct, _t(g, dev), L, 2, T, st_)
    ok &= parity.grad_ok(oracle_mod, gr, None, w, c, g, L, 2, T, s)
    assert ok
    stt, _, cost = dba.viterbi_hard_code(wt, ct, L, 2, st_)
    rst, _, rcost = oracle_mod.viterbi(w, c, L, 2, sigma=s)
    np.testing.assert_array_equal(stt.cpu().numpy(), rst)
    np.testing.assert_array_equal(cost.cpu().numpy().view(np.uint32), rcost.view(np.uint32))


@pytest.mark.parametrize("L,B,n,rows", cases.BATCH_EDGES)
def test_batch_edges(oracle_mod, dev, L, B, n, rows):
    T = 0.1
    w, c, g, _ = _inputs(L, B, n, 900 + L)
    rows = np.asarray(rows)
    wt, ct = _t(w, dev), _t(c, dev)
    got = dba.soft_codeword(wt, ct, L, 2, T).cpu().numpy()[rows]
    ref, _, k_ws, _ = parity.soft_reference(oracle_mod, w[rows], c, L, 2, T)
    ok = check("w_soft", rel_rows(got, ref), k_ws)
    gr = dba.soft_codeword_grad(wt, ct, _t(g, dev), L, 2, T)
    ok &= parity.grad_ok(oracle_mod, gr, None, w, c, g, L, 2, T, None, rows=rows)
    assert ok
    st, _, cost = dba.viterbi_hard_code(wt, ct, L, 2)
    rst, _, rcost = oracle_mod.viterbi(w[rows], c, L, 2)
    np.testing.assert_array_equal(st.cpu().numpy()[rows], rst)
    np.testing.assert_array_equal(cost.cpu().numpy()[rows].view(np.uint32), rcost.view(np.uint32))


def test_mlp_layer_gradient_sampled(oracle_mod, dev):
    """65536 sequences (an 8192x2048 matrix), T = 0.05: soft codeword and gradient."""
    wl = workloads.WORKLOADS[3]
    G = parity.load_golden(3)
    c, w, g = wl.codebook(), wl.weights(), wl.upstream_grad()
    T = wl.temps[0]
    gr, ws = dba.soft_codeword_grad(_t(w, dev), _t(c, dev), _t(g, dev), wl.L, wl.k, T, return_w_soft=True)
    print(f"mlp layer, {len(G['rows'])} rows:", flush=True)
    assert _golden_grad(G, gr, ws, g, c, T)


def test_low_temperature_sweep_and_viterbi_sampled(oracle_mod, dev):
    """16384 sequences (2048x2048): Viterbi bit-exact (free and sigma), soft codeword down to T = 1e-4."""
    wl = workloads.WORKLOADS[4]
    G = parity.load_golden(4)
    rows = G["rows"]
    c, w = wl.codebook(), wl.weights()
    sig = wl.boundary_states()
    wt, ct = _t(w, dev), _t(c, dev)
    st, wh, cost = dba.viterbi_hard_code(wt, ct, wl.L, wl.k)
    rst = _viterbi_rows(oracle_mod, st, wh, cost, w, c, wl, rows)
    sts, whs, costs = dba.viterbi_hard_code(wt, ct, wl.L, wl.k, _t(sig, dev))
    _viterbi_rows(oracle_mod, sts, whs, costs, w, c, wl, rows, sig)
    hard = c[rst]
    ok = True
    for T in wl.temps:
        got = dba.soft_codeword(wt, ct, wl.L, wl.k, T)
        print(f"low-T T={T}, {len(rows)} rows: median |w_soft - c(s*)| "
              f"{float(np.median(np.abs(got.cpu().numpy()[rows] - hard))):.2e}", flush=True)
        ok &= _golden_soft(G, got, None, T)
    assert ok
    # convergence to the hard code as T -> 0
    got = dba.soft_codeword(wt, ct, wl.L, wl.k, 1e-4).cpu().numpy()[rows]
    assert np.mean(np.abs(got - hard) < 1e-3) > 0.9


def test_low_temperature_workload_sigma_sampled(dev):
    """The same 16384 sequences with s_0 = s_n = sigma: soft codeword at T = 0.1 and 0.01, gradient at T = 0.1."""
    wl = workloads.WORKLOADS[4]
    G = parity.load_golden(4)
    c, w, g = wl.codebook(), wl.weights(), wl.upstream_grad()
    sig = wl.boundary_states()
    wt, ct, st_ = _t(w, dev), _t(c, dev), _t(sig, dev)
    ok = True
    for T in (0.1, 0.01):
        got, lz = dba.soft_codeword(wt, ct, wl.L, wl.k, T, st_, return_log_z=True)
        print(f"low-T sigma T={T}, {len(G['rows'])} rows:", flush=True)
        ok &= _golden_soft(G, got, lz, T, sigma=True)
    T = 0.1
    gr, ws = dba.soft_codeword_grad(wt, ct, _t(g, dev), wl.L, wl.k, T, st_, return_w_soft=True)
    print(f"low-T sigma grad T={T}:", flush=True)
    ok &= _golden_grad(G, gr, ws, g, c, T, sigma=True)
    assert ok


@pytest.mark.slow
def test_whole_decoder_layer_sampled(dev):
    """All seven Llama-3.2-1B projection shapes as one batch of 237,568 sequences, T = 0.05."""
    wl = workloads.WORKLOADS[5]
    G = parity.load_golden(5)
    c, w, g = wl.codebook(), wl.weights(), wl.upstream_grad()
    T = wl.temps[0]
    wt, ct, gt = _t(w, dev), _t(c, dev), _t(g, dev)
    ws = dba.soft_codeword(wt, ct, wl.L, wl.k, T)
    gr = dba.soft_codeword_grad(wt, ct, gt, wl.L, wl.k, T)
    print(f"decoder layer, {len(G['rows'])} rows (soft codeword from its own call):", flush=True)
    assert _golden_grad(G, gr, ws, g, c, T)


# ------------------------------------------------------------------------------------------------------------------
# a seeded sweep over shapes, temperatures and boundary modes (every draw is checked like the fixed cases above)

def _random_cases(count=36, seed=2024):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for i in range(count):
        L = int(rng.integers(4, 17))
        n = int(rng.integers(1, 81)) if L <= 12 else int(rng.integers(1, 25))
        B = int(rng.integers(1, 41)) if L <= 12 else int(rng.integers(1, 5))
        T = float(rng.choice([1.0, 0.3, 0.1, 0.05]))
        sigma = bool(rng.integers(0, 2)) and n >= (L + 1) // 2   # sigma needs L/k steps to reach every state
        cases.append((i, L, B, n, T, sigma))
    return cases


@pytest.mark.parametrize("i,L,B,n,T,sigma", _random_cases())
def test_random_configuration(oracle_mod, dev, i, L, B, n, T, sigma):
    w, c, g, s = _inputs(L, B, n, 5000 + i, sigma)
    wt, ct, st_ = _t(w, dev), _t(c, dev), _t(s, dev)
    got, lz = dba.soft_codeword(wt, ct, L, 2, T, st_, return_log_z=True)
    ref, rlz, k_ws, k_lz = parity.soft_reference(oracle_mod, w, c, L, 2, T, sigma=s)
    print(f"random {i}: L={L} B={B} n={n} T={T} sigma={sigma}:", flush=True)
    ok = check("w_soft", rel_rows(got.cpu().numpy(), ref), k_ws)
    ok &= check("ln Z", lz_rows(lz.cpu().numpy(), rlz), k_lz)
    gr, ws = dba.soft_codeword_grad(wt, ct, _t(g, dev), L, 2, T, st_, return_w_soft=True)
    ok &= parity.grad_ok(oracle_mod, gr, ws, w, c, g, L, 2, T, s)
    assert ok
    stt, wh, cost = dba.viterbi_hard_code(wt, ct, L, 2, st_)
    rst, rwh, rcost = oracle_mod.viterbi(w, c, L, 2, sigma=s)
    np.testing.assert_array_equal(stt.cpu().numpy(), rst)
    np.testing.assert_array_equal(wh.cpu().numpy().view(np.uint32), rwh.view(np.uint32))
    np.testing.assert_array_equal(cost.cpu().numpy().view(np.uint32), rcost.view(np.uint32))


# ------------------------------------------------------------------------------------------------------------------
# execution: the entry points allocate nothing and only launch kernels, so they can be captured in a HIP graph and
# run concurrently on separate streams with separate workspaces


def _raw_step(wt, ct, gt, L, n, T, ws, outs, stream):
    B = wt.shape[0]
    w_soft, log_z, grad, states, w_hard, cost = outs
    sp = stream.cuda_stream
    assert abi.bcjr_soft_codeword(wt.data_ptr(), ct.data_ptr(), B, n, L, 2, T, None, w_soft.data_ptr(),
                                  log_z.data_ptr(), ws.data_ptr(), ws.numel(), sp) == abi.BCJR_OK
    assert abi.bcjr_soft_codeword_grad(wt.data_ptr(), ct.data_ptr(), B, n, L, 2, T, None, gt.data_ptr(),
                                       grad.data_ptr(), None, ws.data_ptr(), ws.numel(), sp) == abi.BCJR_OK
    assert abi.viterbi_hard_code(wt.data_ptr(), ct.data_ptr(), B, n, L, 2, None, states.data_ptr(),
                                 w_hard.data_ptr(), cost.data_ptr(), ws.data_ptr(), ws.numel(), sp) == abi.BCJR_OK


def _outs(B, n, dev):
    f = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)
    return [f(B, n), f(B), f(B, n), torch.empty((B, n), dtype=torch.int32, device=dev), f(B, n), f(B)]


def test_graph_capture_replays_match_eager(dev):
    L, B, n, T = 12, 40, 24, 0.2
    w, c, g, _ = _inputs(L, B, n, 31)
    wt, ct, gt = _t(w, dev), _t(c, dev), _t(g, dev)
    ws = torch.empty(max(abi.bcjr_workspace_bytes(op, B, n, L, 2) for op in (0, 1, 2)), dtype=torch.uint8, device=dev)
    eager = _outs(B, n, dev)
    _raw_step(wt, ct, gt, L, n, T, ws, eager, torch.cuda.current_stream(dev))
    torch.cuda.synchronize()
    graph_outs = _outs(B, n, dev)
    side = torch.cuda.Stream(dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        _raw_step(wt, ct, gt, L, n, T, ws, graph_outs, side)
    for rep in range(3):
        for o in graph_outs:
            o.fill_(-7)                      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(graph_outs, eager):
            assert torch.equal(a, b), f"replay {rep} differs from the eager call"


def test_concurrent_streams_with_separate_workspaces(dev):
    L, B, n, T = 14, 6, 32, 0.1
    inputs = [_inputs(L, B, n, 40 + i) for i in range(2)]
    ref = []
    for w, c, g, _ in inputs:
        o = _outs(B, n, dev)
        ws = torch.empty(max(abi.bcjr_workspace_bytes(op, B, n, L, 2) for op in (0, 1, 2)), dtype=torch.uint8,
                         device=dev)
        _raw_step(_t(w, dev), _t(c, dev), _t(g, dev), L, n, T, ws, o, torch.cuda.current_stream(dev))
        ref.append(o)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(dev) for _ in range(2)]
    outs = [_outs(B, n, dev) for _ in range(2)]
    wss = [torch.empty(max(abi.bcjr_workspace_bytes(op, B, n, L, 2) for op in (0, 1, 2)), dtype=torch.uint8,
                       device=dev) for _ in range(2)]
    tens = [tuple(_t(a, dev) for a in inp[:3]) for inp in inputs]
    torch.cuda.synchronize()
    for rep in range(3):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                _raw_step(*tens[i], L, n, T, wss[i], outs[i], streams[i])
        torch.cuda.synchronize()
        for i in range(2):
            for a, b in zip(outs[i], ref[i]):
                assert torch.equal(a, b)


@pytest.mark.parametrize("sigma", [False, True])
def test_soft_quantize_autograd(oracle_mod, dev, sigma):
    """Autograd through soft_quantize gives the soft codeword forward and the exact weights' gradient backward."""
    L, B, n, T = 10, 6, 24, 0.1
    w, c, g, s = _inputs(L, B, n, 61, sigma)
    wt = _t(w, dev).requires_grad_(True)
    out = dba.soft_quantize(wt, _t(c, dev), L, 2, T, _t(s, dev))
    (out * _t(g, dev)).sum().backward()
    ref, _, k_ws, _ = parity.soft_reference(oracle_mod, w, c, L, 2, T, sigma=s)
    ok = check("w_soft", rel_rows(out.detach().cpu().numpy(), ref), k_ws)
    ok &= parity.grad_ok(oracle_mod, wt.grad, None, w, c, g, L, 2, T, s)
    assert ok
    assert wt.grad.dtype == torch.float32
