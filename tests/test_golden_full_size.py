"""The stored full-size references (tests/golden/full_size_cfg<N>.npz) are the oracle's, on the CPU.

Each file holds, for 64 sampled rows of a full-size workload, the oracle's answers and each row's one-ulp conditioning
kappa, written by tests/golden/make_full_size.py.  Here row 0 or row B - 1 of every entry (the first and last rows of
the matrix, both always sampled) is recomputed with the oracle and must match the stored values exactly, and so must
its kappas, recomputed from the same seeded one-ulp draws (the oracle treats every sequence on its own, so a row's
answers and kappa do not depend on the other rows computed with it).  The GPU tests compare the GPU path with these
rows.
"""
import numpy as np
import pytest

import parity
import workloads

SPECS = {
    2: [("soft", 1.0, False), ("soft", 0.1, False), ("soft", 0.01, False), ("grad", 0.1, False)],
    3: [("grad", 0.05, False)],
    4: [("soft", 0.1, False), ("soft", 0.01, False), ("soft", 1e-3, False), ("soft", 1e-4, False),
        ("soft", 0.1, True), ("soft", 0.01, True), ("grad", 0.1, True)],
    5: [("grad", 0.05, False)],
}
ROWS = 64


def _seed(cfg, sigma):
    return 7000 + 10 * cfg + int(sigma)


def test_stored_entries_are_those_the_tests_read():
    """The generator's entry list and row count are the ones checked here and read by the GPU tests."""
    import importlib.util
    import os

    spec = importlib.util.spec_from_file_location(
        "make_full_size", os.path.join(parity.GOLDEN_DIR, "make_full_size.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    assert m.SPECS == SPECS and m.ROWS == ROWS
    assert all(m.seed_of(cfg, s) == _seed(cfg, s) for cfg in SPECS for s in (False, True))


@pytest.mark.parametrize("cfg", sorted(SPECS))
def test_rows_are_the_sampled_rows(cfg):
    wl = workloads.WORKLOADS[cfg]
    G = parity.load_golden(cfg)
    rows = G["rows"]
    np.testing.assert_array_equal(rows, wl.sample_rows(ROWS))
    assert len(rows) == ROWS and rows[0] == 0 and rows[-1] == wl.B - 1
    for op, T, sigma in SPECS[cfg]:
        key = parity.golden_key(op, T, sigma)
        names = ["w_soft", "log_z", "kappa_w_soft", "kappa_log_z"] if op == "soft" else \
            ["grad", "w_soft", "kappa_grad", "kappa_grad_norm", "kappa_w_soft", "grad_floor"]
        for name in names:
            assert key + "/" + name in G
            assert np.all(np.isfinite(G[key + "/" + name]))


def _recompute(oracle_mod, wl, G, w, c, g, sig, op, T, sigma, pick):
    """The stored names of one entry, recomputed by the oracle for the sampled rows at positions `pick`."""
    rows = G["rows"]
    key = parity.golden_key(op, T, sigma)
    s = sig[rows] if sigma else None
    if op == "soft":
        ws, lz, k_ws, k_lz = parity.soft_reference(oracle_mod, w[rows], c, wl.L, wl.k, T, sigma=s,
                                                   seed=_seed(wl.cfg, sigma), rows=pick)
        return {"w_soft": ws, "log_z": lz, "kappa_w_soft": k_ws, "kappa_log_z": k_lz}
    floor = float(G[key + "/grad_floor"])
    assert floor == parity.grad_floor(G[key + "/grad"], g[rows], c, T)
    gr, ws, k_g, k_n, k_ws = parity.grad_reference(oracle_mod, w[rows], c, g[rows], wl.L, wl.k, T, sigma=s,
                                                   seed=_seed(wl.cfg, sigma), rows=pick, floor=floor)
    return {"grad": gr, "w_soft": ws, "kappa_grad": k_g, "kappa_grad_norm": k_n, "kappa_w_soft": k_ws}


@pytest.mark.slow
@pytest.mark.parametrize("cfg", sorted(SPECS))
def test_first_and_last_rows_recomputed_by_the_oracle(oracle_mod, cfg):
    """Row 0 of every other entry and row B - 1 of the rest, answers and kappas, exactly as stored.  The entries run
    in parallel threads (each oracle call releases the interpreter while it computes)."""
    import concurrent.futures

    wl = workloads.WORKLOADS[cfg]
    G = parity.load_golden(cfg)
    w, c, g, sig = wl.weights(), wl.codebook(), wl.upstream_grad(), wl.boundary_states()
    specs = SPECS[cfg]
    picks = [np.array([0 if i % 2 == 0 else ROWS - 1]) for i in range(len(specs))]
    with concurrent.futures.ThreadPoolExecutor(len(specs)) as ex:
        futs = [ex.submit(_recompute, oracle_mod, wl, G, w, c, g, sig, op, T, sigma, pick)
                for (op, T, sigma), pick in zip(specs, picks)]
        results = [f.result() for f in futs]
    for (op, T, sigma), pick, got in zip(specs, picks, results):
        key = parity.golden_key(op, T, sigma)
        for name, val in got.items():
            np.testing.assert_array_equal(np.asarray(val), G[key + "/" + name][pick], err_msg=f"{key}/{name}")
