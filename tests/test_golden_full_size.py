"""The stored full-size references (tests/golden/full_size_cfg<N>.npz) are the oracle's, on the CPU.

Each file holds, for 64 sampled rows of a full-size workload, the oracle's answers and each row's random one-ulp
kappas, and for rows 0 and B - 1 the first-order kappas, written by tests/golden/make_full_size.py.  Here row 0 or row
B - 1 of every entry (the first and last rows of the matrix, both always sampled) is recomputed with the oracle and
must match the stored answers and random kappas exactly, recomputed from the same seeded one-ulp draws (the oracle
treats every sequence on its own, so a row's values do not depend on the other rows computed with it).  The
first-order kappas take about N oracle passes per entry and are not recomputed here.  The GPU tests compare the GPU
path with these rows.
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
    m = _generator()
    assert m.SPECS == SPECS and m.ROWS == ROWS and m.FO_POS == [0, ROWS - 1]
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
        names = ["w_soft", "log_z", "kappa_w_soft", "kappa_w_soft_norm", "kappa_log_z", "fo_kappa_w_soft"] \
            if op == "soft" else ["grad", "w_soft", "kappa_grad", "kappa_grad_norm", "kappa_w_soft", "grad_floor",
                                  "fo_kappa_grad", "fo_kappa_grad_norm", "fo_kappa_w_soft"]
        for name in names:
            assert key + "/" + name in G
            assert np.all(np.isfinite(G[key + "/" + name]))
            if name.startswith("fo_"):
                assert G[key + "/" + name].shape == (2,)


def _generator():
    import importlib.util
    import os

    spec = importlib.util.spec_from_file_location(
        "make_full_size", os.path.join(parity.GOLDEN_DIR, "make_full_size.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


@pytest.mark.slow
@pytest.mark.parametrize("cfg", sorted(SPECS))
def test_first_and_last_rows_recomputed_by_the_oracle(oracle_mod, cfg):
    """Row 0 of every other entry and row B - 1 of the rest, answers and random kappas, exactly as stored.  The
    entries run one after another; each one's oracle calls run in parallel threads."""
    m = _generator()
    wl = workloads.WORKLOADS[cfg]
    G = parity.load_golden(cfg)
    rows = G["rows"]
    w, c, g, sig = wl.weights(), wl.codebook(), wl.upstream_grad(), wl.boundary_states()
    for i, (op, T, sigma) in enumerate(SPECS[cfg]):
        key = parity.golden_key(op, T, sigma)
        pick = np.array([0 if i % 2 == 0 else ROWS - 1])
        floor = None if op == "soft" else float(G[key + "/grad_floor"])
        got = m.reference(wl, rows[pick], w, c, g, sig, op, T, sigma, floor=floor)
        for name, val in got.items():
            stored = G[key + "/" + name]
            np.testing.assert_array_equal(np.asarray(val), stored if name == "grad_floor" else stored[pick],
                                          err_msg=f"{key}/{name}")
