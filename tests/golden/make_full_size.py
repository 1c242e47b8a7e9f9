"""Writes the oracle's answers on 64 sampled rows of each full-size workload, with their one-ulp conditioning.

    python tests/golden/make_full_size.py            # every workload (about an hour on 8 cores)
    python tests/golden/make_full_size.py 2 4        # only these config indices

Output: tests/golden/full_size_cfg<N>.npz, read by the GPU parity tests, which run the full batch on the GPU in the
launch configuration the benchmark times and compare these rows.  Only the CPU oracle and the seeded input generators
are called here.  The rows are workloads.sample_rows(64) (rows 0 and B - 1 always among them, first and last).  Each
entry holds the oracle's float64 answers for those rows at the float32 temperature the C-ABI receives, and kappa
(tests/parity.py):
  * for all 64 rows, the random estimate: the largest change of the row's answer (in each of the tests' error
    measures) over 4 seeded moves of every float32 input by one ulp;
  * for rows 0 and B - 1 ("fo_" names), the first-order worst case: one oracle pass per input column (about 770
    passes for a gradient entry), which is why it is taken on two rows only and stored.
tests/test_golden_full_size.py recomputes rows 0 and B - 1 and their random kappas on the CPU to pin the stored
values to the oracle.
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
for p in (ROOT, os.path.dirname(HERE)):
    if p not in sys.path:
        sys.path.insert(0, p)

import oracle  # noqa: E402
import parity  # noqa: E402
import workloads  # noqa: E402

ROWS = 64

# (op, T, sigma mode) per config: what the full-size GPU tests compare
SPECS = {
    2: [("soft", 1.0, False), ("soft", 0.1, False), ("soft", 0.01, False), ("grad", 0.1, False)],
    3: [("grad", 0.05, False)],
    4: [("soft", 0.1, False), ("soft", 0.01, False), ("soft", 1e-3, False), ("soft", 1e-4, False),
        ("soft", 0.1, True), ("soft", 0.01, True), ("grad", 0.1, True)],
    5: [("grad", 0.05, False)],
}


key = parity.golden_key
path = parity.golden_path


FO_POS = [0, ROWS - 1]   # positions in the sample of rows 0 and B - 1


def reference(wl, sel, w, c, g, sig, op, T, sigma, floor=None):
    """The oracle's answers on the rows ``sel`` at the float32 T and their random kappas (the one-ulp moves are drawn
    for the whole matrix, so a row's values do not depend on which other rows are computed).  ``floor``: the
    gradient measures' floor, by default that of these rows' exact gradient."""
    s = sig[sel] if sigma else None
    seed = seed_of(wl.cfg, sigma)
    T = parity.t32(T)
    if op == "soft":
        (ws, lz), (k_ws, k_nw, k_lz) = parity.one_ulp_conditioning(
            lambda w_, c_, g_, T_: oracle.soft(w_, c_, wl.L, wl.k, T_, sigma=s), w, c,
            [(0, parity.rel_rows), (0, parity.rel_norm_rows), (1, parity.lz_rows)], seed=seed, rows=sel, T=T)
        return {"w_soft": ws, "log_z": lz, "kappa_w_soft": k_ws, "kappa_w_soft_norm": k_nw, "kappa_log_z": k_lz}
    gs = g[sel]
    fl = {} if floor is None else {"v": floor}

    def floor_of(r):
        if "v" not in fl:
            fl["v"] = parity.grad_floor(r, gs, c, T)
        return fl["v"]

    (gr, ws), (k_g, k_n, k_ws) = parity.one_ulp_conditioning(
        lambda w_, c_, g_, T_: oracle.grad(w_, c_, g_, wl.L, wl.k, T_, sigma=s), w, c,
        [(0, lambda x, r: parity.grad_rows(x, r, gs, c, T, floor_of(r))),
         (0, lambda x, r: parity.grad_norm_rows(x, r, gs, c, T, floor_of(r))), (1, parity.rel_rows)],
        seed=seed, rows=sel, g=g, T=T)
    return {"grad": gr, "w_soft": ws, "kappa_grad": k_g, "kappa_grad_norm": k_n, "kappa_w_soft": k_ws,
            "grad_floor": np.array(floor_of(gr))}


def entry(wl, rows, w, c, g, sig, op, T, sigma):
    """The arrays of one entry: reference() on the 64 rows, and the first-order kappas of rows 0 and B - 1."""
    out = reference(wl, rows, w, c, g, sig, op, T, sigma)
    T = parity.t32(T)
    fo = rows[FO_POS]
    s_fo = sig[fo] if sigma else None
    if op == "soft":
        K = parity.soft_first_order(oracle, w[fo], c, wl.L, wl.k, T, sigma=s_fo)
        out["fo_kappa_w_soft"] = parity._k_rel_rows(K, out["w_soft"][FO_POS])
        return out
    floor = float(out["grad_floor"])
    Kg, Kw, _ = parity.grad_first_order(oracle, w[fo], c, g[fo], wl.L, wl.k, T, sigma=s_fo)
    out["fo_kappa_grad"] = parity._k_grad_rows(Kg, out["grad"][FO_POS], floor)
    out["fo_kappa_grad_norm"] = parity._k_grad_norm_rows(Kg, out["grad"][FO_POS], floor)
    out["fo_kappa_w_soft"] = parity._k_rel_rows(Kw, out["w_soft"][FO_POS])
    return out


def seed_of(cfg: int, sigma: bool) -> int:
    """Seed of the one-ulp draws of an entry."""
    return 7000 + 10 * cfg + int(sigma)


def make(cfg: int) -> None:
    wl = workloads.WORKLOADS[cfg]
    rows = wl.sample_rows(ROWS)
    w, c, g, sig = wl.weights(), wl.codebook(), wl.upstream_grad(), wl.boundary_states()
    out = {"rows": rows}
    for op, T, sigma in SPECS[cfg]:
        t0 = time.time()
        for name, arr in entry(wl, rows, w, c, g, sig, op, T, sigma).items():
            out[f"{key(op, T, sigma)}/{name}"] = arr
        kap = {k.split("/")[-1]: float(np.max(v)) for k, v in out.items()
               if k.startswith(key(op, T, sigma) + "/kappa") or k.startswith(key(op, T, sigma) + "/fo_kappa")}
        print(f"cfg {cfg} {key(op, T, sigma)}: largest kappas {kap} ({time.time() - t0:.0f} s)", flush=True)
    np.savez(path(cfg), **out)


if __name__ == "__main__":
    oracle.build(force=False)
    cfgs = [int(a) for a in sys.argv[1:]] or sorted(SPECS)
    for cfg in cfgs:
        make(cfg)
