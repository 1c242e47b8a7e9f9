"""Writes the oracle's answers on 64 sampled rows of each full-size workload, with their one-ulp conditioning.

    python tests/golden/make_full_size.py            # every workload (about half an hour on 8 cores)
    python tests/golden/make_full_size.py 2 4        # only these config indices

Output: tests/golden/full_size_cfg<N>.npz, read by the GPU parity tests, which run the full batch on the GPU in the
launch configuration the benchmark times and compare these rows.  Only the CPU oracle and the seeded input generators
are called here.  The rows are workloads.sample_rows(64) (rows 0 and B - 1 always among them).  Each entry holds the
oracle's float64 answers for those rows and, per row, kappa: the largest change of the row's answer (in the test's
error measure) when every float32 weight and codebook value moves by one float32 ulp, over 4 seeded draws
(tests/parity.py).
Computing kappa this way at L = 16 costs about five oracle passes per entry, which is why it is stored rather than
recomputed on every GPU run; tests/test_golden_full_size.py recomputes sampled rows and one whole entry on the CPU
to pin the stored values to the oracle.
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


def entry(wl, rows, w, c, g, sig, op, T, sigma):
    """The arrays of one entry: the oracle's answers on the rows and their per-row kappas (and, for the gradient,
    the floor of its error measures, from these rows' exact gradient)."""
    s = sig[rows] if sigma else None
    seed = seed_of(wl.cfg, sigma)
    if op == "soft":
        ws, lz, k_ws, k_lz = parity.soft_reference(oracle, w[rows], c, wl.L, wl.k, T, sigma=s, seed=seed)
        return {"w_soft": ws, "log_z": lz, "kappa_w_soft": k_ws, "kappa_log_z": k_lz}
    gr, ws, k_g, k_n, k_ws = parity.grad_reference(oracle, w[rows], c, g[rows], wl.L, wl.k, T, sigma=s, seed=seed)
    return {"grad": gr, "w_soft": ws, "kappa_grad": k_g, "kappa_grad_norm": k_n, "kappa_w_soft": k_ws,
            "grad_floor": np.array(parity.grad_floor(gr, g[rows], c, T))}


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
        kap = {k.split("/")[-1]: float(np.max(v)) for k, v in out.items() if k.startswith(key(op, T, sigma) + "/kappa")}
        print(f"cfg {cfg} {key(op, T, sigma)}: largest kappas {kap} ({time.time() - t0:.0f} s)", flush=True)
    np.savez(path(cfg), **out)


if __name__ == "__main__":
    oracle.build(force=False)
    cfgs = [int(a) for a in sys.argv[1:]] or sorted(SPECS)
    for cfg in cfgs:
        make(cfg)
