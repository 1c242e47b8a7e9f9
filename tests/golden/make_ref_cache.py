"""Store the one-ulp kappas of the oracle's references for the GPU tests' own inputs: python
tests/golden/make_ref_cache.py [--check N].

Each entry is what tests/parity.py's soft_kappas, grad_kappas, codebook_grad_kappas or tail_biting_kappas returns for
one call (the conditioning that soft_reference, grad_reference, codebook_grad_reference and tail_biting_reference
attach to the oracle's answers, which the tests compute on the spot), computed here on the CPU by the oracle alone,
under the digest of the call (function, every input array's bytes, the scalar arguments, the oracle's source,
parity.REF_VERSION).  The calls
below are the ones the slowest GPU tests make (the checkpoint-mode, tail-biting-measure and general-trellis parity
tests, the k = 2 batch edges and the headline codebook-gradient rows), with the inputs built by tests/cases.py and
workloads.py exactly as the tests build them.  A GPU test whose call has no entry computes it on the spot.  With
--check N, N entries taken at random are recomputed and must match what is stored."""
from __future__ import annotations

import argparse
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
TESTS = os.path.dirname(HERE)
ROOT = os.path.dirname(TESTS)
for p in (ROOT, TESTS):
    if p not in sys.path:
        sys.path.insert(0, p)

import numpy as np  # noqa: E402

import cases  # noqa: E402
import oracle  # noqa: E402
import parity  # noqa: E402
import workloads  # noqa: E402


def plan():
    """(kappa function, positional arguments after the oracle, keyword arguments) of every stored call."""
    calls = []
    soft, grad, gcr, tbr = (parity.soft_kappas, parity.grad_kappas, parity.codebook_grad_kappas,
                            parity.tail_biting_kappas)

    def sig_case(L, k, V, B, n, sigma, base):
        if sigma:
            n = cases.sigma_n(L, k, n)
        return cases.vin(L, V, B, n, base + 31 * L + 7 * k + V + n, sigma)

    # checkpoint-and-recompute mode (tests/test_gpu_checkpoint.py)
    for L, k, V, B, n in cases.CHECKPOINT:
        for sigma in (False, True):
            w, c, _, s = sig_case(L, k, V, B, n, sigma, 6100)
            calls += [(soft, (w, c, L, k, T), {"sigma": s}) for T in (1.0, 0.1, 0.05)]
            w, c, g, s = sig_case(L, k, V, B, n, sigma, 6400)
            calls += [(grad, (w, c, g, L, k, T), {"sigma": s}) for T in (1.0, 0.1, 0.05)]
            w, c, g, s = sig_case(L, k, V, B, n, sigma, 6500)
            calls += [(gcr, (w, c, g, L, k, T), {"sigma": s}) for T in (1.0, 0.1)]
    for L, k, V, B, n in cases.CHECKPOINT_SOFT_SEVERAL:
        w, c, _, _ = cases.vin(L, V, B, n, 6200 + L)
        calls.append((soft, (w, c, L, k, 0.1), {"sigma": None}))
    for L, k, V, B, n in cases.CHECKPOINT_GRAD_SEVERAL:
        w, c, g, _ = cases.vin(L, V, B, n, 6600 + L + k)
        calls += [(grad, (w, c, g, L, k, 0.1), {"sigma": None}), (gcr, (w, c, g, L, k, 0.1), {"sigma": None})]

    # tail-biting measure (tests/test_gpu_tail_biting.py, tests/test_gpu_tail_biting_general.py)
    for L, B, n in cases.TAIL_BITING_MEASURE:
        w, c, g, _ = cases.inputs(L, B, n, 1400 + 7 * L + n)
        calls += [(tbr, (w, c, g, L, 2, T), {}) for T in (1.0, 0.1, 0.05)]
    for L, k, V, B, n in cases.TAIL_BITING_MEASURE_GENERAL:
        w, c, g, _ = cases.vin(L, V, B, n, 2400 + 31 * L + 7 * k + V + n)
        calls += [(tbr, (w, c, g, L, k, T), {}) for T in (1.0, 0.1)]

    # general trellis (tests/test_gpu_general_trellis.py)
    for L, k, V, B, n in cases.GENERAL:
        for sigma in (False, True):
            w, c, _, s = sig_case(L, k, V, B, n, sigma, 7000)
            calls += [(soft, (w, c, L, k, T), {"sigma": s}) for T in (1.0, 0.1, 0.05)]
            w, c, g, s = sig_case(L, k, V, B, n, sigma, 7100)
            calls += [(grad, (w, c, g, L, k, T), {"sigma": s}) for T in (1.0, 0.1, 0.05)]
            w, c, g, s = sig_case(L, k, V, B, n, sigma, 7700)
            calls += [(gcr, (w, c, g, L, k, T), {"sigma": s}) for T in (1.0, 0.1, 0.05)]
    for V in (1, 2):
        w, c, g, _ = cases.vin(16, V, 2, 7, 7090 + V)
        calls += [(grad, (w, c, g, 16, 1, 0.3), {"sigma": None}), (gcr, (w, c, g, 16, 1, 0.3), {"sigma": None})]
    for L, k, V, B, n in cases.GENERAL_SEVERAL:
        w, c, g, _ = cases.vin(L, V, B, n, 7300 + L + k + V)
        calls += [(soft, (w, c, L, k, 0.1), {"sigma": None}), (grad, (w, c, g, L, k, 0.1), {"sigma": None})]
    for L, k, V, B, n in cases.GENERAL_GC_SEVERAL:
        w, c, g, _ = cases.vin(L, V, B, n, 8100 + L + k)
        calls.append((gcr, (w, c, g, L, k, 0.2), {"sigma": None}))
    for L, k, V in cases.GENERAL_LONGEST:
        w, c, g, _ = cases.vin(L, V, 2, 4096, 8200 + L)
        calls += [(soft, (w, c, L, k, 0.3), {"sigma": None}), (grad, (w, c, g, L, k, 0.3), {"sigma": None})]
    for wl in workloads.TRELLIS_VARIANTS.values():
        c, w, g = wl.codebook(), wl.weights(), wl.upstream_grad()
        T = wl.temps[0]
        rows = wl.sample_rows(3)
        calls += [(soft, (w[rows], c, wl.L, wl.k, T), {"sigma": None}),
                  (grad, (w[rows], c, g[rows], wl.L, wl.k, T), {"sigma": None}),
                  (gcr, (w[rows], c, g[rows], wl.L, wl.k, T), {"sigma": None})]

    # k = 2 batch edges (tests/test_gpu_parity.py) and the headline codebook-gradient rows
    # (tests/test_gpu_codebook_grad.py)
    for L, B, n, rows in cases.BATCH_EDGES:
        w, c, g, _ = cases.inputs(L, B, n, 900 + L)
        rows = np.asarray(rows)
        calls += [(soft, (w[rows], c, L, 2, 0.1), {}), (grad, (w[rows], c, g[rows], L, 2, 0.1), {"sigma": None})]
    wl = workloads.WORKLOADS[2]
    c, w, g = wl.codebook(), wl.weights(), wl.upstream_grad()
    rows = wl.sample_rows(2)
    calls += [(gcr, (w[rows], c, g[rows], wl.L, wl.k, T), {"sigma": None}) for T in (0.1, 1.0)]
    return calls


def key_of(fn, args, kwargs):
    import inspect

    bound = inspect.signature(fn.uncached).bind(None, *args, **kwargs)
    bound.apply_defaults()
    return parity.ref_key(fn.__name__, {k: v for k, v in bound.arguments.items() if k != "oracle"})


def _same(a, b) -> bool:
    if isinstance(a, (tuple, list)):
        return len(a) == len(b) and all(_same(x, y) for x, y in zip(a, b))
    return np.array_equal(np.asarray(a), np.asarray(b), equal_nan=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--check", type=int, default=0, help="recompute this many stored entries and compare")
    args = ap.parse_args()
    oracle.build(force=False)
    calls = plan()
    if args.check:
        rng = np.random.Generator(np.random.PCG64(1))
        for i in rng.choice(len(calls), size=min(args.check, len(calls)), replace=False):
            fn, a, kw = calls[i]
            stored = parity.load_ref(key_of(fn, a, kw))
            assert stored is not None, f"entry {i} ({fn.__name__}) is not stored"
            assert _same(fn.uncached(oracle, *a, **kw), stored), f"entry {i} ({fn.__name__}) differs"
        print(f"{args.check} stored entries recomputed: identical")
        return
    done = 0
    for fn, a, kw in calls:
        key = key_of(fn, a, kw)
        if parity.load_ref(key) is None:
            parity.store_ref(key, fn.uncached(oracle, *a, **kw))
        done += 1
        if done % 20 == 0:
            print(f"{done}/{len(calls)}", flush=True)
    keep = {key_of(fn, a, kw) + ".npz" for fn, a, kw in calls}
    for f in os.listdir(parity.REF_CACHE_DIR):
        if f not in keep:
            os.remove(os.path.join(parity.REF_CACHE_DIR, f))
    print(f"{len(calls)} references stored in {parity.REF_CACHE_DIR}")


if __name__ == "__main__":
    main()
