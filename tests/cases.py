"""Seeded inputs and case lists of the GPU tests, on the CPU only (numpy; no method arithmetic, no GPU code).

The GPU tests build their inputs here, and tests/golden/make_ref_cache.py builds the same inputs to store the oracle's
references for them ahead of time (tests/parity.py: stored references)."""
import numpy as np


def inputs(L, B, n, seed, sigma=False):
    """k = 2, V = 1 inputs: codebook [2^L] (unit variance), weights and upstream gradient [B, n], sigma [B]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    c = rng.standard_normal(1 << L)
    c = (c / c.std()).astype(np.float32)
    w = rng.standard_normal((B, n)).astype(np.float32)
    g = rng.standard_normal((B, n)).astype(np.float32)
    s = rng.integers(0, 1 << L, size=B).astype(np.int32) if sigma else None
    return w, c, g, s


def vin(L, V, B, n, seed, sigma=False):
    """Codebook ([2^L] for V = 1, else [2^L, V], unit variance), weights and upstream gradient [B, n V], sigma [B]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    c = rng.standard_normal((1 << L, V))
    c = (c / c.std()).astype(np.float32)
    if V == 1:
        c = c[:, 0].copy()
    w = rng.standard_normal((B, n * V)).astype(np.float32)
    g = rng.standard_normal((B, n * V)).astype(np.float32)
    s = rng.integers(0, 1 << L, size=B).astype(np.int32) if sigma else None
    return w, c, g, s


def sigma_n(L, k, n):
    """Enough steps for every sigma to be reachable: the constraint needs at least L/k steps."""
    return max(n, -(-L // k) + 1)


def ids(cases):
    return [f"L{c[0]}k{c[1]}V{c[2]}B{c[3]}n{c[4]}" for c in cases]


# general trellis (L, k, V, B, n steps)
GENERAL = [(4, 1, 1, 16, 6), (4, 1, 2, 7, 5), (5, 1, 1, 5, 8), (5, 2, 2, 9, 9), (6, 3, 1, 5, 4), (6, 3, 2, 3, 7),
           (7, 3, 1, 4, 9), (8, 1, 1, 6, 33), (8, 4, 1, 4, 5), (8, 4, 2, 3, 6), (9, 1, 2, 5, 17), (9, 3, 2, 4, 12),
           (10, 4, 1, 3, 10), (11, 1, 1, 2, 20), (12, 3, 1, 2, 16), (12, 4, 2, 2, 9), (13, 1, 2, 2, 7),
           (14, 3, 2, 2, 6), (15, 1, 1, 2, 6), (16, 1, 1, 2, 4), (16, 1, 2, 1, 4), (16, 2, 2, 2, 5), (16, 3, 1, 2, 5),
           (16, 3, 2, 2, 4), (16, 4, 1, 2, 4), (16, 4, 2, 2, 5)]
GENERAL_SEVERAL = [(8, 1, 2, 4600, 5), (9, 3, 1, 4200, 4), (16, 3, 1, 260, 3), (16, 4, 2, 258, 3), (16, 1, 1, 260, 3),
                   (16, 1, 2, 258, 3)]
GENERAL_GC_SEVERAL = [(9, 3, 2, 4200, 3), (8, 1, 1, 4400, 4), (16, 4, 2, 300, 2), (16, 1, 1, 260, 3),
                      (16, 1, 2, 258, 3)]
GENERAL_LONGEST = [(10, 3, 2), (8, 1, 1), (12, 4, 1)]

# checkpoint-and-recompute mode (L, k, V, B, n steps)
CHECKPOINT = [(8, 2, 1, 5, 37), (8, 2, 1, 4, 40), (9, 3, 2, 3, 50), (6, 3, 1, 4, 1), (8, 1, 2, 4, 2),
              (12, 1, 1, 3, 100), (13, 4, 1, 2, 26), (16, 2, 1, 2, 40), (16, 3, 1, 2, 33), (16, 4, 2, 2, 20),
              (16, 1, 1, 1, 17)]
CHECKPOINT_SOFT_SEVERAL = [(8, 3, 2, 4300, 9), (16, 2, 1, 270, 5)]
CHECKPOINT_GRAD_SEVERAL = [(8, 3, 2, 4300, 9), (16, 2, 1, 270, 5), (8, 1, 1, 4200, 10)]

# tail-biting measure: k = 2 (L, B, n) and the general trellis (L, k, V, B, n)
TAIL_BITING_MEASURE = [(4, 16, 6), (4, 37, 5), (5, 9, 1), (6, 5, 2), (6, 7, 33), (8, 16, 64), (9, 5, 17), (10, 3, 40)]
TAIL_BITING_MEASURE_GENERAL = [(4, 1, 1, 9, 6), (4, 1, 2, 5, 5), (6, 3, 1, 5, 2), (6, 3, 2, 4, 9), (8, 4, 1, 3, 2),
                               (8, 4, 2, 3, 12), (8, 2, 2, 4, 10), (9, 1, 2, 2, 13), (10, 3, 1, 2, 24),
                               (10, 4, 2, 2, 16)]

# batch edges of the k = 2 kernels: (L, B, n, sampled rows)
BATCH_EDGES = [
    (16, 1, 64, [0]),                    # one sequence on the 2^16-state trellis
    (16, 260, 8, [0, 3, 255, 256, 259]),  # blocks 0..3 take a second sequence (grid = 256)
    (8, 8200, 4, [0, 8191, 8192, 8199]),  # 4 sequences per block, 2048 blocks: rows past 8191 come back round
    (4, 65, 5, [0, 63, 64]),              # 64 sequences per block: the second block has one active sequence
]
