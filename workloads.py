"""Seeded synthetic inputs for the BCJR soft quantizer.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic, so both the CPU oracle's tests and the GPU path can take
their inputs from it without sharing any computation.

Every array is drawn in float64 with NumPy's PCG64 generator and cast to
float32 (int32 for boundary states), so the GPU and the oracle see the same
values.  Seeds follow one rule per config index ``cfg``: codebook 1000+cfg,
weights 2000+cfg, upstream gradient 3000+cfg, sampled rows 4000+cfg,
boundary states 5000+cfg.

The workloads stand in for the weight matrices the pages quantize (Llama-3.2-1B
projections at 2 bits per weight, BCJR-QAT abstract): the real weights are not
available, so i.i.d. N(0,1) matrices of the same shapes are used, cut row-major
into sequences of n = 256 weights, one trellis sequence each.
"""
from __future__ import annotations

import dataclasses

import numpy as np

SEQ_LEN = 256

# Llama-3.2-1B decoder projection shapes (rows x cols), used by the
# whole-layer workload: q, o, k, v, gate, up, down.
LLAMA32_1B_PROJECTIONS = (
    ("q_proj", 2048, 2048),
    ("o_proj", 2048, 2048),
    ("k_proj", 512, 2048),
    ("v_proj", 512, 2048),
    ("gate_proj", 8192, 2048),
    ("up_proj", 8192, 2048),
    ("down_proj", 2048, 8192),
)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def codebook(L: int, seed: int, unit_variance: bool = True) -> np.ndarray:
    """2^L codebook entries ~ N(0,1); scaled by 1/std (ddof=0, not centred)."""
    z = _rng(seed).standard_normal(1 << L)
    if unit_variance:
        z = z / z.std()
    return z.astype(np.float32)


def codebook_v(L: int, V: int, seed: int) -> np.ndarray:
    """A codebook of V-vectors: [2^L, V] entries ~ N(0,1), scaled by 1/std over all entries (ddof=0, not centred).
    V = 1 gives codebook(L, seed) as a column."""
    z = _rng(seed).standard_normal((1 << L, V))
    return (z / z.std()).astype(np.float32)


def weights(B: int, n: int, seed: int) -> np.ndarray:
    """B sequences of n weights ~ N(0,1), float32, row-major [B, n]."""
    return _rng(seed).standard_normal((B, n)).astype(np.float32)


def upstream_grad(B: int, n: int, seed: int) -> np.ndarray:
    """Upstream dL/dw_soft ~ N(0,1), float32 [B, n]."""
    return _rng(seed).standard_normal((B, n)).astype(np.float32)


def boundary_states(B: int, L: int, seed: int) -> np.ndarray:
    """Per-sequence boundary state sigma, uniform on [0, 2^L), int32 [B]."""
    return _rng(seed).integers(0, 1 << L, size=B).astype(np.int32)


def sample_rows(B: int, count: int, seed: int) -> np.ndarray:
    """Sorted distinct row indices that always include row 0 and row B-1."""
    if count >= B:
        return np.arange(B, dtype=np.int64)
    rest = _rng(seed).choice(np.arange(1, B - 1), size=max(count - 2, 0), replace=False)
    return np.unique(np.concatenate([[0, B - 1], rest])).astype(np.int64)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, trellis parameters and temperatures."""

    cfg: int
    name: str
    L: int
    k: int
    B: int
    n: int
    temps: tuple
    matrix: str
    V: int = 1   # weights per trellis step; n counts weights, so a sequence has n / V steps

    @property
    def steps(self) -> int:
        return self.n // self.V

    def codebook(self) -> np.ndarray:
        """[2^L] for V = 1, else [2^L, V]."""
        if self.V == 1:
            return codebook(self.L, 1000 + self.cfg)
        return codebook_v(self.L, self.V, 1000 + self.cfg)

    def weights(self, B: int | None = None) -> np.ndarray:
        return weights(self.B if B is None else B, self.n, 2000 + self.cfg)

    def upstream_grad(self, B: int | None = None) -> np.ndarray:
        return upstream_grad(self.B if B is None else B, self.n, 3000 + self.cfg)

    def boundary_states(self, B: int | None = None) -> np.ndarray:
        return boundary_states(self.B if B is None else B, self.L, 5000 + self.cfg)

    def sample_rows(self, count: int) -> np.ndarray:
        return sample_rows(self.B, count, 4000 + self.cfg)


def _layer_sequences() -> int:
    return sum(r * c for _, r, c in LLAMA32_1B_PROJECTIONS) // SEQ_LEN


WORKLOADS = {
    1: Workload(1, "tiny_L8", 8, 2, 16, 64, (1.0, 0.1, 0.01), "16x64"),
    2: Workload(2, "qtip_1024x1024", 16, 2, 4096, SEQ_LEN, (1.0, 0.1, 0.01), "1024x1024"),
    3: Workload(3, "llama_mlp_8192x2048", 16, 2, 65536, SEQ_LEN, (0.05,), "8192x2048"),
    4: Workload(4, "low_temp_2048x2048", 16, 2, 16384, SEQ_LEN, (1e-1, 1e-2, 1e-3, 1e-4), "2048x2048"),
    5: Workload(5, "llama_layer_all_proj", 16, 2, _layer_sequences(), SEQ_LEN, (0.05,), "q,o,k,v,gate,up,down"),
}

# Trellis variants of the 1024x1024 workload (the same weights and upstream gradient): 3 bits per weight (k = 3), and
# 2 bits per weight with two weights per step (k = 4, V = 2).  The pages fix neither k nor V.
TRELLIS_VARIANTS = {
    "k3": Workload(2, "qtip_1024x1024_k3", 16, 3, 4096, SEQ_LEN, (0.1,), "1024x1024"),
    "k4v2": Workload(2, "qtip_1024x1024_k4_v2", 16, 4, 4096, SEQ_LEN, (0.1,), "1024x1024", V=2),
}

# The brute-force companion of the tiny workload: L=4, k=2, n=6, 16 sequences.
TINY_BRUTE = Workload(1, "tiny_L4_brute", 4, 2, 16, 6, (1.0, 0.1, 0.01), "16x6")
