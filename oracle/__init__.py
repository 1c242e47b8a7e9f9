"""CPU oracle for the temperature-T BCJR soft quantizer (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It loads ``liboracle.so``, built from
``oracle.c`` with gcc (``-O2``, no fast-math, no FMA contraction, OpenMP over
sequences), and shares no code with the GPU path.

What the oracle computes follows "BCJR-QAT: A Differentiable Relaxation of
Trellis-Coded Weight Quantization" (arXiv 2605.10655): the Boltzmann path
measure at temperature T, the soft codeword as the expectation of c(s_t)
(gist.science Technical Summary, "Core Mechanism"), its exact gradient in the
weights, and the Viterbi hard code as the T -> 0 limit (abstract).  The
readings the pages leave open are stated in ``oracle.c``'s header.

Shapes: a codebook of shape [2^L] is the scalar trellis (V = 1); one of shape
[2^L, V] emits V weights per trellis step.  Weights are [B, N] with N = n V:
step t of a row owns its weights t V .. t V + V - 1.  Soft codewords and
gradients have the weights' shape; Viterbi states are [B, n], one per step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
             "-fexcess-precision=standard"]


# Host sanitizers (AddressSanitizer and UndefinedBehaviorSanitizer): a separate build for test sessions run with
# gcc's libasan preloaded; any finding aborts the process.
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc; returns its path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(path: str) -> str:
    """Compile oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer into `path` (use with
    LD_PRELOAD=$(gcc -print-file-name=libasan.so) and ORACLE_LIB=path); returns path."""
    subprocess.check_call(["gcc", *GCC_FLAGS, *SANITIZE_FLAGS, "-o", path, _SRC, "-lm"])
    return path


class _Handle:
    """ctypes handle on one build of the oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        i32p = ctypes.POINTER(ctypes.c_int32)
        i64 = ctypes.c_int64
        ci = ctypes.c_int
        lib.oracle_soft.argtypes = [f32p, f32p, i64, i64, ci, ci, ci, ctypes.c_double, i32p, f64p, f64p, f64p]
        lib.oracle_soft.restype = ci
        lib.oracle_grad.argtypes = [f32p, f32p, f32p, i64, i64, ci, ci, ci, ctypes.c_double, i32p, f64p, f64p]
        lib.oracle_grad.restype = ci
        lib.oracle_grad_codebook.argtypes = [f32p, f32p, f32p, i64, i64, ci, ci, ci, ctypes.c_double, i32p, f64p,
                                             f64p, f64p]
        lib.oracle_grad_codebook.restype = ci
        lib.oracle_viterbi.argtypes = [f32p, f32p, i64, i64, ci, ci, ci, i32p, i32p, f32p, f32p]
        lib.oracle_viterbi.restype = ci
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ci
        self.lib = lib


_handle = None


def _load():
    global _handle
    if _handle is None:
        build(force=False)
        _handle = _Handle(_LIB)
    return _handle.lib


def use_library(path: str) -> None:
    """Point this module at another build of oracle.c (the mutation tests plant mistakes in copies)."""
    global _handle
    _handle = _Handle(path)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a, ctype):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctype))


def _check_shapes(w, c, L):
    """(B, n steps, V) from w [B, n V] and c [2^L] (V = 1) or [2^L, V]."""
    if w.ndim != 2:
        raise ValueError("w must be [B, N]")
    if c.ndim not in (1, 2) or c.shape[0] != 1 << L:
        raise ValueError(f"codebook must be [2^L] or [2^L, V] with 2^L = {1 << L}")
    V = 1 if c.ndim == 1 else c.shape[1]
    if V < 1 or w.shape[1] % V:
        raise ValueError("the weights per row must be a multiple of V")
    return w.shape[0], w.shape[1] // V, V


def soft(w, c, L: int, k: int, T: float, sigma=None, with_check: bool = False):
    """Soft codeword w_soft [B, n] (float64) and ln Z [B] for float32 inputs.

    With ``with_check`` also returns max_t |logsumexp_s(alpha_t + beta_t) - ln Z| per sequence.
    """
    w = _f32(w)
    c = _f32(c)
    B, n, V = _check_shapes(w, c, L)
    sg = None if sigma is None else np.ascontiguousarray(sigma, dtype=np.int32)
    out = np.empty(w.shape, np.float64)
    lz = np.empty(B, np.float64)
    dev = np.empty(B, np.float64)
    rc = _load().oracle_soft(_ptr(w, ctypes.c_float), _ptr(c, ctypes.c_float), B, n, L, k, V, float(T),
                             _ptr(sg, ctypes.c_int32), _ptr(out, ctypes.c_double), _ptr(lz, ctypes.c_double),
                             _ptr(dev, ctypes.c_double))
    if rc != 0:
        raise RuntimeError(f"oracle_soft failed ({rc})")
    return (out, lz, dev) if with_check else (out, lz)


def grad(w, c, g, L: int, k: int, T: float, sigma=None):
    """dL/dw [B, N] (float64) for upstream g = dL/dw_soft, plus w_soft [B, N]."""
    w = _f32(w)
    c = _f32(c)
    g = _f32(g)
    B, n, V = _check_shapes(w, c, L)
    if g.shape != w.shape:
        raise ValueError("g must match w")
    sg = None if sigma is None else np.ascontiguousarray(sigma, dtype=np.int32)
    out = np.empty(w.shape, np.float64)
    ws = np.empty(w.shape, np.float64)
    rc = _load().oracle_grad(_ptr(w, ctypes.c_float), _ptr(c, ctypes.c_float), _ptr(g, ctypes.c_float), B, n,
                             L, k, V, float(T), _ptr(sg, ctypes.c_int32), _ptr(out, ctypes.c_double),
                             _ptr(ws, ctypes.c_double))
    if rc != 0:
        raise RuntimeError(f"oracle_grad failed ({rc})")
    return out, ws


def grad_codebook(w, c, g, L: int, k: int, T: float, sigma=None, per_sequence: bool = False):
    """dL/dc (the codebook's shape) summed over the batch (float64), dL/dw [B, N] and w_soft [B, N], for upstream
    g = dL/dw_soft.

    With ``per_sequence`` the first result has a leading batch axis, one entry per sequence.  A sequence with no admissible path
    (sigma mode, n < L/k) has a NaN row, so the batch sum is NaN.
    """
    w = _f32(w)
    c = _f32(c)
    g = _f32(g)
    B, n, V = _check_shapes(w, c, L)
    if g.shape != w.shape:
        raise ValueError("g must match w")
    sg = None if sigma is None else np.ascontiguousarray(sigma, dtype=np.int32)
    gw = np.empty(w.shape, np.float64)
    ws = np.empty(w.shape, np.float64)
    gc = np.empty((B,) + c.shape, np.float64)
    rc = _load().oracle_grad_codebook(_ptr(w, ctypes.c_float), _ptr(c, ctypes.c_float), _ptr(g, ctypes.c_float), B,
                                      n, L, k, V, float(T), _ptr(sg, ctypes.c_int32), _ptr(gw, ctypes.c_double),
                                      _ptr(ws, ctypes.c_double), _ptr(gc, ctypes.c_double))
    if rc != 0:
        raise RuntimeError(f"oracle_grad_codebook failed ({rc})")
    return (gc if per_sequence else gc.sum(axis=0)), gw, ws


def viterbi(w, c, L: int, k: int, sigma=None):
    """Viterbi states [B, n] int32 (s_1..s_n, one per step), c(states) [B, N] float32 and path cost [B] float32."""
    w = _f32(w)
    c = _f32(c)
    B, n, V = _check_shapes(w, c, L)
    sg = None if sigma is None else np.ascontiguousarray(sigma, dtype=np.int32)
    st = np.empty((B, n), np.int32)
    wh = np.empty(w.shape, np.float32)
    cost = np.empty(B, np.float32)
    rc = _load().oracle_viterbi(_ptr(w, ctypes.c_float), _ptr(c, ctypes.c_float), B, n, L, k, V,
                                _ptr(sg, ctypes.c_int32), _ptr(st, ctypes.c_int32), _ptr(wh, ctypes.c_float),
                                _ptr(cost, ctypes.c_float))
    if rc != 0:
        raise RuntimeError(f"oracle_viterbi failed ({rc})")
    return st, wh, cost


TB_EXACT, TB_ROTATE = 0, 1


def viterbi_tail_biting(w, c, L: int, k: int, mode: int = TB_EXACT):
    """Tail-biting Viterbi with the start state chosen by the decoder: (states [B, n], c(states), cost [B], sigma [B]).

    A tail-biting path has s_0 = s_n (the non-emitting start equals the last emitting state).  Both modes end with a
    sigma-mode decode, so the result is a tail-biting path and its cost follows the fixed float32 order.
      TB_EXACT:  sigma = the smallest state whose sigma-mode cost is the minimum over all 2^L states.
      TB_ROTATE: decode the sequence rotated left by n // 2 trellis steps with a free boundary; sigma = the state of
                 that path at the original last step (rotated position n - 1 - n // 2), where the cycle closes.
    w is [B, n V] for a codebook [2^L, V] (n steps of V weights).  Composed from this module's Viterbi (its own pins
    cover it); the selection is a plain argmin.
    """
    w = _f32(w)
    c = _f32(c)
    B, n, V = _check_shapes(w, c, L)
    S = 1 << L
    if mode == TB_EXACT:
        reps = np.repeat(w, S, axis=0)
        sig_all = np.tile(np.arange(S, dtype=np.int32), B)
        _, _, costs = viterbi(reps, c, L, k, sigma=sig_all)
        costs = costs.reshape(B, S)
        sigma = np.argmin(costs, axis=1).astype(np.int32)   # first index attaining the minimum
    elif mode == TB_ROTATE:
        r = n // 2
        st, _, _ = viterbi(np.roll(w, -r * V, axis=1), c, L, k)
        sigma = st[:, n - 1 - r].astype(np.int32)
    else:
        raise ValueError("mode must be TB_EXACT or TB_ROTATE")
    st, wh, cost = viterbi(w, c, L, k, sigma=sigma)
    return st, wh, cost, sigma


def soft_tail_biting(w, c, L: int, k: int, T: float):
    """Soft codeword [B, n] and ln Z [B] under the tail-biting measure: every path with s_0 = s_n, whatever the state.

    The measure is the mixture over sigma of the sigma-constrained measures with weights Z_sigma / sum Z, so
    w_soft = sum_sigma pi_sigma w_soft_sigma and ln Z = logsumexp_sigma ln Z_sigma (a sigma with no admissible path
    has Z_sigma = 0).  w is [B, n V] for a codebook [2^L, V].  Composed from this module's sigma-mode soft codeword.
    """
    w = _f32(w)
    _check_shapes(w, _f32(c), L)
    B, n = w.shape   # n: weights per row (steps times V)
    S = 1 << L
    ws_all, lz_all = soft(np.repeat(w, S, axis=0), c, L, k, T, sigma=np.tile(np.arange(S, dtype=np.int32), B))
    lz_all = lz_all.reshape(B, S)
    ws_all = ws_all.reshape(B, S, n)
    m = lz_all.max(axis=1, keepdims=True)
    pz = np.exp(lz_all - m)                      # 0 where ln Z_sigma = -inf
    lnz = m[:, 0] + np.log(pz.sum(axis=1))
    pi = pz / pz.sum(axis=1, keepdims=True)
    ws_all = np.where(pi[:, :, None] > 0, ws_all, 0.0)
    return (pi[:, :, None] * ws_all).sum(axis=1), lnz


def grad_tail_biting(w, c, g, L: int, k: int, T: float):
    """dL/dw [B, n] for upstream g = dL/dw_soft under the tail-biting measure, plus that measure's w_soft [B, n].

    With pi_sigma = Z_sigma / sum Z and d ln Z_sigma / d w_u = (2/T) (w_soft_sigma,u - w_u):
      grad_u = sum_sigma pi_sigma grad_sigma,u
             + (2/T) sum_sigma pi_sigma (w_soft_sigma,u - w_soft_u) (F_sigma - sum_sigma' pi_sigma' F_sigma'),
    F_sigma = sum_t g_t w_soft_sigma,t.  With V weights per step the same holds for every weight component (u, v), the
    energy being a sum over components.  Composed from this module's sigma-mode soft codeword and gradient.
    """
    w = _f32(w)
    g = _f32(g)
    _check_shapes(w, _f32(c), L)
    B, n = w.shape   # n: weights per row (steps times V)
    S = 1 << L
    sig = np.tile(np.arange(S, dtype=np.int32), B)
    W = np.repeat(w, S, axis=0)
    ws_all, lz_all = soft(W, c, L, k, T, sigma=sig)
    gr_all, _ = grad(W, c, np.repeat(g, S, axis=0), L, k, T, sigma=sig)
    lz_all = lz_all.reshape(B, S)
    m = lz_all.max(axis=1, keepdims=True)
    pz = np.exp(lz_all - m)
    pi = pz / pz.sum(axis=1, keepdims=True)
    live = pi[:, :, None] > 0
    ws_all = np.where(live, ws_all.reshape(B, S, n), 0.0)
    gr_all = np.where(live, gr_all.reshape(B, S, n), 0.0)
    ws = (pi[:, :, None] * ws_all).sum(axis=1)
    F = (ws_all * g.astype(np.float64)[:, None, :]).sum(axis=2)        # [B, S]
    Fbar = (pi * F).sum(axis=1, keepdims=True)
    mix = (2.0 / T) * (pi[:, :, None] * (ws_all - ws[:, None, :]) * (F - Fbar)[:, :, None]).sum(axis=1)
    return (pi[:, :, None] * gr_all).sum(axis=1) + mix, ws


def num_threads() -> int:
    """OpenMP threads one oracle call uses."""
    return int(_load().oracle_num_threads())
