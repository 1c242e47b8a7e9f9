"""Independent references that pin the oracle (fp64 NumPy, tiny trellises).

None of this shares code with ``oracle/``: paths are enumerated from the
bit-stream picture of a shift-register trellis (the state at step t is the
L-bit window of a k-bit-per-step stream), and the transfer matrices are built
from the window-overlap rule.  Both are other descriptions of the trellis the
oracle walks with its Succ/Pred recursions, so an index, sign or convention
slip in the oracle shows up as a mismatch here.

Sources: the path measure p_T(path) proportional to exp(-E/T) and the soft
codeword sum_s c(s) p_T(s_t = s) (gist.science Technical Summary, "Core
Mechanism"); the equality with a 1-D Ising transfer-matrix product and the
T -> 0 limit (arXiv abstract).

A codebook [2^L] emits one weight per step; a codebook [2^L, V] emits a
V-vector, and the weights of a sequence are then read as n rows of V.  The
helpers return per-weight quantities flattened in that order.
"""
from __future__ import annotations

import itertools

import numpy as np


# ------------------------------------------------------------------------------------------------
# path enumeration from the bit stream


def free_paths(L: int, k: int, n: int) -> np.ndarray:
    """All free-mode paths [P, n]: every stream of L + k(n-1) bits, s_t = its t-th L-bit window."""
    nbits = L + k * (n - 1)
    x = np.arange(1 << nbits, dtype=np.int64)
    mask = (1 << L) - 1
    cols = [(x >> (k * (n - 1 - t))) & mask for t in range(n)]
    return np.stack(cols, axis=1)


def sigma_paths(L: int, k: int, n: int, sigma: int) -> np.ndarray:
    """Paths with a non-emitting s_0 = sigma and s_n = sigma: streams of L + k n bits led by sigma."""
    y = np.arange(1 << (k * n), dtype=np.int64)
    x = (np.int64(sigma) << (k * n)) | y
    mask = (1 << L) - 1
    cols = [(x >> (k * (n - 1 - t))) & mask for t in range(n)]   # s_1 .. s_n
    p = np.stack(cols, axis=1)
    return p[p[:, -1] == sigma]


def _cw(c, w):
    """Codebook as [S, V] and weights as [n, V] (float64)."""
    c2 = np.asarray(c, np.float64).reshape(np.shape(c)[0], -1)
    return c2, np.asarray(w, np.float64).reshape(-1, c2.shape[1])


def path_energies(paths: np.ndarray, w: np.ndarray, c: np.ndarray) -> np.ndarray:
    """E(path) = sum_t |w_t - c(s_t)|^2 in float64 (V components per step)."""
    c2, w2 = _cw(c, w)
    d = w2[None, :, :] - c2[paths]
    return (d * d).sum(axis=(1, 2))


def _lse(x):
    m = np.max(x)
    return m + np.log(np.sum(np.exp(x - m)))


def _emitted(paths, c):
    """c(s_t) of every path, flattened per weight: [P, n V]."""
    c2 = np.asarray(c, np.float64).reshape(np.shape(c)[0], -1)
    return c2[paths].reshape(paths.shape[0], -1)


def brute_soft(paths, w, c, T):
    """(w_soft [n V], ln Z, probabilities [P]) by summing over every path."""
    E = path_energies(paths, w, c)
    lw = -E / T
    lnz = _lse(lw)
    p = np.exp(lw - lnz)
    cv = _emitted(paths, c)
    return (p[:, None] * cv).sum(axis=0), lnz, p


def brute_jacobian(paths, w, c, T):
    """J_tu = d w_soft_t / d w_u = (2/T) Cov_p(c(s_t), c(s_u)) over all paths (t, u index weights)."""
    _, _, p = brute_soft(paths, w, c, T)
    cv = _emitted(paths, c)
    mu = (p[:, None] * cv).sum(axis=0)
    cc = cv - mu[None, :]
    return (2.0 / T) * (cc * p[:, None]).T @ cc


def brute_codebook_jacobian(paths, w, c, T):
    """K_tv = d w_soft_t / d c(v) over all paths ([n, S] for a scalar codebook, [n V, S V] for a [S, V] one).

    c(v) enters w_soft_t = sum_path p(path) c(s_t) twice: directly (the emitted value, weight P(s_t = v)) and
    through the path measure, where d log p / d c(v) = h_v - E[h_v] with h_v = (2/T) sum_u (w_u - c(v)) [s_u = v]
    (per component when V > 1: the direct term only links equal components).
    """
    _, _, p = brute_soft(paths, w, c, T)
    c2, w2 = _cw(c, w)
    S, V = c2.shape
    n = paths.shape[1]
    onehot = (paths[:, :, None] == np.arange(S)[None, None, :]).astype(np.float64)      # [P, n, S]
    occ = np.einsum("p,pts->ts", p, onehot)                                               # P(s_t = v)
    direct = np.einsum("ts,ab->tasb", occ, np.eye(V)).reshape(n * V, S * V)
    dw = w2[:, None, :] - c2[None, :, :]                                                  # [n, S, V]
    h = (2.0 / T) * np.einsum("pus,usb->psb", onehot, dw).reshape(-1, S * V)              # [P, S V]
    hc = h - (p[:, None] * h).sum(axis=0)[None, :]
    cv = _emitted(paths, c)
    cc = cv - (p[:, None] * cv).sum(axis=0)[None, :]
    K = direct + np.einsum("p,pt,ps->ts", p, cc, hc)
    return K if np.ndim(c) == 2 else K.reshape(n, S)


def brute_viterbi_fp32(paths, w, c):
    """Per-path float32 cost accumulated in step order, ((e_1 + e_2) + e_3) + ..., and the argmin set.

    e_t = |w_t - c(s_t)|^2 in float32 with the V components added in index order."""
    c32 = np.asarray(c, np.float32).reshape(np.shape(c)[0], -1)
    V = c32.shape[1]
    w32 = np.asarray(w, np.float32).reshape(-1, V)
    acc = np.zeros(paths.shape[0], np.float32)
    for t in range(paths.shape[1]):
        e = None
        for v in range(V):
            d = (w32[t, v] - c32[paths[:, t], v]).astype(np.float32)
            dd = (d * d).astype(np.float32)
            e = dd if e is None else (e + dd).astype(np.float32)
        acc = (e + acc).astype(np.float32) if t else e
    best = acc.min()
    return acc, np.flatnonzero(acc == best)


# ------------------------------------------------------------------------------------------------
# Ising transfer matrices


def shift_matrix(L: int, k: int) -> np.ndarray:
    """A[s, s'] = 1 iff the low L-k bits of s are the high L-k bits of s' (the windows overlap)."""
    S = 1 << L
    s = np.arange(S)
    low = s & ((1 << (L - k)) - 1)
    high = s >> k
    return (low[:, None] == high[None, :]).astype(np.float64)


def transfer_product_log(w, c, T, L, k):
    """log of the (scaled) product (A D_1)(A D_2)...(A D_n) as (matrix, log scale), D_t = diag exp(theta_t)."""
    A = shift_matrix(L, k)
    M = np.eye(1 << L)
    logscale = 0.0
    c2, w2 = _cw(c, w)
    for t in range(w2.shape[0]):
        D = np.exp(-((w2[t][None, :] - c2) ** 2).sum(axis=1) / T)
        M = (M @ A) * D[None, :]
        s = M.max()
        M = M / s
        logscale += np.log(s)
    return M, logscale


def transfer_lnz_free(w, c, T, L, k):
    """ln Z_free from 1^T (A D_1)...(A D_n) 1 = 2^k Z_free (a free non-emitting s_0 adds 2^k choices)."""
    M, ls = transfer_product_log(w, c, T, L, k)
    return np.log(M.sum()) + ls - k * np.log(2.0)


def transfer_lnz_sigma(w, c, T, L, k, sigma):
    """ln Z_sigma = ln [(A D_1)...(A D_n)]_{sigma, sigma}."""
    M, ls = transfer_product_log(w, c, T, L, k)
    return np.log(M[sigma, sigma]) + ls


# ------------------------------------------------------------------------------------------------
# uniform-measure covariances (the T -> infinity limit)


def uniform_lag_cov(L: int, k: int, lag: int, f, g) -> float:
    """Cov(f(s_t), g(s_{t+lag})) under the uniform path measure, by enumerating the joint window."""
    S = 1 << L
    if k * lag >= L:
        return 0.0
    nbits = L + k * lag
    x = np.arange(1 << nbits, dtype=np.int64)
    st = (x >> (k * lag)) & (S - 1)
    su = x & (S - 1)
    fv = f[st]
    gv = g[su]
    return float((fv * gv).mean() - fv.mean() * gv.mean())


def symbol_reverse(L: int, k: int) -> np.ndarray:
    """rho(s): reverse the order of the k-bit symbols of an L-bit state (L a multiple of k)."""
    S = 1 << L
    m = L // k
    out = np.zeros(S, np.int64)
    for s in range(S):
        r = 0
        for i in range(m):
            r = (r << k) | ((s >> (k * i)) & ((1 << k) - 1))
        out[s] = r
    return out


def dyadic(a: np.ndarray, bits: int = 12) -> np.ndarray:
    """Round to multiples of 2^-bits so that small dyadic shifts stay exact in float32."""
    return (np.round(np.asarray(a, np.float64) * (1 << bits)) / (1 << bits)).astype(np.float32)


def all_tuples(P: int, n: int):
    return itertools.product(range(P), repeat=n)
