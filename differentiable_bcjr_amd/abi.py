"""ctypes view of libbcjr.so, the C-ABI declared in include/bcjr.h.

The functions keep the C names and argument lists (plain integers for device pointers and the stream).  Loading fails
loudly when the library has not been built: there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbcjr.so")

BCJR_OK = 0
BCJR_ERR_NULL = -1
BCJR_ERR_SHAPE = -2
BCJR_ERR_TEMP = -3
BCJR_ERR_UNSUPPORTED = -4
BCJR_ERR_WORKSPACE = -5
BCJR_ERR_HIP = -6

BCJR_OP_SOFT = 0
BCJR_OP_GRAD = 1
BCJR_OP_VITERBI = 2
BCJR_OP_GRAD_CODEBOOK = 3
BCJR_OP_VITERBI_TB_EXACT = 4
BCJR_OP_VITERBI_TB_ROTATE = 5
BCJR_OP_SOFT_TAIL_BITING = 6
BCJR_OP_GRAD_TAIL_BITING = 7

BCJR_TB_EXACT = 0
BCJR_TB_ROTATE = 1

EXPORTS = ("bcjr_soft_codeword", "bcjr_soft_codeword_grad", "bcjr_soft_codeword_grad_codebook", "viterbi_hard_code",
           "viterbi_tail_biting", "bcjr_soft_codeword_tail_biting", "bcjr_soft_codeword_grad_tail_biting",
           "bcjr_soft_codeword_v", "bcjr_soft_codeword_grad_v", "bcjr_soft_codeword_grad_codebook_v",
           "viterbi_hard_code_v", "bcjr_soft_codeword_tail_biting_v", "bcjr_soft_codeword_grad_tail_biting_v",
           "viterbi_tail_biting_v", "bcjr_workspace_bytes", "bcjr_workspace_bytes_min",
           "bcjr_workspace_bytes_v", "bcjr_status_string")

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m differentiable_bcjr_amd.build` "
                           "(or __graft_entry__.build()); the BCJR path has no fallback")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.bcjr_soft_codeword.argtypes = [vp, vp, i64, i64, i32, i32, f32, vp, vp, vp, vp, sz, vp]
    lib.bcjr_soft_codeword.restype = ctypes.c_int
    lib.bcjr_soft_codeword_grad.argtypes = [vp, vp, i64, i64, i32, i32, f32, vp, vp, vp, vp, vp, sz, vp]
    lib.bcjr_soft_codeword_grad.restype = ctypes.c_int
    lib.bcjr_soft_codeword_grad_codebook.argtypes = [vp, vp, i64, i64, i32, i32, f32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.bcjr_soft_codeword_grad_codebook.restype = ctypes.c_int
    lib.viterbi_hard_code.argtypes = [vp, vp, i64, i64, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.viterbi_hard_code.restype = ctypes.c_int
    lib.bcjr_soft_codeword_tail_biting.argtypes = [vp, vp, i64, i64, i32, i32, f32, vp, vp, vp, sz, vp]
    lib.bcjr_soft_codeword_tail_biting.restype = ctypes.c_int
    lib.bcjr_soft_codeword_grad_tail_biting.argtypes = [vp, vp, i64, i64, i32, i32, f32, vp, vp, vp, vp, sz, vp]
    lib.bcjr_soft_codeword_grad_tail_biting.restype = ctypes.c_int
    lib.viterbi_tail_biting.argtypes = [vp, vp, i64, i64, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.viterbi_tail_biting.restype = ctypes.c_int
    lib.bcjr_soft_codeword_v.argtypes = [vp, vp, i64, i64, i32, i32, i32, f32, vp, vp, vp, vp, sz, vp]
    lib.bcjr_soft_codeword_v.restype = ctypes.c_int
    lib.bcjr_soft_codeword_grad_v.argtypes = [vp, vp, i64, i64, i32, i32, i32, f32, vp, vp, vp, vp, vp, sz, vp]
    lib.bcjr_soft_codeword_grad_v.restype = ctypes.c_int
    lib.bcjr_soft_codeword_grad_codebook_v.argtypes = [vp, vp, i64, i64, i32, i32, i32, f32, vp, vp, vp, vp, vp, vp,
                                                       sz, vp]
    lib.bcjr_soft_codeword_grad_codebook_v.restype = ctypes.c_int
    lib.viterbi_hard_code_v.argtypes = [vp, vp, i64, i64, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.viterbi_hard_code_v.restype = ctypes.c_int
    lib.bcjr_soft_codeword_tail_biting_v.argtypes = [vp, vp, i64, i64, i32, i32, i32, f32, vp, vp, vp, sz, vp]
    lib.bcjr_soft_codeword_tail_biting_v.restype = ctypes.c_int
    lib.bcjr_soft_codeword_grad_tail_biting_v.argtypes = [vp, vp, i64, i64, i32, i32, i32, f32, vp, vp, vp, vp, sz,
                                                          vp]
    lib.bcjr_soft_codeword_grad_tail_biting_v.restype = ctypes.c_int
    lib.viterbi_tail_biting_v.argtypes = [vp, vp, i64, i64, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.viterbi_tail_biting_v.restype = ctypes.c_int
    lib.bcjr_workspace_bytes.argtypes = [i32, i64, i64, i32, i32]
    lib.bcjr_workspace_bytes.restype = sz
    lib.bcjr_workspace_bytes_v.argtypes = [i32, i64, i64, i32, i32, i32]
    lib.bcjr_workspace_bytes_v.restype = sz
    lib.bcjr_workspace_bytes_min.argtypes = [i32, i64, i64, i32, i32, i32]
    lib.bcjr_workspace_bytes_min.restype = sz
    lib.bcjr_status_string.argtypes = [i32]
    lib.bcjr_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def bcjr_soft_codeword(w, codebook, B, n, L, k, T, boundary_state, w_soft, log_z, workspace, workspace_bytes,
                       stream) -> int:
    return load().bcjr_soft_codeword(w, codebook, B, n, L, k, T, boundary_state, w_soft, log_z, workspace,
                                     workspace_bytes, stream)


def bcjr_soft_codeword_grad(w, codebook, B, n, L, k, T, boundary_state, grad_w_soft, grad_w, w_soft, workspace,
                            workspace_bytes, stream) -> int:
    return load().bcjr_soft_codeword_grad(w, codebook, B, n, L, k, T, boundary_state, grad_w_soft, grad_w, w_soft,
                                          workspace, workspace_bytes, stream)


def bcjr_soft_codeword_grad_codebook(w, codebook, B, n, L, k, T, boundary_state, grad_w_soft, grad_codebook, grad_w,
                                     w_soft, workspace, workspace_bytes, stream) -> int:
    return load().bcjr_soft_codeword_grad_codebook(w, codebook, B, n, L, k, T, boundary_state, grad_w_soft,
                                                   grad_codebook, grad_w, w_soft, workspace, workspace_bytes, stream)


def viterbi_hard_code(w, codebook, B, n, L, k, boundary_state, states, w_hard, cost, workspace, workspace_bytes,
                      stream) -> int:
    return load().viterbi_hard_code(w, codebook, B, n, L, k, boundary_state, states, w_hard, cost, workspace,
                                    workspace_bytes, stream)


def bcjr_soft_codeword_tail_biting(w, codebook, B, n, L, k, T, w_soft, log_z, workspace, workspace_bytes,
                                   stream) -> int:
    return load().bcjr_soft_codeword_tail_biting(w, codebook, B, n, L, k, T, w_soft, log_z, workspace,
                                                 workspace_bytes, stream)


def bcjr_soft_codeword_grad_tail_biting(w, codebook, B, n, L, k, T, grad_w_soft, grad_w, w_soft, workspace,
                                        workspace_bytes, stream) -> int:
    return load().bcjr_soft_codeword_grad_tail_biting(w, codebook, B, n, L, k, T, grad_w_soft, grad_w, w_soft,
                                                      workspace, workspace_bytes, stream)


def viterbi_tail_biting(w, codebook, B, n, L, k, mode, states, w_hard, cost, sigma, workspace, workspace_bytes,
                        stream) -> int:
    return load().viterbi_tail_biting(w, codebook, B, n, L, k, mode, states, w_hard, cost, sigma, workspace,
                                      workspace_bytes, stream)


def bcjr_soft_codeword_v(w, codebook, B, n, L, k, V, T, boundary_state, w_soft, log_z, workspace, workspace_bytes,
                         stream) -> int:
    return load().bcjr_soft_codeword_v(w, codebook, B, n, L, k, V, T, boundary_state, w_soft, log_z, workspace,
                                       workspace_bytes, stream)


def bcjr_soft_codeword_grad_v(w, codebook, B, n, L, k, V, T, boundary_state, grad_w_soft, grad_w, w_soft, workspace,
                              workspace_bytes, stream) -> int:
    return load().bcjr_soft_codeword_grad_v(w, codebook, B, n, L, k, V, T, boundary_state, grad_w_soft, grad_w,
                                            w_soft, workspace, workspace_bytes, stream)


def bcjr_soft_codeword_grad_codebook_v(w, codebook, B, n, L, k, V, T, boundary_state, grad_w_soft, grad_codebook,
                                       grad_w, w_soft, workspace, workspace_bytes, stream) -> int:
    return load().bcjr_soft_codeword_grad_codebook_v(w, codebook, B, n, L, k, V, T, boundary_state, grad_w_soft,
                                                     grad_codebook, grad_w, w_soft, workspace, workspace_bytes, stream)


def viterbi_hard_code_v(w, codebook, B, n, L, k, V, boundary_state, states, w_hard, cost, workspace, workspace_bytes,
                        stream) -> int:
    return load().viterbi_hard_code_v(w, codebook, B, n, L, k, V, boundary_state, states, w_hard, cost, workspace,
                                      workspace_bytes, stream)


def bcjr_soft_codeword_tail_biting_v(w, codebook, B, n, L, k, V, T, w_soft, log_z, workspace, workspace_bytes,
                                     stream) -> int:
    return load().bcjr_soft_codeword_tail_biting_v(w, codebook, B, n, L, k, V, T, w_soft, log_z, workspace,
                                                   workspace_bytes, stream)


def bcjr_soft_codeword_grad_tail_biting_v(w, codebook, B, n, L, k, V, T, grad_w_soft, grad_w, w_soft, workspace,
                                          workspace_bytes, stream) -> int:
    return load().bcjr_soft_codeword_grad_tail_biting_v(w, codebook, B, n, L, k, V, T, grad_w_soft, grad_w, w_soft,
                                                        workspace, workspace_bytes, stream)


def viterbi_tail_biting_v(w, codebook, B, n, L, k, V, mode, states, w_hard, cost, sigma, workspace, workspace_bytes,
                          stream) -> int:
    return load().viterbi_tail_biting_v(w, codebook, B, n, L, k, V, mode, states, w_hard, cost, sigma, workspace,
                                        workspace_bytes, stream)


def bcjr_workspace_bytes(op, B, n, L, k) -> int:
    return int(load().bcjr_workspace_bytes(op, B, n, L, k))


def bcjr_workspace_bytes_v(op, B, n, L, k, V) -> int:
    return int(load().bcjr_workspace_bytes_v(op, B, n, L, k, V))


def bcjr_workspace_bytes_min(op, B, n, L, k, V) -> int:
    return int(load().bcjr_workspace_bytes_min(op, B, n, L, k, V))


def bcjr_status_string(status) -> str:
    return load().bcjr_status_string(status).decode()
