"""ctypes view of libbcjr.so, the C-ABI declared in include/bcjr.h.

Each entry point is the library's own ctypes function under its C name, with the argument types of the header (plain
integers for device pointers and the stream), e.g. ``abi.bcjr_soft_codeword(...)``.  Loading fails loudly when the
library has not been built: there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# BCJR_LIB selects another build of the library (the host-sanitizer build of the CPU test sessions)
LIB_PATH = os.environ.get("BCJR_LIB") or os.path.join(_PKG, "libbcjr.so")

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

BCJR_NOALLOC_SCRATCH_BYTES = 256 << 20

_vp, _i64, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_int = ctypes.c_int

# C name -> (argument types, result type), in the order of include/bcjr.h
_SIGNATURES = {
    "bcjr_soft_codeword": ([_vp, _vp, _i64, _i64, _i32, _i32, _f32, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "bcjr_soft_codeword_grad": ([_vp, _vp, _i64, _i64, _i32, _i32, _f32, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "bcjr_soft_codeword_grad_codebook": ([_vp, _vp, _i64, _i64, _i32, _i32, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                          _vp], _int),
    "viterbi_hard_code": ([_vp, _vp, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "bcjr_soft_codeword_tail_biting": ([_vp, _vp, _i64, _i64, _i32, _i32, _f32, _vp, _vp, _vp, _sz, _vp], _int),
    "bcjr_soft_codeword_grad_tail_biting": ([_vp, _vp, _i64, _i64, _i32, _i32, _f32, _vp, _vp, _vp, _vp, _sz, _vp],
                                            _int),
    "viterbi_tail_biting": ([_vp, _vp, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "bcjr_soft_codeword_v": ([_vp, _vp, _i64, _i64, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "bcjr_soft_codeword_grad_v": ([_vp, _vp, _i64, _i64, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
                                  _int),
    "viterbi_hard_code_v": ([_vp, _vp, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "bcjr_soft_codeword_grad_codebook_v": ([_vp, _vp, _i64, _i64, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _vp, _vp,
                                            _vp, _sz, _vp], _int),
    "bcjr_soft_codeword_tail_biting_v": ([_vp, _vp, _i64, _i64, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _sz, _vp],
                                         _int),
    "bcjr_soft_codeword_grad_tail_biting_v": ([_vp, _vp, _i64, _i64, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _vp, _sz,
                                               _vp], _int),
    "viterbi_tail_biting_v": ([_vp, _vp, _i64, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
                              _int),
    "bcjr_workspace_bytes": ([_i32, _i64, _i64, _i32, _i32], _sz),
    "bcjr_workspace_bytes_v": ([_i32, _i64, _i64, _i32, _i32, _i32], _sz),
    "bcjr_workspace_bytes_min": ([_i32, _i64, _i64, _i32, _i32, _i32], _sz),
    "bcjr_soft_codeword_noalloc": ([_vp, _vp, _i64, _i64, _i32, _i32, _f32, _vp, _vp, _vp, _vp], _int),
    "bcjr_status_string": ([_i32], ctypes.c_char_p),
}

EXPORTS = tuple(_SIGNATURES)

_lib = None


def load() -> ctypes.CDLL:
    """The library with every entry point's argument and result types set."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m differentiable_bcjr_amd.build` "
                           "(or __graft_entry__.build()); the BCJR path has no fallback")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (args, res) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def bcjr_status_string(status: int) -> str:
    """The library's text for a status code."""
    return load().bcjr_status_string(status).decode()


def __getattr__(name: str):
    # every other entry point is the ctypes function itself
    if name in _SIGNATURES:
        return getattr(load(), name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")
