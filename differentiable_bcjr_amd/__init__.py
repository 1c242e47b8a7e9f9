"""differentiable_bcjr_amd -- the temperature-T BCJR soft quantizer of BCJR-QAT on MI355X (gfx950).

Three operations, each a hand-written HIP kernel behind the C-ABI of ``include/bcjr.h``:

* ``soft_codeword``      -- w_soft[b, t] = E_p[c(s_t)], the Boltzmann expectation of the codebook value over all
  bitshift-trellis paths at temperature T, and ln Z (BCJR-QAT, arXiv 2605.10655; gist.science Technical Summary,
  "Core Mechanism"); ``soft_codeword_noalloc`` is the same in the library's static scratch, for callers that cannot
  allocate;
* ``soft_codeword_grad`` -- dL/dw from an upstream dL/dw_soft, the exact derivative of the soft codeword;
* ``soft_codeword_grad_codebook`` -- dL/dc [2^L], the exact derivative in the codebook values (the trellis
  parameters), summed over the batch, together with dL/dw;
* ``viterbi_hard_code``  -- the minimum-energy path (the T -> 0 limit, abstract), bit-exact in float32;
* ``viterbi_tail_biting`` -- the same with s_0 = s_n and the start state chosen exactly or by rotate-and-decode;
* ``soft_codeword_tail_biting``, ``soft_codeword_grad_tail_biting`` -- the soft codeword and its weights' gradient
  under the tail-biting measure (every s_0 = s_n path, summed over the state; L <= 10).

``soft_quantize`` ties them together for autograd: its forward is ``soft_codeword``; its backward is
``soft_codeword_grad``, or ``soft_codeword_grad_codebook`` when the codebook needs a gradient too.  Both gradients
are exact: the pages state that the soft codeword is differentiable without approximation in the weights and in the
trellis parameters (Technical Summary, "Core Mechanism").

``temperature_schedule`` gives the annealing sequence T0 -> T_end for a QAT run (host-side, see ``anneal``).

Trellis variants: ``k`` (bits shifted in per step) may be 1 to 4 for every operation.  A codebook of shape [2^L, V]
emits V weights per step (V = 1 or 2): the weights are then [B, n V], step t of a row owning its weights
t V .. t V + V - 1, and Viterbi returns one state per step.

These wrappers only marshal arguments: they check tensor dtypes/devices, allocate outputs and the workspace with
torch, and pass raw device pointers and the current HIP stream to the library.  Every step of the computation runs
in the library's kernels.
"""
from __future__ import annotations

import torch

from . import abi
from .anneal import temperature_schedule

__all__ = ["soft_codeword", "soft_codeword_noalloc", "soft_codeword_grad", "soft_codeword_grad_codebook", "viterbi_hard_code",
           "viterbi_tail_biting", "soft_codeword_tail_biting", "soft_codeword_grad_tail_biting", "soft_quantize",
           "temperature_schedule", "workspace_bytes", "BCJRError", "abi"]


class BCJRError(RuntimeError):
    """A non-zero status from libbcjr.so."""

    def __init__(self, status: int):
        super().__init__(abi.bcjr_status_string(status))
        self.status = status


def _check(rc: int) -> None:
    if rc != abi.BCJR_OK:
        raise BCJRError(rc)


def _f32(x: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if x.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")
    return x.contiguous()


def _sigma(s, B: int, device) -> torch.Tensor | None:
    if s is None:
        return None
    if not isinstance(s, torch.Tensor) or not s.is_cuda or s.dtype != torch.int32 or s.numel() != B:
        raise TypeError("boundary_state must be an int32 CUDA tensor with one entry per sequence")
    return s.contiguous()


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def workspace_bytes(op: int, B: int, n: int, L: int, k: int = 2, V: int = 1) -> int:
    """Device workspace bytes the library needs for op (abi.BCJR_OP_SOFT / _GRAD / _VITERBI / _GRAD_CODEBOOK ...) on
    B sequences of n trellis steps."""
    return abi.bcjr_workspace_bytes_v(op, B, n, L, k, V)


def _workspace(op, B, n, L, k, device, workspace, V=1, checkpoint=False):
    """The caller's workspace, or a new one: the full tape, or with ``checkpoint`` the smallest the op accepts (the
    checkpoint-and-recompute memory mode).  A caller's workspace must be a contiguous device tensor on the weights'
    device; its size in bytes is what the library is told."""
    need = workspace_bytes(op, B, n, L, k, V)
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or workspace.device != device:
            raise TypeError("workspace must be a CUDA (HIP) tensor on the weights' device")
        if not workspace.is_contiguous():
            raise TypeError("workspace must be contiguous")
    if checkpoint and workspace is None:
        workspace = torch.empty(max(abi.bcjr_workspace_bytes_min(op, B, n, L, k, V), 1), dtype=torch.uint8,
                                device=device)
    if workspace is None:
        # torch's allocator hands out 512-byte aligned blocks; the library checks 256-byte alignment itself
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return workspace, need


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _steps(w: torch.Tensor, codebook: torch.Tensor, L: int):
    """(B, trellis steps n, V) for w [B, n V] and a codebook [2^L] (V = 1) or [2^L, V]."""
    if w.dim() != 2:
        raise ValueError("w must be [B, n] (or [B, n V] with a codebook [2^L, V])")
    if codebook.dim() == 1:
        V = 1
    elif codebook.dim() == 2:
        V = codebook.shape[1]
    else:
        raise ValueError("codebook must be [2^L] or [2^L, V]")
    if codebook.shape[0] != 1 << L or V < 1 or w.shape[1] % V:
        raise ValueError(f"codebook must have 2^L = {1 << L} rows and the weights per row must be a multiple of V")
    return w.shape[0], w.shape[1] // V, V


def soft_codeword(w: torch.Tensor, codebook: torch.Tensor, L: int, k: int = 2, T: float = 1.0,
                  boundary_state: torch.Tensor | None = None, *, return_log_z: bool = False,
                  workspace: torch.Tensor | None = None, checkpoint: bool = False):
    """Soft codeword with w's shape (and ln Z [B] if ``return_log_z``) for weights w [B, n] and codebook [2^L], or
    w [B, n V] and codebook [2^L, V].  ``checkpoint`` allocates the smallest workspace, which runs the checkpoint-and-
    recompute memory mode (about 2 sqrt(n) message rows per in-flight sequence instead of n + 1)."""
    w = _f32(w, "w")
    codebook = _f32(codebook, "codebook")
    B, n, V = _steps(w, codebook, L)
    sig = _sigma(boundary_state, B, w.device)
    out = torch.empty_like(w)
    lz = torch.empty(B, dtype=torch.float32, device=w.device) if return_log_z else None
    ws, need = _workspace(abi.BCJR_OP_SOFT, B, n, L, k, w.device, workspace, V, checkpoint)
    if V == 1:
        _check(abi.bcjr_soft_codeword(w.data_ptr(), codebook.data_ptr(), B, n, L, k, float(T), _ptr(sig),
                                      out.data_ptr(), _ptr(lz), ws.data_ptr(), _nbytes(ws), _stream(w.device)))
    else:
        _check(abi.bcjr_soft_codeword_v(w.data_ptr(), codebook.data_ptr(), B, n, L, k, V, float(T), _ptr(sig),
                                        out.data_ptr(), _ptr(lz), ws.data_ptr(), _nbytes(ws), _stream(w.device)))
    return (out, lz) if return_log_z else out


def soft_codeword_noalloc(w: torch.Tensor, codebook: torch.Tensor, L: int, k: int = 2, T: float = 1.0,
                          boundary_state: torch.Tensor | None = None, *, out: torch.Tensor | None = None,
                          log_z: torch.Tensor | None = None) -> torch.Tensor:
    """``soft_codeword`` for a codebook [2^L] through ``bcjr_soft_codeword_noalloc``, which works in the library's
    static device scratch and allocates nothing.  Pass ``out`` (w's shape) and optionally ``log_z`` ([B]) to keep this
    call free of allocations too.  Calls that overlap in time on one device race on that scratch."""
    w = _f32(w, "w")
    codebook = _f32(codebook, "codebook")
    B, n, V = _steps(w, codebook, L)
    if V != 1:
        raise ValueError("soft_codeword_noalloc takes a codebook [2^L] (one weight per step)")
    sig = _sigma(boundary_state, B, w.device)
    if out is None:
        out = torch.empty_like(w)
    for t, shape in ((out, w.shape), (log_z, (B,))):
        if t is not None and (not t.is_cuda or t.device != w.device or t.dtype != torch.float32
                              or tuple(t.shape) != tuple(shape) or not t.is_contiguous()):
            raise TypeError(f"outputs must be contiguous float32 tensors of shape {tuple(shape)} on w's device")
    _check(abi.bcjr_soft_codeword_noalloc(w.data_ptr(), codebook.data_ptr(), B, n, L, k, float(T), _ptr(sig),
                                          out.data_ptr(), _ptr(log_z), _stream(w.device)))
    return out


def soft_codeword_grad(w: torch.Tensor, codebook: torch.Tensor, grad_w_soft: torch.Tensor, L: int, k: int = 2,
                       T: float = 1.0, boundary_state: torch.Tensor | None = None, *, return_w_soft: bool = False,
                       workspace: torch.Tensor | None = None, checkpoint: bool = False):
    """dL/dw given dL/dw_soft, both with w's shape (and the soft codeword if ``return_w_soft``).  ``checkpoint``
    allocates the smallest workspace, which runs the checkpoint-and-recompute memory mode."""
    w = _f32(w, "w")
    codebook = _f32(codebook, "codebook")
    g = _f32(grad_w_soft, "grad_w_soft")
    B, n, V = _steps(w, codebook, L)
    if g.shape != w.shape:
        raise ValueError("grad_w_soft must have w's shape")
    sig = _sigma(boundary_state, B, w.device)
    grad = torch.empty_like(w)
    ws_out = torch.empty_like(w) if return_w_soft else None
    ws, need = _workspace(abi.BCJR_OP_GRAD, B, n, L, k, w.device, workspace, V, checkpoint)
    if V == 1:
        _check(abi.bcjr_soft_codeword_grad(w.data_ptr(), codebook.data_ptr(), B, n, L, k, float(T), _ptr(sig),
                                           g.data_ptr(), grad.data_ptr(), _ptr(ws_out), ws.data_ptr(), _nbytes(ws),
                                           _stream(w.device)))
    else:
        _check(abi.bcjr_soft_codeword_grad_v(w.data_ptr(), codebook.data_ptr(), B, n, L, k, V, float(T), _ptr(sig),
                                             g.data_ptr(), grad.data_ptr(), _ptr(ws_out), ws.data_ptr(), _nbytes(ws),
                                             _stream(w.device)))
    return (grad, ws_out) if return_w_soft else grad


def soft_codeword_grad_codebook(w: torch.Tensor, codebook: torch.Tensor, grad_w_soft: torch.Tensor, L: int,
                                k: int = 2, T: float = 1.0, boundary_state: torch.Tensor | None = None, *,
                                return_grad_w: bool = True, return_w_soft: bool = False,
                                workspace: torch.Tensor | None = None, checkpoint: bool = False):
    """dL/dc with the codebook's shape ([2^L], or [2^L, V] for V weights per step; summed over the batch) given
    dL/dw_soft with w's shape; then dL/dw if ``return_grad_w`` and the soft codeword if ``return_w_soft``.  Returns a
    tuple when either is asked for.  ``checkpoint`` allocates the smallest workspace (checkpoint-and-recompute)."""
    w = _f32(w, "w")
    codebook = _f32(codebook, "codebook")
    g = _f32(grad_w_soft, "grad_w_soft")
    B, n, V = _steps(w, codebook, L)
    if g.shape != w.shape:
        raise ValueError("grad_w_soft must have w's shape")
    sig = _sigma(boundary_state, B, w.device)
    gc = torch.empty(codebook.shape, dtype=torch.float32, device=w.device)
    grad = torch.empty_like(w) if return_grad_w else None
    ws_out = torch.empty_like(w) if return_w_soft else None
    ws, need = _workspace(abi.BCJR_OP_GRAD_CODEBOOK, B, n, L, k, w.device, workspace, V, checkpoint)
    if V == 1:
        _check(abi.bcjr_soft_codeword_grad_codebook(w.data_ptr(), codebook.data_ptr(), B, n, L, k, float(T),
                                                    _ptr(sig), g.data_ptr(), gc.data_ptr(), _ptr(grad), _ptr(ws_out),
                                                    ws.data_ptr(), _nbytes(ws), _stream(w.device)))
    else:
        _check(abi.bcjr_soft_codeword_grad_codebook_v(w.data_ptr(), codebook.data_ptr(), B, n, L, k, V, float(T),
                                                      _ptr(sig), g.data_ptr(), gc.data_ptr(), _ptr(grad),
                                                      _ptr(ws_out), ws.data_ptr(), _nbytes(ws), _stream(w.device)))
    extra = tuple(x for x in (grad, ws_out) if x is not None)
    return (gc, *extra) if extra else gc


def viterbi_hard_code(w: torch.Tensor, codebook: torch.Tensor, L: int, k: int = 2,
                      boundary_state: torch.Tensor | None = None, *, workspace: torch.Tensor | None = None):
    """(states [B, n] int32, one per step, w_hard with w's shape, cost [B] float32) of the minimum-energy paths."""
    w = _f32(w, "w")
    codebook = _f32(codebook, "codebook")
    B, n, V = _steps(w, codebook, L)
    sig = _sigma(boundary_state, B, w.device)
    states = torch.empty((B, n), dtype=torch.int32, device=w.device)
    w_hard = torch.empty_like(w)
    cost = torch.empty(B, dtype=torch.float32, device=w.device)
    ws, need = _workspace(abi.BCJR_OP_VITERBI, B, n, L, k, w.device, workspace, V)
    if V == 1:
        _check(abi.viterbi_hard_code(w.data_ptr(), codebook.data_ptr(), B, n, L, k, _ptr(sig), states.data_ptr(),
                                     w_hard.data_ptr(), cost.data_ptr(), ws.data_ptr(), _nbytes(ws),
                                     _stream(w.device)))
    else:
        _check(abi.viterbi_hard_code_v(w.data_ptr(), codebook.data_ptr(), B, n, L, k, V, _ptr(sig),
                                       states.data_ptr(), w_hard.data_ptr(), cost.data_ptr(), ws.data_ptr(),
                                       _nbytes(ws), _stream(w.device)))
    return states, w_hard, cost


def soft_codeword_tail_biting(w: torch.Tensor, codebook: torch.Tensor, L: int, k: int = 2, T: float = 1.0, *,
                              return_log_z: bool = False, workspace: torch.Tensor | None = None):
    """Soft codeword with w's shape (and ln Z [B]) under the tail-biting measure: every path with s_0 = s_n
    (L <= 10).  w [B, n] with codebook [2^L], or w [B, n V] with codebook [2^L, V]."""
    w = _f32(w, "w")
    codebook = _f32(codebook, "codebook")
    B, n, V = _steps(w, codebook, L)
    out = torch.empty_like(w)
    lz = torch.empty(B, dtype=torch.float32, device=w.device) if return_log_z else None
    ws, need = _workspace(abi.BCJR_OP_SOFT_TAIL_BITING, B, n, L, k, w.device, workspace, V)
    if V == 1:
        _check(abi.bcjr_soft_codeword_tail_biting(w.data_ptr(), codebook.data_ptr(), B, n, L, k, float(T),
                                                  out.data_ptr(), _ptr(lz), ws.data_ptr(), _nbytes(ws),
                                                  _stream(w.device)))
    else:
        _check(abi.bcjr_soft_codeword_tail_biting_v(w.data_ptr(), codebook.data_ptr(), B, n, L, k, V, float(T),
                                                    out.data_ptr(), _ptr(lz), ws.data_ptr(), _nbytes(ws),
                                                    _stream(w.device)))
    return (out, lz) if return_log_z else out


def soft_codeword_grad_tail_biting(w: torch.Tensor, codebook: torch.Tensor, grad_w_soft: torch.Tensor, L: int,
                                   k: int = 2, T: float = 1.0, *, return_w_soft: bool = False,
                                   workspace: torch.Tensor | None = None):
    """dL/dw under the tail-biting measure given dL/dw_soft, both with w's shape (and that measure's soft
    codeword).  w [B, n] with codebook [2^L], or w [B, n V] with codebook [2^L, V]."""
    w = _f32(w, "w")
    codebook = _f32(codebook, "codebook")
    g = _f32(grad_w_soft, "grad_w_soft")
    B, n, V = _steps(w, codebook, L)
    if g.shape != w.shape:
        raise ValueError("grad_w_soft must have w's shape")
    grad = torch.empty_like(w)
    ws_out = torch.empty_like(w) if return_w_soft else None
    ws, need = _workspace(abi.BCJR_OP_GRAD_TAIL_BITING, B, n, L, k, w.device, workspace, V)
    if V == 1:
        _check(abi.bcjr_soft_codeword_grad_tail_biting(w.data_ptr(), codebook.data_ptr(), B, n, L, k, float(T),
                                                       g.data_ptr(), grad.data_ptr(), _ptr(ws_out), ws.data_ptr(),
                                                       _nbytes(ws), _stream(w.device)))
    else:
        _check(abi.bcjr_soft_codeword_grad_tail_biting_v(w.data_ptr(), codebook.data_ptr(), B, n, L, k, V, float(T),
                                                         g.data_ptr(), grad.data_ptr(), _ptr(ws_out), ws.data_ptr(),
                                                         _nbytes(ws), _stream(w.device)))
    return (grad, ws_out) if return_w_soft else grad


_TB_MODES = {"exact": (abi.BCJR_TB_EXACT, abi.BCJR_OP_VITERBI_TB_EXACT),
             "rotate": (abi.BCJR_TB_ROTATE, abi.BCJR_OP_VITERBI_TB_ROTATE)}


def viterbi_tail_biting(w: torch.Tensor, codebook: torch.Tensor, L: int, k: int = 2, mode: str = "exact", *,
                        workspace: torch.Tensor | None = None):
    """(states [B, n] int32, w_hard with w's shape, cost [B], sigma [B] int32) of the minimum-energy tail-biting
    paths (s_0 = s_n), the start state chosen ``"exact"``ly (L <= 10) or by ``"rotate"``-and-decode.  w [B, n] with
    codebook [2^L], or w [B, n V] with codebook [2^L, V] (n trellis steps)."""
    if mode not in _TB_MODES:
        raise ValueError(f"mode must be one of {sorted(_TB_MODES)}")
    tb_mode, op = _TB_MODES[mode]
    w = _f32(w, "w")
    codebook = _f32(codebook, "codebook")
    B, n, V = _steps(w, codebook, L)
    states = torch.empty((B, n), dtype=torch.int32, device=w.device)
    w_hard = torch.empty_like(w)
    cost = torch.empty(B, dtype=torch.float32, device=w.device)
    sigma = torch.empty(B, dtype=torch.int32, device=w.device)
    ws, need = _workspace(op, B, n, L, k, w.device, workspace, V)
    if V == 1:
        _check(abi.viterbi_tail_biting(w.data_ptr(), codebook.data_ptr(), B, n, L, k, tb_mode, states.data_ptr(),
                                       w_hard.data_ptr(), cost.data_ptr(), sigma.data_ptr(), ws.data_ptr(),
                                       _nbytes(ws), _stream(w.device)))
    else:
        _check(abi.viterbi_tail_biting_v(w.data_ptr(), codebook.data_ptr(), B, n, L, k, V, tb_mode,
                                         states.data_ptr(), w_hard.data_ptr(), cost.data_ptr(), sigma.data_ptr(),
                                         ws.data_ptr(), _nbytes(ws), _stream(w.device)))
    return states, w_hard, cost, sigma


class _SoftQuantize(torch.autograd.Function):
    """w_soft = soft_codeword(w, c); dL/dw and dL/dc from the exact gradient kernels."""

    @staticmethod
    def forward(ctx, w, codebook, L, k, T, boundary_state, checkpoint):
        ctx.save_for_backward(w, codebook, boundary_state)
        ctx.params = (L, k, T, checkpoint)
        return soft_codeword(w, codebook, L, k, T, boundary_state, checkpoint=checkpoint)

    @staticmethod
    def backward(ctx, grad_w_soft):
        w, codebook, boundary_state = ctx.saved_tensors
        L, k, T, ck = ctx.params
        g = grad_w_soft.contiguous()
        grad_w = grad_c = None
        if ctx.needs_input_grad[1]:
            if ctx.needs_input_grad[0]:
                grad_c, grad_w = soft_codeword_grad_codebook(w, codebook, g, L, k, T, boundary_state, checkpoint=ck)
            else:
                grad_c = soft_codeword_grad_codebook(w, codebook, g, L, k, T, boundary_state, return_grad_w=False,
                                                     checkpoint=ck)
            grad_c = grad_c.to(codebook.dtype)
        elif ctx.needs_input_grad[0]:
            grad_w = soft_codeword_grad(w, codebook, g, L, k, T, boundary_state, checkpoint=ck)
        return grad_w, grad_c, None, None, None, None, None


def soft_quantize(w: torch.Tensor, codebook: torch.Tensor, L: int, k: int = 2, T: float = 1.0,
                  boundary_state: torch.Tensor | None = None, *, checkpoint: bool = False) -> torch.Tensor:
    """The soft codeword of w as a differentiable function of w and of the codebook ([2^L], or [2^L, V] with w
    [B, n V]); autograd runs the exact gradient kernels.  ``checkpoint`` runs the forward and backward calls with
    the smallest workspaces (checkpoint-and-recompute: about 2 sqrt(n) message rows per in-flight sequence)."""
    return _SoftQuantize.apply(w, codebook, L, k, T, boundary_state, checkpoint)
