"""Host-side checks of the C-ABI (no GPU needed): the library loads, exports every symbol include/bcjr.h declares,
reports status strings and workspace sizes, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

from differentiable_bcjr_amd import abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bcjr.h")

FAKE = 0x100000   # a non-NULL pointer value; every call below fails a host check before it could be used


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined", "if", "extern"})


def test_header_declares_every_op():
    fns = declared_functions()
    for name in ["bcjr_soft_codeword", "bcjr_soft_codeword_grad", "bcjr_soft_codeword_grad_codebook",
                 "viterbi_hard_code", "viterbi_tail_biting", "bcjr_soft_codeword_tail_biting",
                 "bcjr_soft_codeword_grad_tail_biting", "bcjr_soft_codeword_v", "bcjr_soft_codeword_grad_v",
                 "bcjr_soft_codeword_grad_codebook_v", "viterbi_hard_code_v", "bcjr_soft_codeword_tail_biting_v",
                 "bcjr_soft_codeword_grad_tail_biting_v", "viterbi_tail_biting_v", "bcjr_workspace_bytes_min",
                 "bcjr_workspace_bytes", "bcjr_workspace_bytes_v", "bcjr_status_string"]:
        assert name in fns


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(abi.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in bcjr.h but not exported"
    assert set(declared_functions()) == set(abi.EXPORTS)


def test_status_strings():
    for code in [abi.BCJR_OK, abi.BCJR_ERR_NULL, abi.BCJR_ERR_SHAPE, abi.BCJR_ERR_TEMP, abi.BCJR_ERR_UNSUPPORTED,
                 abi.BCJR_ERR_WORKSPACE, abi.BCJR_ERR_HIP]:
        s = abi.bcjr_status_string(code)
        assert s.startswith("BCJR")
    assert "unknown" in abi.bcjr_status_string(-99)


def _geo(L):
    G, Q = 1 << (L - 2), 1 << (L - 4)
    QPT = (1 << (L - 14)) if L >= 14 else 1
    TPS = Q // QPT
    NT = max(TPS, 64)
    return G, TPS, NT // TPS


def _wps(L):
    _, TPS, _ = _geo(L)
    return TPS // 64 if TPS >= 64 else 1


def _a256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("L", [4, 5, 8, 12, 14, 15, 16])
@pytest.mark.parametrize("B,n", [(1, 1), (16, 64), (4096, 256), (1000, 7)])
def test_workspace_bytes_formula(L, B, n):
    G, TPS, SPB = _geo(L)
    bpc = 1 if L >= 15 else (2 if L == 14 else 8)
    grid = min((B + SPB - 1) // SPB, 256 * bpc)
    slots = grid * SPB
    msgs = _a256((n + 1) * G * 4)
    nrm = _a256(n * 4)
    part = _a256(n * _wps(L) * 8) if _wps(L) > 1 else 0   # per-wave partial sums of every step
    assert abi.bcjr_workspace_bytes(abi.BCJR_OP_SOFT, B, n, L, 2) == slots * (msgs + nrm + part)
    part4 = _a256(n * _wps(L) * 16) if _wps(L) > 1 else 0
    assert abi.bcjr_workspace_bytes(abi.BCJR_OP_GRAD, B, n, L, 2) == slots * (2 * msgs + 2 * nrm + part4)
    acc = 3 * _a256((1 << L) * 4)   # per state one float accumulator and two pending contributions
    assert abi.bcjr_workspace_bytes(abi.BCJR_OP_GRAD_CODEBOOK, B, n, L, 2) == slots * (2 * msgs + 2 * nrm + part4 + acc)
    assert abi.bcjr_workspace_bytes(abi.BCJR_OP_VITERBI, B, n, L, 2) == slots * _a256(2 * n * TPS * 4)


def test_workspace_bytes_for_the_headline_workload():
    # 4096 sequences of 256 weights on a 2^16-state trellis: one 16 MiB forward tape per CU (+ 16 waves' partial sums)
    assert abi.bcjr_workspace_bytes(abi.BCJR_OP_SOFT, 4096, 256, 16, 2) == 256 * (257 * 65536 + 1024 + 256 * 16 * 8)


@pytest.mark.parametrize("args", [(0, 1, 8, 2), (-3, 1, 8, 2), (1, 0, 8, 2), (1, 4097, 8, 2), (1, 4, 3, 2),
                                  (1, 4, 17, 2), (1, 4, 8, 0), (1 << 31, 4, 8, 2)])
def test_workspace_bytes_invalid_shapes_are_zero(args):
    for op in (0, 1, 2, 3, 4, 5, 6, 7):
        assert abi.bcjr_workspace_bytes(op, *args) == 0
    assert abi.bcjr_workspace_bytes(99, 1, 4, 8, 2) == 0


def _gen_bytes(op, B, n, L, k, V, ckpt=0):
    """The general trellis kernels' workspace: one sequence per workgroup of 2^L / 64 threads (2^L below L = 6), a
    slot per workgroup of the persistent grid, G = 2^(L-k) message floats per LDS buffer.  ckpt > 0: the checkpoint
    mode (n / c + 1 checkpoint rows and c - 1 segment rows per message tape; the soft codeword saves one message and
    uses one LDS buffer, the gradients save two messages and keep the [n] per-step Q input offsets)."""
    S = 1 << L
    tps = S // min(S, 64)
    wps = tps // 64 if tps >= 64 else 1
    G = S >> k
    lds_cap, lds_static = 160 * 1024, 2048
    nsq = 1
    qg = 0
    if op in (abi.BCJR_OP_GRAD, abi.BCJR_OP_GRAD_CODEBOOK):
        # R~ and Q^ in LDS, or Q^ in a buffer of the slot when the two exceed it (k = 1 at L = 16)
        qg = 1 if 2 * G * 4 + lds_static > lds_cap and G * 4 + lds_static <= lds_cap else 0
        lds = G * 4 if qg else 2 * G * 4
    else:
        # Viterbi with V = 2 at L >= 12 decodes two sequences per workgroup (they share the codebook reads)
        if op == abi.BCJR_OP_VITERBI and V == 2 and L >= 12 and 2 * G * 4 + lds_static <= lds_cap:
            nsq = 2
        lds = nsq * (2 * G * 4 if (ckpt == 0 and nsq * 2 * G * 4 + lds_static <= lds_cap) else G * 4)
    if lds + lds_static > lds_cap:
        return 0
    bpc = max(1, min(16 // (tps // 64 if tps >= 64 else 1), lds_cap // (lds + lds_static)))
    grid = min(-(-B // nsq), 256 * bpc)
    tapes, nrm = _a256(((n + 1) if ckpt == 0 else (n // ckpt + ckpt)) * G * 4), _a256(n * 4)
    if op == abi.BCJR_OP_SOFT:
        slot = tapes + nrm + (_a256(n * wps * (1 + V) * 4) if wps > 1 else 0) + (_a256(G * 4) if ckpt else 0)
    elif op in (abi.BCJR_OP_GRAD, abi.BCJR_OP_GRAD_CODEBOOK):   # GC: + per state and component one float
        slot = 2 * tapes + 2 * nrm + (_a256(n * wps * (2 + 2 * V) * 4) if wps > 1 else 0)   # accumulator, two pending
        slot += 3 * _a256(S * V * 4) if op == abi.BCJR_OP_GRAD_CODEBOOK else 0
        slot += nrm + _a256(2 * G * 4) if ckpt else 0
        slot += _a256(G * 4) if qg else 0
    else:
        slot = _a256(2 * nsq * n * tps * 4)
    return grid * slot


@pytest.mark.parametrize("L,k", [(4, 1), (5, 2), (6, 3), (8, 4), (9, 1), (12, 3), (15, 1), (16, 1), (16, 3), (16, 4)])
@pytest.mark.parametrize("V", [1, 2])
@pytest.mark.parametrize("B,n", [(1, 1), (16, 64), (4096, 256), (1000, 7)])
def test_general_trellis_workspace_formula(L, k, V, B, n):
    for op in (abi.BCJR_OP_SOFT, abi.BCJR_OP_GRAD, abi.BCJR_OP_GRAD_CODEBOOK, abi.BCJR_OP_VITERBI):
        if (k, V) == (2, 1):
            continue
        assert abi.bcjr_workspace_bytes_v(op, B, n, L, k, V) == _gen_bytes(op, B, n, L, k, V)
        if V == 1:
            assert abi.bcjr_workspace_bytes(op, B, n, L, k) == _gen_bytes(op, B, n, L, k, V)


def _tuned_ck_bytes(op, B, n, L, c):
    """The k = 2 kernels in checkpoint mode: their slots (SPB sequences per block) hold n / c + c rows of each forward
    message, the [n] normalisers (and for the gradients the [n] Q offset sums), the per-wave partial sums of every
    step, (codebook gradient) one float accumulator per state, and then the checkpoint mode's own: the gradients' [n]
    Q input offsets, and each thread's share of the saved backward message(s)."""
    G, TPS, SPB = _geo(L)
    bpc = 1 if L >= 15 else (2 if L == 14 else 8)
    slots = min((B + SPB - 1) // SPB, 256 * bpc) * SPB
    rows, nrm = _a256((n // c + c) * G * 4), _a256(n * 4)
    if op == abi.BCJR_OP_SOFT:
        part = _a256(n * _wps(L) * 8) if _wps(L) > 1 else 0
        return slots * (rows + nrm + part + _a256(G * 4))
    part = _a256(n * _wps(L) * 16) if _wps(L) > 1 else 0
    acc = 3 * _a256((1 << L) * 4) if op == abi.BCJR_OP_GRAD_CODEBOOK else 0
    return slots * (2 * rows + 2 * nrm + part + acc + nrm + _a256(2 * G * 4))


@pytest.mark.parametrize("L,k,V", [(16, 2, 1), (16, 3, 1), (16, 4, 2), (16, 1, 1), (16, 1, 2), (12, 1, 2), (8, 2, 1),
                                   (4, 1, 1)])
@pytest.mark.parametrize("B,n", [(1, 1), (16, 2), (4096, 256), (100, 4096), (3, 17)])
def test_workspace_min_is_the_checkpoint_mode(L, k, V, B, n):
    """The smallest workspace of the soft codeword and the two gradients: checkpoints every c = ceil(sqrt(n)) rows,
    when that is smaller than the full tape; Viterbi has one memory mode."""
    c = 1
    while c * c < n:
        c += 1
    for op in (abi.BCJR_OP_SOFT, abi.BCJR_OP_GRAD, abi.BCJR_OP_GRAD_CODEBOOK):
        full = abi.bcjr_workspace_bytes_v(op, B, n, L, k, V)
        if (k, V) == (2, 1):
            ckb = _tuned_ck_bytes(op, B, n, L, c)   # the k = 2 kernels' own checkpoint mode
        else:
            ckb = _gen_bytes(op, B, n, L, k, V, ckpt=c)
        want = min(full, ckb) if full else 0
        assert abi.bcjr_workspace_bytes_min(op, B, n, L, k, V) == want
        if n >= 256 and L == 16 and full:   # the codebook gradient's three [2^L][V] arrays are not reduced
            factor = 6 if op != abi.BCJR_OP_GRAD_CODEBOOK else 3
            assert abi.bcjr_workspace_bytes_min(op, B, n, L, k, V) * factor < full
    # Viterbi and the tail-biting ops have one memory mode: their smallest workspace is the full one
    for op in (abi.BCJR_OP_VITERBI, abi.BCJR_OP_VITERBI_TB_EXACT, abi.BCJR_OP_VITERBI_TB_ROTATE,
               abi.BCJR_OP_SOFT_TAIL_BITING, abi.BCJR_OP_GRAD_TAIL_BITING):
        assert abi.bcjr_workspace_bytes_min(op, B, n, L, k, V) == abi.bcjr_workspace_bytes_v(op, B, n, L, k, V)


@pytest.mark.parametrize("L,k,V", [(8, 2, 1), (8, 1, 2), (10, 3, 1)])
def test_workspace_min_of_the_tail_biting_ops_runs_them(L, k, V):
    """The size bcjr_workspace_bytes_min gives a tail-biting op is one that op accepts (at B = 4, n = 64, L = 8 it
    was once a plain Viterbi slot, far smaller than the op needs)."""
    B, n = 4, 64
    for op in (abi.BCJR_OP_VITERBI_TB_EXACT, abi.BCJR_OP_VITERBI_TB_ROTATE, abi.BCJR_OP_SOFT_TAIL_BITING,
               abi.BCJR_OP_GRAD_TAIL_BITING):
        full = abi.bcjr_workspace_bytes_v(op, B, n, L, k, V)
        assert full > 0 and abi.bcjr_workspace_bytes_min(op, B, n, L, k, V) == full


def test_workspace_v_matches_the_scalar_query():
    for op in range(8):
        for L in (8, 16):
            assert abi.bcjr_workspace_bytes_v(op, 64, 32, L, 2, 1) == abi.bcjr_workspace_bytes(op, 64, 32, L, 2)


def test_unsupported_trellis_has_no_workspace():
    assert abi.bcjr_workspace_bytes(0, 4, 8, 10, 5) == 0                 # k > 4
    assert abi.bcjr_workspace_bytes_v(0, 4, 8, 8, 2, 3) == 0             # V > 2
    assert abi.bcjr_workspace_bytes_v(0, 4, 8, 8, 2, 0) == 0             # V < 1
    assert abi.bcjr_workspace_bytes(abi.BCJR_OP_GRAD, 4, 8, 16, 1) > 0   # k = 1, L = 16: Q^ in the workspace
    assert abi.bcjr_workspace_bytes(abi.BCJR_OP_GRAD_CODEBOOK, 4, 8, 16, 1) > 0
    assert abi.bcjr_workspace_bytes(abi.BCJR_OP_GRAD, 4, 8, 15, 1) > 0
    for op in (4, 6, 7):                                                 # exact tail-biting: L <= 10, any (k, V)
        assert abi.bcjr_workspace_bytes_v(op, 4, 8, 12, 3, 2) == 0
        assert abi.bcjr_workspace_bytes_v(op, 4, 8, 10, 3, 2) > 0
        assert abi.bcjr_workspace_bytes_v(op, 4, 8, 10, 5, 1) == 0       # k > 4
    assert abi.bcjr_workspace_bytes_v(5, 4, 8, 16, 4, 2) > 0             # rotate: any L


def _soft(**kw):
    a = dict(w=FAKE, codebook=FAKE, B=4, n=8, L=8, k=2, T=0.5, boundary_state=None, w_soft=FAKE, log_z=None,
             workspace=FAKE, workspace_bytes=0, stream=None)
    a.update(kw)
    return abi.bcjr_soft_codeword(*a.values())


def _grad(**kw):
    a = dict(w=FAKE, codebook=FAKE, B=4, n=8, L=8, k=2, T=0.5, boundary_state=None, grad_w_soft=FAKE,
             grad_w=FAKE, w_soft=None, workspace=FAKE, workspace_bytes=0, stream=None)
    a.update(kw)
    return abi.bcjr_soft_codeword_grad(*a.values())


def _gc(**kw):
    a = dict(w=FAKE, codebook=FAKE, B=4, n=8, L=8, k=2, T=0.5, boundary_state=None, grad_w_soft=FAKE,
             grad_codebook=FAKE, grad_w=None, w_soft=None, workspace=FAKE, workspace_bytes=0, stream=None)
    a.update(kw)
    return abi.bcjr_soft_codeword_grad_codebook(*a.values())


def _tb(**kw):
    a = dict(w=FAKE, codebook=FAKE, B=4, n=8, L=8, k=2, mode=abi.BCJR_TB_EXACT, states=FAKE, w_hard=None, cost=None,
             sigma=None, workspace=FAKE, workspace_bytes=0, stream=None)
    a.update(kw)
    return abi.viterbi_tail_biting(*a.values())


@pytest.mark.parametrize("L", [4, 8, 10, 12, 16])
@pytest.mark.parametrize("B,n", [(1, 1), (16, 64), (1000, 7)])
def test_tail_biting_workspace_formula(L, B, n):
    G, TPS, SPB = _geo(L)
    bpc = 1 if L >= 15 else (2 if L == 14 else 8)

    def slots(rows):
        return min((rows + SPB - 1) // SPB, 256 * bpc) * SPB

    vslot = _a256(2 * n * TPS * 4)
    rot = _a256(slots(B) * vslot) + _a256(B * n * 4) + _a256(B * 4)
    assert abi.bcjr_workspace_bytes(abi.BCJR_OP_VITERBI_TB_ROTATE, B, n, L, 2) == rot
    exact = abi.bcjr_workspace_bytes(abi.BCJR_OP_VITERBI_TB_EXACT, B, n, L, 2)
    if L <= 10:
        first = max(slots(B << L), slots(B)) * vslot
        assert exact == _a256(first) + _a256((B << L) * 4) + _a256(B * 4)
    else:
        assert exact == 0   # every one of 2^L start states would be decoded: refused above L = 10


@pytest.mark.parametrize("L", [4, 6, 8, 10, 12])
@pytest.mark.parametrize("B,n", [(1, 1), (16, 64), (33, 7)])
def test_tail_biting_measure_workspace_formula(L, B, n):
    G, TPS, SPB = _geo(L)
    bpc = 1 if L >= 15 else (2 if L == 14 else 8)
    V = B << L
    slots = min((V + SPB - 1) // SPB, 256 * bpc) * SPB
    msgs, nrm = _a256((n + 1) * G * 4), _a256(n * 4)
    soft_slot = msgs + nrm + (_a256(n * _wps(L) * 8) if _wps(L) > 1 else 0)
    grad_slot = 2 * msgs + 2 * nrm + (_a256(n * _wps(L) * 16) if _wps(L) > 1 else 0)
    soft = abi.bcjr_workspace_bytes(abi.BCJR_OP_SOFT_TAIL_BITING, B, n, L, 2)
    grad = abi.bcjr_workspace_bytes(abi.BCJR_OP_GRAD_TAIL_BITING, B, n, L, 2)
    if L > 10:
        assert soft == 0 and grad == 0
        return
    assert soft == _a256(slots * soft_slot) + _a256(V * n * 4) + _a256(V * 4)
    assert grad == _a256(slots * grad_slot) + _a256(V * n * 4) + _a256(V * 4) + _a256(V * n * 4)


@pytest.mark.parametrize("L,k,V", [(4, 1, 1), (6, 3, 2), (8, 4, 1), (10, 1, 2), (8, 2, 2), (12, 3, 1), (16, 4, 2)])
@pytest.mark.parametrize("B,n", [(1, 1), (16, 64), (33, 7)])
def test_general_tail_biting_workspace_formula(L, k, V, B, n):
    """The general kernels' plans: the Viterbi slots of the larger pass, then the per-(row, sigma) costs (exact) or
    the rotated pass's states, then sigma (and the rotated rows, rotate); the mixture: the soft (and gradient) slots of the B 2^L virtual
    sequences, then their soft codewords, ln Z (and gradients)."""
    vit_rows = _gen_bytes(abi.BCJR_OP_VITERBI, B, n, L, k, V)
    rot = _a256(vit_rows) + _a256(B * n * 4) + _a256(B * 4) + _a256(B * n * V * 4)   # + the rotated rows
    assert abi.bcjr_workspace_bytes_v(abi.BCJR_OP_VITERBI_TB_ROTATE, B, n, L, k, V) == rot
    exact = abi.bcjr_workspace_bytes_v(abi.BCJR_OP_VITERBI_TB_EXACT, B, n, L, k, V)
    soft = abi.bcjr_workspace_bytes_v(abi.BCJR_OP_SOFT_TAIL_BITING, B, n, L, k, V)
    grad = abi.bcjr_workspace_bytes_v(abi.BCJR_OP_GRAD_TAIL_BITING, B, n, L, k, V)
    if L > 10:
        assert exact == 0 and soft == 0 and grad == 0
        return
    S = B << L
    first = max(_gen_bytes(abi.BCJR_OP_VITERBI, S, n, L, k, V), vit_rows)
    assert exact == _a256(first) + _a256(S * 4) + _a256(B * 4)
    s_slots = _gen_bytes(abi.BCJR_OP_SOFT, S, n, L, k, V)
    g_slots = max(s_slots, _gen_bytes(abi.BCJR_OP_GRAD, S, n, L, k, V))
    assert soft == _a256(s_slots) + _a256(S * n * V * 4) + _a256(S * 4)
    assert grad == _a256(g_slots) + _a256(S * n * V * 4) + _a256(S * 4) + _a256(S * n * V * 4)


def test_tail_biting_measure_checks():
    def soft(**kw):
        a = dict(w=FAKE, codebook=FAKE, B=4, n=8, L=8, k=2, T=0.5, w_soft=FAKE, log_z=None, workspace=FAKE,
                 workspace_bytes=0, stream=None)
        a.update(kw)
        return abi.bcjr_soft_codeword_tail_biting(*a.values())

    def grad(**kw):
        a = dict(w=FAKE, codebook=FAKE, B=4, n=8, L=8, k=2, T=0.5, grad_w_soft=FAKE, grad_w=FAKE, w_soft=None,
                 workspace=FAKE, workspace_bytes=0, stream=None)
        a.update(kw)
        return abi.bcjr_soft_codeword_grad_tail_biting(*a.values())

    assert soft(w_soft=None) == abi.BCJR_ERR_NULL and grad(grad_w=None) == abi.BCJR_ERR_NULL
    assert grad(grad_w_soft=None) == abi.BCJR_ERR_NULL
    assert soft(n=0) == abi.BCJR_ERR_SHAPE and grad(B=0) == abi.BCJR_ERR_SHAPE
    assert soft(T=0.0) == abi.BCJR_ERR_TEMP and grad(T=float("nan")) == abi.BCJR_ERR_TEMP
    assert soft(L=12) == abi.BCJR_ERR_UNSUPPORTED and grad(L=11) == abi.BCJR_ERR_UNSUPPORTED
    assert soft(L=10, k=5) == abi.BCJR_ERR_UNSUPPORTED and grad(L=10, k=5) == abi.BCJR_ERR_UNSUPPORTED
    assert soft(k=1) == abi.BCJR_ERR_WORKSPACE and grad(k=3) == abi.BCJR_ERR_WORKSPACE   # the general kernels
    need = abi.bcjr_workspace_bytes(abi.BCJR_OP_SOFT_TAIL_BITING, 4, 8, 8, 2)
    assert soft(workspace_bytes=need - 1) == abi.BCJR_ERR_WORKSPACE
    assert soft(workspace=FAKE + 8, workspace_bytes=need) == abi.BCJR_ERR_WORKSPACE
    needg = abi.bcjr_workspace_bytes(abi.BCJR_OP_GRAD_TAIL_BITING, 4, 8, 8, 2)
    assert needg > need and grad(workspace_bytes=needg - 1) == abi.BCJR_ERR_WORKSPACE


def test_tail_biting_checks():
    assert _tb(states=None) == abi.BCJR_ERR_NULL
    assert _tb(w=None) == abi.BCJR_ERR_NULL
    assert _tb(n=0) == abi.BCJR_ERR_SHAPE
    assert _tb(k=1) == abi.BCJR_ERR_WORKSPACE and _tb(k=4) == abi.BCJR_ERR_WORKSPACE   # the general kernels
    assert _tb(L=10, k=5) == abi.BCJR_ERR_UNSUPPORTED
    assert _tb(mode=7) == abi.BCJR_ERR_UNSUPPORTED
    assert _tb(L=12) == abi.BCJR_ERR_UNSUPPORTED                       # exact above L = 10
    assert _tb(L=12, mode=abi.BCJR_TB_ROTATE) == abi.BCJR_ERR_WORKSPACE   # rotate has no L limit
    need = abi.bcjr_workspace_bytes(abi.BCJR_OP_VITERBI_TB_EXACT, 4, 8, 8, 2)
    assert _tb(workspace_bytes=need - 1) == abi.BCJR_ERR_WORKSPACE
    assert _tb(workspace=FAKE + 32, workspace_bytes=need) == abi.BCJR_ERR_WORKSPACE
    assert _tb(workspace=None, workspace_bytes=need) == abi.BCJR_ERR_WORKSPACE


def _vit(**kw):
    a = dict(w=FAKE, codebook=FAKE, B=4, n=8, L=8, k=2, boundary_state=None, states=FAKE, w_hard=None, cost=None,
             workspace=FAKE, workspace_bytes=0, stream=None)
    a.update(kw)
    return abi.viterbi_hard_code(*a.values())


def test_null_pointers_rejected():
    assert _soft(w=None) == abi.BCJR_ERR_NULL
    assert _soft(codebook=None) == abi.BCJR_ERR_NULL
    assert _soft(w_soft=None) == abi.BCJR_ERR_NULL
    assert _grad(grad_w_soft=None) == abi.BCJR_ERR_NULL
    assert _grad(grad_w=None) == abi.BCJR_ERR_NULL
    assert _gc(grad_codebook=None) == abi.BCJR_ERR_NULL
    assert _gc(grad_w_soft=None) == abi.BCJR_ERR_NULL
    assert _gc(w=None) == abi.BCJR_ERR_NULL
    # grad_w and w_soft are optional for the codebook gradient: with them NULL the next check is the workspace
    assert _gc() == abi.BCJR_ERR_WORKSPACE
    assert _vit(states=None) == abi.BCJR_ERR_NULL
    assert _vit(codebook=None) == abi.BCJR_ERR_NULL


@pytest.mark.parametrize("kw", [dict(B=0), dict(n=0), dict(n=4097), dict(L=3), dict(L=17), dict(k=0), dict(L=4, k=3)])
def test_bad_shapes_rejected(kw):
    assert _soft(**kw) == abi.BCJR_ERR_SHAPE
    assert _grad(**kw) == abi.BCJR_ERR_SHAPE
    assert _gc(**kw) == abi.BCJR_ERR_SHAPE
    assert _vit(**kw) == abi.BCJR_ERR_SHAPE


def _soft_v(**kw):
    a = dict(w=FAKE, codebook=FAKE, B=4, n=8, L=8, k=2, V=2, T=0.5, boundary_state=None, w_soft=FAKE, log_z=None,
             workspace=FAKE, workspace_bytes=0, stream=None)
    a.update(kw)
    return abi.bcjr_soft_codeword_v(*a.values())


def _grad_v(**kw):
    a = dict(w=FAKE, codebook=FAKE, B=4, n=8, L=8, k=2, V=2, T=0.5, boundary_state=None, grad_w_soft=FAKE,
             grad_w=FAKE, w_soft=None, workspace=FAKE, workspace_bytes=0, stream=None)
    a.update(kw)
    return abi.bcjr_soft_codeword_grad_v(*a.values())


def _gc_v(**kw):
    a = dict(w=FAKE, codebook=FAKE, B=4, n=8, L=8, k=2, V=2, T=0.5, boundary_state=None, grad_w_soft=FAKE,
             grad_codebook=FAKE, grad_w=None, w_soft=None, workspace=FAKE, workspace_bytes=0, stream=None)
    a.update(kw)
    return abi.bcjr_soft_codeword_grad_codebook_v(*a.values())


def _vit_v(**kw):
    a = dict(w=FAKE, codebook=FAKE, B=4, n=8, L=8, k=2, V=2, boundary_state=None, states=FAKE, w_hard=None,
             cost=None, workspace=FAKE, workspace_bytes=0, stream=None)
    a.update(kw)
    return abi.viterbi_hard_code_v(*a.values())


def test_unsupported_trellis_rejected():
    assert _soft(L=10, k=5) == abi.BCJR_ERR_UNSUPPORTED
    assert _grad(L=12, k=6) == abi.BCJR_ERR_UNSUPPORTED
    assert _vit(L=10, k=5) == abi.BCJR_ERR_UNSUPPORTED
    assert _gc(L=10, k=5) == abi.BCJR_ERR_UNSUPPORTED
    assert _grad(L=16, k=1) == abi.BCJR_ERR_WORKSPACE                   # Q^ in the workspace at k = 1, L = 16
    assert _gc(L=16, k=1) == abi.BCJR_ERR_WORKSPACE
    for fn in (_soft_v, _grad_v, _gc_v, _vit_v):
        assert fn(V=3) == abi.BCJR_ERR_UNSUPPORTED
        assert fn(V=0) == abi.BCJR_ERR_SHAPE
        assert fn(V=-1) == abi.BCJR_ERR_SHAPE


def test_general_trellis_reaches_the_workspace_check():
    # k = 1, 3, 4 and V = 2 have kernels: with no workspace the call stops at the workspace check
    for L, k in ((8, 1), (9, 3), (8, 4), (16, 4)):
        assert _soft(L=L, k=k) == abi.BCJR_ERR_WORKSPACE
        assert _grad(L=L, k=k) == abi.BCJR_ERR_WORKSPACE
        assert _vit(L=L, k=k) == abi.BCJR_ERR_WORKSPACE
        assert _gc(L=L, k=k) == abi.BCJR_ERR_WORKSPACE
        for V in (1, 2):
            assert _gc_v(L=L, k=k, V=V) == abi.BCJR_ERR_WORKSPACE
            assert _soft_v(L=L, k=k, V=V) == abi.BCJR_ERR_WORKSPACE
            assert _grad_v(L=L, k=k, V=V) == abi.BCJR_ERR_WORKSPACE
            assert _vit_v(L=L, k=k, V=V) == abi.BCJR_ERR_WORKSPACE
    need = abi.bcjr_workspace_bytes_min(abi.BCJR_OP_SOFT, 4, 8, 9, 3, 2)   # below it no memory mode fits
    assert _soft_v(L=9, k=3, workspace_bytes=need - 1) == abi.BCJR_ERR_WORKSPACE
    assert _soft_v(L=9, k=3, workspace=FAKE + 16, workspace_bytes=need) == abi.BCJR_ERR_WORKSPACE


@pytest.mark.parametrize("L,k", [(2, 1), (3, 1)])
def test_trellis_below_four_state_bits_rejected(L, k):
    """L < 4 is refused for every k (the kernels give every thread at least 16 states): each entry point returns
    BCJR_ERR_SHAPE before anything else, and every workspace query returns 0."""
    for fn in (_soft, _grad, _gc, _vit):
        assert fn(L=L, k=k) == abi.BCJR_ERR_SHAPE
    for fn in (_soft_v, _grad_v, _gc_v, _vit_v):
        for V in (1, 2):
            assert fn(L=L, k=k, V=V) == abi.BCJR_ERR_SHAPE
    assert _tb(L=L, k=k) == abi.BCJR_ERR_SHAPE and _tb(L=L, k=k, mode=abi.BCJR_TB_ROTATE) == abi.BCJR_ERR_SHAPE
    a = [FAKE, FAKE, 4, 8, L, k, 0.5]
    assert abi.bcjr_soft_codeword_tail_biting(*a, FAKE, None, FAKE, 1 << 30, None) == abi.BCJR_ERR_SHAPE
    assert abi.bcjr_soft_codeword_grad_tail_biting(*a, FAKE, FAKE, None, FAKE, 1 << 30, None) == abi.BCJR_ERR_SHAPE
    assert abi.bcjr_soft_codeword_noalloc(*a, None, FAKE, None, None) == abi.BCJR_ERR_SHAPE
    for op in range(8):
        for V in (1, 2):
            assert abi.bcjr_workspace_bytes_v(op, 4, 8, L, k, V) == 0
            assert abi.bcjr_workspace_bytes_min(op, 4, 8, L, k, V) == 0
        assert abi.bcjr_workspace_bytes(op, 4, 8, L, k) == 0


def _noalloc(**kw):
    a = dict(w=FAKE, codebook=FAKE, B=4, n=8, L=8, k=2, T=0.5, boundary_state=None, w_soft=FAKE, log_z=None,
             stream=None)
    a.update(kw)
    return abi.bcjr_soft_codeword_noalloc(*a.values())


def test_noalloc_entry_point_checks_on_the_host():
    """The allocation-free soft codeword runs the soft codeword's checks, in the same order, before it touches the
    device (the scratch address is looked up only for a valid call)."""
    assert abi.BCJR_NOALLOC_SCRATCH_BYTES == 256 << 20
    assert _noalloc(w=None) == abi.BCJR_ERR_NULL
    assert _noalloc(codebook=None) == abi.BCJR_ERR_NULL
    assert _noalloc(w_soft=None) == abi.BCJR_ERR_NULL
    for kw in (dict(B=0), dict(n=4097), dict(L=17), dict(L=3), dict(k=0)):
        assert _noalloc(**kw) == abi.BCJR_ERR_SHAPE
    assert _noalloc(L=10, k=5) == abi.BCJR_ERR_UNSUPPORTED
    for T in (0.0, float("nan"), 1e-13):
        assert _noalloc(T=T) == abi.BCJR_ERR_TEMP
    assert _noalloc(w=None, B=0, T=-1.0) == abi.BCJR_ERR_NULL
    assert _noalloc(B=0, T=-1.0) == abi.BCJR_ERR_SHAPE


def test_python_wrapper_checks_a_callers_workspace():
    """A caller's workspace must be a contiguous device tensor on the weights' device; a host tensor would hand the
    kernels a host pointer."""
    import torch

    import differentiable_bcjr_amd as dba

    for ws in (torch.empty(1 << 12, dtype=torch.uint8), object()):
        with pytest.raises(TypeError):
            dba._workspace(abi.BCJR_OP_SOFT, 2, 8, 8, 2, torch.device("cuda:0"), ws)


@pytest.mark.parametrize("kw", [dict(B=0), dict(n=0), dict(n=4097), dict(L=3), dict(L=17), dict(k=0), dict(L=5, k=3)])
def test_bad_shapes_rejected_v(kw):
    assert _gc_v(**kw) == abi.BCJR_ERR_SHAPE
    assert _soft_v(**kw) == abi.BCJR_ERR_SHAPE
    assert _grad_v(**kw) == abi.BCJR_ERR_SHAPE
    assert _vit_v(**kw) == abi.BCJR_ERR_SHAPE


@pytest.mark.parametrize("T", [0.0, -1.0, float("nan"), float("inf"), 1e-13])
def test_bad_temperature_rejected(T):
    assert _soft(T=T) == abi.BCJR_ERR_TEMP
    assert _grad(T=T) == abi.BCJR_ERR_TEMP
    assert _gc(T=T) == abi.BCJR_ERR_TEMP


def test_viterbi_ignores_temperature_and_checks_workspace():
    need = abi.bcjr_workspace_bytes(abi.BCJR_OP_VITERBI, 4, 8, 8, 2)
    assert _vit(workspace_bytes=need - 1) == abi.BCJR_ERR_WORKSPACE
    assert _vit(workspace=None, workspace_bytes=need) == abi.BCJR_ERR_WORKSPACE
    assert _vit(workspace=FAKE + 16, workspace_bytes=need) == abi.BCJR_ERR_WORKSPACE


def test_workspace_too_small_or_misaligned_rejected():
    need = abi.bcjr_workspace_bytes_min(abi.BCJR_OP_SOFT, 4, 8, 8, 2, 1)   # the checkpoint mode's size
    assert need < abi.bcjr_workspace_bytes(abi.BCJR_OP_SOFT, 4, 8, 8, 2)
    assert _soft(workspace_bytes=need - 1) == abi.BCJR_ERR_WORKSPACE
    assert _soft(workspace=None, workspace_bytes=need) == abi.BCJR_ERR_WORKSPACE
    assert _soft(workspace=FAKE + 64, workspace_bytes=need) == abi.BCJR_ERR_WORKSPACE
    needg = abi.bcjr_workspace_bytes_min(abi.BCJR_OP_GRAD, 4, 8, 8, 2, 1)   # the checkpoint mode's sizes
    assert needg < abi.bcjr_workspace_bytes(abi.BCJR_OP_GRAD, 4, 8, 8, 2)
    assert _grad(workspace_bytes=needg - 1) == abi.BCJR_ERR_WORKSPACE
    needc = abi.bcjr_workspace_bytes_min(abi.BCJR_OP_GRAD_CODEBOOK, 4, 8, 8, 2, 1)
    assert needc > needg
    assert _gc(workspace_bytes=needg) == abi.BCJR_ERR_WORKSPACE   # the gradient's workspace is not enough
    assert _gc(workspace_bytes=needc - 1) == abi.BCJR_ERR_WORKSPACE
    assert _gc(workspace=FAKE + 128, workspace_bytes=needc) == abi.BCJR_ERR_WORKSPACE


def test_checks_precede_each_other_in_documented_order():
    # NULL before shape before temperature before workspace
    assert _soft(w=None, B=0, T=-1.0) == abi.BCJR_ERR_NULL
    assert _soft(B=0, T=-1.0) == abi.BCJR_ERR_SHAPE
    assert _soft(T=-1.0, workspace=None) == abi.BCJR_ERR_TEMP


def test_python_wrapper_refuses_cpu_tensors():
    import torch

    import differentiable_bcjr_amd as dba

    w = torch.zeros(2, 4)
    c = torch.zeros(256)
    with pytest.raises(TypeError):
        dba.soft_codeword(w, c, 8)
    with pytest.raises(TypeError):
        dba.viterbi_hard_code(w, c, 8)
    with pytest.raises(TypeError):
        dba.soft_codeword_grad_codebook(w, c, w, 8)
    with pytest.raises(TypeError):
        dba.viterbi_tail_biting(w, c, 8)
    with pytest.raises(ValueError):
        dba.viterbi_tail_biting(w.cuda() if torch.cuda.is_available() else w, c, 8, mode="nearest")


def test_largest_shape_keeps_workspace_offsets_in_32_bits():
    # the kernels address one block's slots with 32-bit buffer offsets
    for op in (abi.BCJR_OP_SOFT, abi.BCJR_OP_GRAD, abi.BCJR_OP_VITERBI, abi.BCJR_OP_GRAD_CODEBOOK,
               abi.BCJR_OP_VITERBI_TB_ROTATE):
        for L in (8, 12, 16):
            G, TPS, SPB = _geo(L)
            per_block = abi.bcjr_workspace_bytes(op, SPB, 4096, L, 2)
            assert 0 < per_block < 2 ** 31
    # the general trellis: one sequence per block
    for op in (abi.BCJR_OP_SOFT, abi.BCJR_OP_GRAD, abi.BCJR_OP_GRAD_CODEBOOK, abi.BCJR_OP_VITERBI):
        for L, k in ((16, 1), (15, 1), (16, 3), (16, 4), (8, 1)):
            for V in (1, 2):
                per_block = abi.bcjr_workspace_bytes_v(op, 1, 4096, L, k, V)
                assert per_block < 2 ** 31
                assert per_block > 0
