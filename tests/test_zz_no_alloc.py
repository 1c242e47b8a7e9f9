"""The allocation-free soft codeword, bcjr_soft_codeword_noalloc, called through the C-ABI.

It must give what bcjr_soft_codeword gives with a caller-owned workspace of the same memory mode (the full tape when
every workgroup's tape fits in the static scratch, else the checkpoint mode with fewer workgroups), bit for bit, and
stay within the parity bars of tests/parity.py against the oracle.  Each pair runs two calls in a row on the shared
scratch, the second smaller, so the second call starts from the first call's leftovers.  The file is named to be
collected last: it passes alone in a fresh process and after every other GPU test.
"""
import numpy as np
import pytest
import torch

import parity
from differentiable_bcjr_amd import abi

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def _inputs(L, B, n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    c = rng.standard_normal(1 << L)
    c = (c / c.std()).astype(np.float32)
    w = rng.standard_normal((B, n)).astype(np.float32)
    s = rng.integers(0, 1 << L, size=B).astype(np.int32)
    return w, c, s


def _noalloc(wt, ct, L, T, st, stream):
    B, n = wt.shape
    out = torch.full_like(wt, float("nan"))
    lz = torch.full((B,), float("nan"), dtype=torch.float32, device=wt.device)
    rc = abi.bcjr_soft_codeword_noalloc(wt.data_ptr(), ct.data_ptr(), B, n, L, 2, T,
                                        None if st is None else st.data_ptr(), out.data_ptr(), lz.data_ptr(),
                                        stream.cuda_stream)
    assert rc == abi.BCJR_OK, abi.bcjr_status_string(rc)
    return out, lz


def _with_workspace(wt, ct, L, T, st, stream):
    """bcjr_soft_codeword with a workspace of the mode the scratch runs: the full tape when the whole grid's tape fits
    in the scratch, else the checkpoint mode."""
    B, n = wt.shape
    full = abi.bcjr_workspace_bytes(abi.BCJR_OP_SOFT, B, n, L, 2)
    need = full if full <= abi.BCJR_NOALLOC_SCRATCH_BYTES else abi.bcjr_workspace_bytes_min(abi.BCJR_OP_SOFT, B, n,
                                                                                           L, 2, 1)
    ws = torch.empty(need, dtype=torch.uint8, device=wt.device)
    out = torch.empty_like(wt)
    lz = torch.empty(B, dtype=torch.float32, device=wt.device)
    rc = abi.bcjr_soft_codeword(wt.data_ptr(), ct.data_ptr(), B, n, L, 2, T, None if st is None else st.data_ptr(),
                                out.data_ptr(), lz.data_ptr(), ws.data_ptr(), need, stream.cuda_stream)
    assert rc == abi.BCJR_OK, abi.bcjr_status_string(rc)
    return out, lz, need < full


# (L, B, n, sigma) of the first call, then of the second, smaller call
PAIRS = [
    # L = 16, n = 256: the full tape (4.3 GB) does not fit, so checkpoints on the 122 workgroups whose slots fit, each
    # decoding up to three sequences
    ((16, 300, 256, False), (16, 5, 40, False)),
    # L = 10: the full tape of the whole grid fits, so the tuned kernel with its full tape
    ((10, 3000, 64, True), (10, 9, 13, False)),
]


@pytest.mark.parametrize("first,second", PAIRS, ids=["L16-checkpoint", "L10-full-tape"])
def test_noalloc_matches_the_workspace_entry_point(oracle_mod, dev, first, second):
    stream = torch.cuda.current_stream(dev)
    for call, (L, B, n, sigma) in enumerate((first, second)):
        T = 0.1
        w, c, s = _inputs(L, B, n, 6100 + 10 * L + call)
        s = s if sigma else None
        wt, ct = torch.from_numpy(w).to(dev), torch.from_numpy(c).to(dev)
        st = None if s is None else torch.from_numpy(s).to(dev)
        print(f"noalloc call {call}: L={L} B={B} n={n} sigma={sigma}", flush=True)
        got, lz = _noalloc(wt, ct, L, T, st, stream)
        ref, rlz, ckpt = _with_workspace(wt, ct, L, T, st, stream)
        torch.cuda.synchronize()
        assert ckpt == (L == 16 and n == 256)
        assert torch.equal(got, ref), "the scratch and the caller's workspace gave different soft codewords"
        assert torch.equal(lz, rlz)
        rows = np.unique(np.array([0, B // 2, B - 1]))
        print(f"  rows {rows.tolist()} against the oracle:", flush=True)
        assert parity.soft_ok(oracle_mod, got, lz, w, c, L, 2, T, s, rows=rows)
