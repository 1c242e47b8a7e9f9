#!/usr/bin/env python3
"""Throughput of the BCJR soft-quantizer hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic weights, inputs resident in HBM:

  1. bcjr_soft_codeword       temperature-T forward-backward over the bitshift trellis -> soft codeword, ln Z
  2. bcjr_soft_codeword_grad  the exact gradient w.r.t. the weights (expectation semiring), upstream grad ~ N(0,1)
  3. viterbi_hard_code        the T -> 0 limit: minimum-energy path, its codeword and cost

(BCJR-QAT, arXiv 2605.10655: abstract; gist.science Technical Summary, "Core Mechanism" and "Key Technical
Innovations".)  The default workload is a 1024x1024 Gaussian matrix cut into 4096 sequences of 256 weights on the
L = 16, k = 2 trellis (65536 states), T = 0.1, free boundary.

Counting.  A state-update is one trellis state at one step in one direction: the soft and gradient passes do
2 * B * n * 2^L each (forward and backward), Viterbi B * n * 2^L (its traceback touches one state per step).
``value`` is the step's state-updates per second; ``weights_per_s`` is B * n per step time.

The roofline object covers the step's longest kernel.  Its bound is VALU issue: the work per state-step is counted in
full-rate fp32 VALU lane slots (a half-rate max/compare/select costs 2, a quarter-rate exp2/log2/rcp 4), and the peak is
256 CUs x 128 fp32 lanes x 2.4 GHz = 78.6e12 slots/s (the published 157.3 TFLOP/s fp32 vector rate with an FMA as
two flops).  Kernel times come from HIP events recorded on the stream the kernels run on.  Its ``hbm_view`` puts the
same kernel's counter-measured HBM bytes (the message tape) over its time against a plain 1 GiB device copy timed in
the same run: the gradient kernel's forward pass writes its tape near that rate.

After the timed steps, and outside them, the codebook gradient (bcjr_soft_codeword_grad_codebook, the exact dL/dc
summed over the batch) is timed on the same inputs and reported under ``next_rows`` with its own roofline.  Its bound
is HBM: besides the 4 bytes of forward tape per state-step (written once, read once), every state's float32
accumulator is read and written once per step, 12 bytes per state-step against the 8 TB/s peak.  The tail-biting
Viterbi with rotate-and-decode start-state choice (viterbi_tail_biting, two decodes) is timed the same way, and so
are the general-trellis kernels on the same 1024x1024 matrix at 3 bits per weight (k = 3) and at 2 bits per weight with
two weights per step (k = 4, V = 2): soft codeword, gradient and Viterbi, each against the ALU roofline of its own
slot count (general_slots).  The soft codeword and the gradient are also timed in their checkpoint-and-recompute
memory mode (given bcjr_workspace_bytes_min: every ceil(sqrt(n))-th message row kept, the rest rebuilt per segment),
with the workspace that mode needs beside the full tape's (at k = 2 the tuned kernels' own checkpoint mode).

``--gpus N`` with N > 1 exits: the path runs on one GPU (sequences are independent; sharding B needs no exchange).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Algorithmic VALU work per state-step (one state, one step), in fp32 lane slots of a full-rate instruction
# (add, mul, fma).  Measured on gfx950: max/min/compare/select issue at half that rate (2 slots), exp2/log2/rcp at a
# quarter (4 slots).  Per-state counts of the grouped-message form (one log-sum-exp of 4 per group of 4 states):
#   soft    forward 4.25 full + 1 half + 1.25 trans; backward the same; posterior 2 full + 0.25 trans
#           -> 10.5 full + 2 half + 2.75 trans = 25.5 slots
#   grad    forward 6.5 full + 1 half + 1.5 trans (adds the Q message); backward 13 full + 1 half + 1.75 trans
#           (adds the P message and the four covariance sums) -> 19.5 full + 2 half + 3.25 trans = 36.5 slots
#   viterbi sub, mul, add, 0.5 back-pointer packing (full) + 2.25 compare/select for the min of 4 with its index
#           -> 3.5 full + 2.25 half = 8 slots
HALF_SLOTS, TRANS_SLOTS = 2.0, 4.0
ALU_SLOTS = {
    "soft": 10.5 + 2.0 * HALF_SLOTS + 2.75 * TRANS_SLOTS,
    "grad": 19.5 + 2.0 * HALF_SLOTS + 3.25 * TRANS_SLOTS,
    "viterbi": 3.5 + 2.25 * HALF_SLOTS,
}
DIRECTIONS = {"soft": 2, "grad": 2, "viterbi": 1}
# The flat planning count of the same work: every VALU instruction one slot whatever its issue rate, a transcendental
# four: soft about 11 VALU + 2.75 transcendentals, grad 17 + 3.25, Viterbi 5.5 + 0 per state-step.  The line reports
# the fraction of the peak under both counts; the issue-rate-weighted one above is the primary (``frac``).
FLAT_SLOTS = {"soft": 11.0 + 2.75 * TRANS_SLOTS, "grad": 17.0 + 3.25 * TRANS_SLOTS, "viterbi": 5.5}


def general_slots(k: int, V: int) -> dict:
    """The same counts for P = 2^k predecessors (and successors) per group and V weights per step: one log-sum-exp of
    P per group, a squared distance of V components per state.  At k = 2, V = 1 they are the counts above.
      soft     full 5V + 2(2P+1)/P + (3+V)/P, half 2, trans (2P+3)/P
      grad     full 3V + 1 + (2P+2)/P (forward) + 6V + 5 + (6+2V)/P (backward), half 2, trans (P+2)/P + 1 + 3/P
      viterbi  full 3V + 0.5, half 2.25"""
    P = 2 ** k
    return {
        "soft": 5 * V + 2 * (2 * P + 1) / P + (3 + V) / P + 2.0 * HALF_SLOTS + (2 * P + 3) / P * TRANS_SLOTS,
        "grad": (3 * V + 1 + (2 * P + 2) / P + 6 * V + 5 + (6 + 2 * V) / P + 2.0 * HALF_SLOTS
                 + ((P + 2) / P + 1 + 3 / P) * TRANS_SLOTS),
        "viterbi": 3 * V + 0.5 + 2.25 * HALF_SLOTS,
    }

PEAK_SLOTS_PER_S = 256 * 128 * 2.4e9
KERNEL_SOURCES = {
    "soft": ["soft.hip"],
    "grad": ["grad.hip"],
    "viterbi": ["viterbi.hip"],
    "grad_codebook": ["grad.hip"],
}
KERNEL_SOURCES.update({f"gen_{op}_k{k}v{V}": ["general.hip"] for op in ("soft", "grad", "viterbi")
                       for k, V in ((3, 1), (4, 2))})
COMMON_SOURCES = ["trellis.hpp", "kernel_args.hpp"]
# the kernels' template names as the profiler lists them: soft_kernel<L, checkpoint>, grad_kernel<L, codebook-gradient
# mode, checkpoint>, viterbi_kernel<L>
KERNEL_NAMES = {"soft": "soft_kernel<16, false>", "grad": "grad_kernel<16, 0, false>",
                "viterbi": "viterbi_kernel<16>", "grad_codebook": "grad_kernel<16, 1, false>"}
CHECKPOINT_KERNELS = {"soft": "soft_kernel<16, true>", "grad": "grad_kernel<16, 0, true>"}
# HBM bytes per state-step of the codebook gradient: forward tape R~ and Q^ (one float per group each, i.e. 2 bytes
# per state, written by the forward pass and read by the backward pass) + the per-state accumulator (4 bytes read
# and 4 written per step)
CODEBOOK_GRAD_BYTES = 2 * 2.0 + 8.0
HBM_PEAK_GBS = 8000.0


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=2, choices=[2, 3, 4, 5],
                    help="synthetic workload (2: 1024x1024 matrix, 3: 8192x2048, 4: 2048x2048, 5: whole layer)")
    ap.add_argument("--temperature", type=float, default=0.1)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the CPU oracle")
    ap.add_argument("--codebook-grad-steps", type=int, default=3,
                    help="calls of the codebook gradient (and of the tail-biting Viterbi) timed after the step "
                         "(0 skips them)")
    ap.add_argument("--trellis-variant-steps", type=int, default=2,
                    help="calls of each op on the 1024x1024 matrix at k = 3 and at k = 4 with V = 2, timed after the "
                         "step (0 skips them)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (reference dispatch for HBM byte counters)")
    return ap.parse_args()


def viterbi_pairs(L: int, k: int, V: int) -> int:
    """Sequences per workgroup of the general Viterbi kernel: 2 where the codebook is read from memory (V = 2,
    L >= 12) and two message arrays fit in LDS, as the library's plan chooses."""
    return 2 if V == 2 and L >= 12 and 2 * (4 << (L - k)) + 2048 <= 160 * 1024 else 1


def device_copy_rate(dev, stream, reps: int = 5) -> float:
    """GB/s of read plus write traffic of a plain 1 GiB device-to-device copy, timed with events on `stream`."""
    import torch

    src = torch.empty((1 << 28,), dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2.0 * (1 << 30) / (ms * 1e-3) / 1e9


def source_digest(op: str) -> str:
    """Digest of a kernel's sources with comments and whitespace removed (comment edits keep counters valid)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "differentiable_bcjr_amd", "csrc")
    for f in KERNEL_SOURCES[op] + COMMON_SOURCES:
        with open(os.path.join(csrc, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(op: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{op}_kernel_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.startswith("- "):
                key, val = line[2:].split(":", 1)
                fields[key.strip()] = val.strip().strip("`")
    if fields.get("source_sha256") != source_digest(op):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, T, n_rows_per_thread=4):
    """The oracle (plain fp64 C, OpenMP over sequences) on a bounded sample of the same workload and step."""
    import numpy as np

    import oracle

    oracle.build(force=False)
    threads = oracle.num_threads()
    rows = wl.sample_rows(max(4, n_rows_per_thread * threads))
    c = wl.codebook()
    w = wl.weights()[rows]
    g = wl.upstream_grad()[rows]
    t0 = time.perf_counter()
    oracle.soft(w, c, wl.L, wl.k, T)
    oracle.grad(w, c, g, wl.L, wl.k, T)
    oracle.viterbi(w, c, wl.L, wl.k)
    dt = time.perf_counter() - t0
    S = 1 << wl.L
    upd = sum(DIRECTIONS.values()) * len(rows) * wl.n * S
    return {"value": upd / dt, "unit": "state-updates/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(rows)} of the {wl.B} sequences (rows 0 and B-1 included, seed {4000 + wl.cfg}), "
                      f"one full step (soft + grad + viterbi), {dt:.1f} s, weights/s {len(rows) * wl.n / dt:.3g}",
            "weights_per_s": len(rows) * wl.n / dt}


def time_variant(vw, T, K, dev, stream, check):
    """Soft codeword, gradient and Viterbi of one trellis variant of a workload, each timed over K calls with HIP
    events on the launch stream, with the ALU roofline of each kernel."""
    import numpy as np
    import torch

    from differentiable_bcjr_amd import abi

    S, steps, V, k, L, B = 1 << vw.L, vw.steps, vw.V, vw.k, vw.L, vw.B
    c = torch.from_numpy(vw.codebook()).to(dev)
    w = torch.from_numpy(vw.weights()).to(dev)
    g = torch.from_numpy(vw.upstream_grad()).to(dev)
    out = torch.empty_like(w)
    grad = torch.empty_like(w)
    states = torch.empty((B, steps), dtype=torch.int32, device=dev)
    w_hard = torch.empty_like(w)
    cost = torch.empty((B,), dtype=torch.float32, device=dev)
    nbytes = max(abi.bcjr_workspace_bytes_v(op, B, steps, L, k, V)
                 for op in (abi.BCJR_OP_SOFT, abi.BCJR_OP_GRAD, abi.BCJR_OP_VITERBI))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sp = stream.cuda_stream
    calls = {
        "soft": lambda: check(abi.bcjr_soft_codeword_v(w.data_ptr(), c.data_ptr(), B, steps, L, k, V, T, None,
                                                       out.data_ptr(), None, ws.data_ptr(), nbytes, sp), "soft_v"),
        "grad": lambda: check(abi.bcjr_soft_codeword_grad_v(w.data_ptr(), c.data_ptr(), B, steps, L, k, V, T, None,
                                                            g.data_ptr(), grad.data_ptr(), None, ws.data_ptr(), nbytes,
                                                            sp), "grad_v"),
        "viterbi": lambda: check(abi.viterbi_hard_code_v(w.data_ptr(), c.data_ptr(), B, steps, L, k, V, None,
                                                         states.data_ptr(), w_hard.data_ptr(), cost.data_ptr(),
                                                         ws.data_ptr(), nbytes, sp), "viterbi_v"),
    }
    slots = general_slots(k, V)
    ops = {}
    for name, fn in calls.items():
        fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        ev[0].record(stream)
        for i in range(K):
            fn()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(K)]))
        units = B * steps * S
        tail = {"grad": ", false, false, false", "viterbi": f", {viterbi_pairs(L, k, V)}"}.get(name, "")
        ops[name] = {"kernel": f"gen_{name}_kernel<{k}, {V}, 64, 16{tail}>",
                     "ms": round(ms, 4), "state_updates_per_s": DIRECTIONS[name] * units / (ms * 1e-3),
                     "weights_per_s": B * vw.n / (ms * 1e-3),
                     "roofline": {"bound": "alu", "achieved": round(slots[name] * units / (ms * 1e-3) / 1e12, 3),
                                  "peak": round(PEAK_SLOTS_PER_S / 1e12, 3), "unit": "T VALU-slots/s",
                                  "frac": round(slots[name] * units / (ms * 1e-3) / PEAK_SLOTS_PER_S, 4),
                                  "traffic": recorded_traffic(f"gen_{name}_k{k}v{V}", "qtip_1024x1024"),
                                  "per_unit": f"{slots[name]:.4g} fp32 VALU slots per state-step",
                                  "units_per_launch": units}}
    step_ms = sum(o["ms"] for o in ops.values())
    return {"workload": vw.name, "L": L, "k": k, "V": V, "B": B, "steps_per_sequence": steps, "T": T,
            "entry_points": "bcjr_soft_codeword_v, bcjr_soft_codeword_grad_v, viterbi_hard_code_v",
            "calls": K, "step_ms": round(step_ms, 4), "weights_per_s": B * vw.n / (step_ms * 1e-3),
            "state_updates_per_s": 5 * B * steps * S / (step_ms * 1e-3), "ops": ops}


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): sequences are "
              "independent, so more GPUs would shard the batch with no exchange; no multi-GPU figure is produced.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads
    from differentiable_bcjr_amd import abi

    abi.load()   # fails loudly if the HIP library has not been built
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X (no GPU visible)", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    wl = workloads.WORKLOADS[args.workload]
    B, n, L, k, T = wl.B, wl.n, wl.L, wl.k, float(args.temperature)
    S = 1 << L

    c = torch.from_numpy(wl.codebook()).to(dev)
    w = torch.from_numpy(wl.weights()).to(dev)
    g = torch.from_numpy(wl.upstream_grad()).to(dev)
    w_soft = torch.empty((B, n), dtype=torch.float32, device=dev)
    log_z = torch.empty((B,), dtype=torch.float32, device=dev)
    grad = torch.empty((B, n), dtype=torch.float32, device=dev)
    states = torch.empty((B, n), dtype=torch.int32, device=dev)
    w_hard = torch.empty((B, n), dtype=torch.float32, device=dev)
    cost = torch.empty((B,), dtype=torch.float32, device=dev)
    ops_ws = (0, 1, 2, 3, 5) if args.codebook_grad_steps > 0 else (0, 1, 2)
    ws_bytes = max(abi.bcjr_workspace_bytes(op, B, n, L, k) for op in ops_ws)
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: {abi.bcjr_status_string(rc)}")

    def soft():
        check(abi.bcjr_soft_codeword(w.data_ptr(), c.data_ptr(), B, n, L, k, T, None, w_soft.data_ptr(),
                                     log_z.data_ptr(), ws.data_ptr(), ws_bytes, sp), "bcjr_soft_codeword")

    def grad_op():
        check(abi.bcjr_soft_codeword_grad(w.data_ptr(), c.data_ptr(), B, n, L, k, T, None, g.data_ptr(),
                                          grad.data_ptr(), None, ws.data_ptr(), ws_bytes, sp),
              "bcjr_soft_codeword_grad")

    def viterbi():
        check(abi.viterbi_hard_code(w.data_ptr(), c.data_ptr(), B, n, L, k, None, states.data_ptr(),
                                    w_hard.data_ptr(), cost.data_ptr(), ws.data_ptr(), ws_bytes, sp),
              "viterbi_hard_code")

    ops = [("soft", soft), ("grad", grad_op), ("viterbi", viterbi)]

    if args.copy_calibration:
        # a plain copy of 1 GiB: reads 2^30 bytes and writes 2^30 bytes once each
        src = torch.empty((1 << 28,), dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print("copy calibration: one device copy of 1073741824 bytes", file=sys.stderr, flush=True)
        del src, dst

    for _ in range(args.warmup):
        for _, f in ops:
            f()
    torch.cuda.synchronize()

    K = args.steps
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        ev = events[s]
        ev[0].record(stream)
        for i, (_, f) in enumerate(ops):
            f()
            ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / K

    per_op = {}
    for i, (name, _) in enumerate(ops):
        ms = float(np.mean([events[s][i].elapsed_time(events[s][i + 1]) for s in range(K)]))
        upd = DIRECTIONS[name] * B * n * S
        slots = ALU_SLOTS[name] * B * n * S
        per_op[name] = {"kernel": KERNEL_NAMES[name], "ms": round(ms, 4), "state_updates_per_s": upd / (ms * 1e-3),
                        "weights_per_s": B * n / (ms * 1e-3),
                        "alu_frac": slots / (ms * 1e-3) / PEAK_SLOTS_PER_S,
                        "alu_frac_flat_count": FLAT_SLOTS[name] * B * n * S / (ms * 1e-3) / PEAK_SLOTS_PER_S}
    dom = max(per_op, key=lambda o: per_op[o]["ms"])
    d = per_op[dom]
    achieved = ALU_SLOTS[dom] * B * n * S / (d["ms"] * 1e-3) / 1e12
    peak = PEAK_SLOTS_PER_S / 1e12
    flat = FLAT_SLOTS[dom] * B * n * S / (d["ms"] * 1e-3) / 1e12
    roofline = {"bound": "alu", "kernel": d["kernel"], "achieved": round(achieved, 3), "peak": round(peak, 3),
                "unit": "T VALU-slots/s", "frac": round(achieved / peak, 4),
                "traffic": recorded_traffic(dom, wl.name),
                "per_unit": f"{ALU_SLOTS[dom]} fp32 VALU slots per state-step (half-rate op = 2, transcendental = 4)",
                "units_per_launch": B * n * S,
                "flat_count": {"achieved": round(flat, 3), "frac": round(flat / peak, 4),
                               "per_unit": f"{FLAT_SLOTS[dom]} slots per state-step: every VALU instruction 1, a "
                                           "transcendental 4"}}
    # The same kernel seen from HBM: its counter-measured bytes (the message tape) over its time, against a plain
    # 1 GiB device copy (2^30 bytes read and 2^30 written) timed here, after the step, on the same stream.
    copy_rate = device_copy_rate(dev, stream)
    if roofline["traffic"]:
        rate = roofline["traffic"] / (d["ms"] * 1e-3) / 1e9
        roofline["hbm_view"] = {"traffic_GBps": round(rate, 1), "device_copy_GBps": round(copy_rate, 1),
                                "frac_of_copy": round(rate / copy_rate, 4),
                                "note": "tape bytes per launch from the committed counters over the launch time, "
                                        "against a plain device copy measured in this run"}

    next_rows = {}
    if args.codebook_grad_steps > 0:
        # the codebook gradient, timed on its own after the step (it is not part of the step)
        grad_c = torch.empty((S,), dtype=torch.float32, device=dev)

        def grad_codebook():
            check(abi.bcjr_soft_codeword_grad_codebook(w.data_ptr(), c.data_ptr(), B, n, L, k, T, None, g.data_ptr(),
                                                       grad_c.data_ptr(), grad.data_ptr(), None, ws.data_ptr(),
                                                       ws_bytes, sp), "bcjr_soft_codeword_grad_codebook")

        grad_codebook()
        torch.cuda.synchronize()
        K2 = args.codebook_grad_steps
        ev2 = [torch.cuda.Event(enable_timing=True) for _ in range(K2 + 1)]
        ev2[0].record(stream)
        for i in range(K2):
            grad_codebook()
            ev2[i + 1].record(stream)
        torch.cuda.synchronize()
        ms2 = float(np.mean([ev2[i].elapsed_time(ev2[i + 1]) for i in range(K2)]))
        nbytes = CODEBOOK_GRAD_BYTES * B * n * S
        gbs = nbytes / (ms2 * 1e-3) / 1e9
        next_rows["grad_codebook"] = {
            "entry_point": "bcjr_soft_codeword_grad_codebook", "kernel": KERNEL_NAMES["grad_codebook"],
            "calls": K2, "ms": round(ms2, 4), "state_updates_per_s": 2 * B * n * S / (ms2 * 1e-3),
            "weights_per_s": B * n / (ms2 * 1e-3),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": recorded_traffic("grad_codebook", wl.name),
                         "per_unit": f"{CODEBOOK_GRAD_BYTES:g} B per state-step (tape 4, accumulator 8)",
                         "units_per_launch": B * n * S}}

    if args.codebook_grad_steps > 0:
        sigma_tb = torch.empty((B,), dtype=torch.int32, device=dev)

        def tail_biting():
            check(abi.viterbi_tail_biting(w.data_ptr(), c.data_ptr(), B, n, L, k, abi.BCJR_TB_ROTATE,
                                          states.data_ptr(), w_hard.data_ptr(), cost.data_ptr(), sigma_tb.data_ptr(),
                                          ws.data_ptr(), ws_bytes, sp), "viterbi_tail_biting")

        tail_biting()
        torch.cuda.synchronize()
        K3 = args.codebook_grad_steps
        ev3 = [torch.cuda.Event(enable_timing=True) for _ in range(K3 + 1)]
        ev3[0].record(stream)
        for i in range(K3):
            tail_biting()
            ev3[i + 1].record(stream)
        torch.cuda.synchronize()
        ms3 = float(np.mean([ev3[i].elapsed_time(ev3[i + 1]) for i in range(K3)]))
        slots3 = 2 * ALU_SLOTS["viterbi"] * B * n * S
        next_rows["viterbi_tail_biting_rotate"] = {
            "entry_point": "viterbi_tail_biting (BCJR_TB_ROTATE)", "kernel": "2 x viterbi_kernel<16>",
            "calls": K3, "ms": round(ms3, 4), "weights_per_s": B * n / (ms3 * 1e-3),
            "roofline": {"bound": "alu", "achieved": round(slots3 / (ms3 * 1e-3) / 1e12, 3),
                         "peak": round(PEAK_SLOTS_PER_S / 1e12, 3), "unit": "T VALU-slots/s",
                         "frac": round(slots3 / (ms3 * 1e-3) / PEAK_SLOTS_PER_S, 4),
                         "per_unit": f"2 x {ALU_SLOTS['viterbi']} fp32 VALU slots per state-step (two decodes)",
                         "units_per_launch": B * n * S}}

    if args.codebook_grad_steps > 0:
        # the soft codeword and the gradient in their checkpoint-and-recompute memory mode (the smallest workspace)
        g_ck = torch.empty_like(w)
        for name, op_id in (("soft", abi.BCJR_OP_SOFT), ("grad", abi.BCJR_OP_GRAD)):
            ck_bytes = abi.bcjr_workspace_bytes_min(op_id, B, n, L, k, 1)
            ws_ck = torch.empty(ck_bytes, dtype=torch.uint8, device=dev)
            out_ck = torch.empty_like(w)

            def run_ck(name=name, ws_ck=ws_ck, out_ck=out_ck, ck_bytes=ck_bytes):
                if name == "soft":
                    check(abi.bcjr_soft_codeword(w.data_ptr(), c.data_ptr(), B, n, L, k, T, None, out_ck.data_ptr(),
                                                 None, ws_ck.data_ptr(), ck_bytes, sp), "soft checkpoint")
                else:
                    check(abi.bcjr_soft_codeword_grad(w.data_ptr(), c.data_ptr(), B, n, L, k, T, None, g.data_ptr(),
                                                      out_ck.data_ptr(), g_ck.data_ptr(), ws_ck.data_ptr(), ck_bytes,
                                                      sp), "grad checkpoint")

            run_ck()
            torch.cuda.synchronize()
            K4 = args.codebook_grad_steps
            ev4 = [torch.cuda.Event(enable_timing=True) for _ in range(K4 + 1)]
            ev4[0].record(stream)
            for i in range(K4):
                run_ck()
                ev4[i + 1].record(stream)
            torch.cuda.synchronize()
            ms4 = float(np.mean([ev4[i].elapsed_time(ev4[i + 1]) for i in range(K4)]))
            slots4 = ALU_SLOTS[name] * B * n * S
            entry = "bcjr_soft_codeword" if name == "soft" else "bcjr_soft_codeword_grad"
            next_rows[f"{name}_checkpoint"] = {
                "entry_point": f"{entry} with bcjr_workspace_bytes_min",
                "kernel": CHECKPOINT_KERNELS[name],
                "checkpoint_interval": int(np.ceil(np.sqrt(n))), "workspace_bytes": ck_bytes,
                "full_tape_workspace_bytes": abi.bcjr_workspace_bytes(op_id, B, n, L, k),
                "calls": K4, "ms": round(ms4, 4), "state_updates_per_s": 2 * B * n * S / (ms4 * 1e-3),
                "weights_per_s": B * n / (ms4 * 1e-3),
                "roofline": {"bound": "alu", "achieved": round(slots4 / (ms4 * 1e-3) / 1e12, 3),
                             "peak": round(PEAK_SLOTS_PER_S / 1e12, 3), "unit": "T VALU-slots/s",
                             "frac": round(slots4 / (ms4 * 1e-3) / PEAK_SLOTS_PER_S, 4),
                             "per_unit": f"{ALU_SLOTS[name]} fp32 VALU slots per state-step (the method's work; the "
                                         "recompute's extra forward pass is overhead)",
                             "units_per_launch": B * n * S}}
            del ws_ck

    if args.trellis_variant_steps > 0:
        for key, vw in workloads.TRELLIS_VARIANTS.items():
            next_rows[f"trellis_{key}"] = time_variant(vw, T, args.trellis_variant_steps, dev, stream, check)

    total_upd = sum(DIRECTIONS[o] for o, _ in ops) * B * n * S
    line = {
        "metric": "trellis state-updates/sec and weights/sec, BCJR fwd+bwd, L=16 k=2 n=256",
        "value": total_upd / (ms_per_step * 1e-3),
        "unit": "state-updates/s",
        "weights_per_s": B * n / (ms_per_step * 1e-3),
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "matrix": wl.matrix, "L": L, "k": k, "B": B, "n": n, "T": T,
                   "boundary": "free", "step": "soft + grad + viterbi"},
        "ops": per_op,
        "roofline": roofline,
    }
    if next_rows:
        line["next_rows"] = next_rows
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, T)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
