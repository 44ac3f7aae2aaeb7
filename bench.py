"""Benchmark of the chunkwise linear-recurrence layer on one MI355X.

One step is one pass of the whole path over the 256K-token sequence: the
forward over 64 sub-sequences of 4096 tokens in order, carrying S, then the
backward over them in reverse, carrying dS (sequence accumulation), through
the library's native sequence drivers.  Workload: B=1, H=16, T=262144,
d_k=d_v=128, bf16 inputs and outputs, per-head decay a_h = 1 - 2^-(5+8h/H),
chunk 64; inputs are seeded synthetic tensors resident in HBM before timing.

Prints one JSON line: fwd+bwd tokens/s (B*T / step time, the state
transitions on the library's auxiliary stream overlapping the segment
kernels), the roofline of the dominant kernel, the MFMA utilisation implied
by the algorithmic flop count, and the fp64 CPU oracle's rate on a bounded
sample of the same workload.

Per-kernel durations come from a second timed pass of the same work in
which every piece is issued through the per-piece calls on one stream, so
that no two kernels share the GPU and each kernel's HIP-event bracket (on
the stream it runs on) is its own duration.  The dominant kernel is the one
with the largest share of that pass; its roofline "achieved" figure is its
algorithmic bytes per launch over its mean duration.

The line also carries the two backward variants, timed the same way over
the 64 pieces in reverse: from boundary states alone (the per-segment states
rebuilt, so only one state per piece is kept between the passes) and with the
decay gradient.

Flags: --gpus N (only 1 is supported: one GPU), --steps K, --warmup W,
--no-cpu-baseline, --copy-probe BYTES (run only a device copy of that size,
for calibrating rocprofv3 byte counters), --profile (run only the
serialized pass, so a profiler sees undisturbed dispatches).
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

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
# Algorithmic work per token-head at d_k = d_v = 128, chunk 64 (bf16 I/O):
#   bytes: forward reads q, k, v and writes o; backward reads q, k, v, dO and
#   writes dq, dk, dv.  flops: forward 4Cd + 4d^2, backward 10Cd + 8d^2.
FWD_BYTES, BWD_BYTES = 1024, 1792
FWD_FLOPS, BWD_FLOPS = 98304, 212992
# per-launch algorithmic bytes of each kernel, per token-head of the piece
KERNEL_BYTES = {
    "fwd_sum": 512,        # reads k, v
    "fwd_fold": 0,         # moves per-segment states only
    "fwd_seg": 1024,       # reads q, k, v, writes o
    "bwd_sum": 512,        # reads q, dO
    "bwd_fold": 0,
    # reads q, k, v, dO, writes dq, dk, dv; in the sequence backward the
    # launch also computes another piece's segment sums (q, dO: 62 launches
    # of 64 in a step)
    "bwd_seg": 1792 + 512 * 62 / 64,
}
# per-launch bytes of each kernel as designed, per token-head: one fp32
# d_k x d_v record or state per 256-token segment is 256 B per token-head
KERNEL_DESIGN_BYTES = {
    "fwd_sum": 512 + 256,          # k, v; writes the segment records
    "fwd_fold": 256 + 256,         # reads records, writes segment-start states
    "fwd_seg": 1024 + 256,         # q, k, v, o; reads the segment-start state
    "bwd_sum": 512 + 256,          # q, dO; writes the gradient records
    "bwd_fold": 256 + 256,
    # k, v, dO for dQ; q, and k, v, dO again for the segment's first chunk
    # only (walk 2 finds the last chunk in LDS and the two before it in
    # registers); dq, dk, dv; the S and G segment states; the fold it
    # carries (63 launches of 64 in a step) and the segment sums it carries
    # (62 of 64)
    "bwd_seg": 768 + 256 + 192 + 768 + 512 + 512 * 63 / 64 + 768 * 62 / 64,
}
KERNEL_SYMBOL = {
    "fwd_sum": "seg_sum_kernel<bf16,128,128,false,false>",
    "fwd_fold": "seg_fold_kernel<128,128,false>",
    "fwd_seg": "fwd_seg_kernel<bf16,bf16,128,128,false>",
    "bwd_sum": "seg_sum_kernel<bf16,128,128,true,false>",
    "bwd_fold": "seg_fold_kernel<128,128,true>",
    "bwd_seg": "bwd_seg_kernel<bf16,bf16,128,128,false,false>",
}
# gated delta rule, per head-token at d = 128, bf16 activations, fp32 beta and gate
DELTA_BYTES = {"fwd": 4 * 256 + 2 * 4,          # q, k, v, o; beta, gate
               "bwd": 7 * 256 + 2 * 4 + 4}      # q, k, v, dO, dq, dk, dv; beta, gate; dbeta
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bwd_seg_sa256k_traffic.txt")
SQ_FILE = os.path.join(ROOT, "profiles", "linrec_kernels_sa256k_sq_counters.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "state_passing_amd", "csrc", f)
                  for f in ("kernels.hip", "device.hpp", "launch.hpp")]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-probe", type=int, default=0)
    p.add_argument("--profile", action="store_true")
    p.add_argument("--profile-delta", action="store_true",
                   help="run one forward and one backward of the delta-rule workload's sequence drivers only")
    return p.parse_args()


def kernel_source_hash() -> str:
    """Hash of the device-code sources; counters taken on other code are stale."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel: str, launch_units: int):
    """HBM bytes per launch from the committed counter summary, scaled by the
    copy-kernel calibration; None if missing or taken on other kernel code."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    txt = open(TRAFFIC_FILE).read()
    m = re.search(r"kernel_source_sha256_16:\s*(\w+)", txt)
    if not m or m.group(1) != kernel_source_hash():
        return None
    m = re.search(r"bytes_per_launch_calibrated:\s*([0-9.eE+]+)", txt)
    return float(m.group(1)) if m else None


def mfma_busy_from_profile(kernel: str):
    """A kernel's MFMA busy percentage from the committed shader counter
    summary; None if missing or taken on other kernel code."""
    if not os.path.exists(SQ_FILE):
        return None
    txt = open(SQ_FILE).read()
    m = re.search(r"kernel_source_sha256_16:\s*(\w+)", txt)
    if not m or m.group(1) != kernel_source_hash():
        return None
    m = re.search(r"mfma_busy_pct_%s:\s*([0-9.eE+]+)" % kernel, txt)
    return float(m.group(1)) if m else None


def copy_probe(nbytes: int) -> float:
    """Read + write GB/s of a plain device copy of `nbytes` (torch's copy
    kernel), timed with events over 10 copies after 3 untimed ones: the HBM
    rate a streaming kernel can reach on this GPU, beside the 8 TB/s spec."""
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    reps = 10
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    dt = a.elapsed_time(b) * 1e-3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / dt / 1e9


def cpu_baseline(inp, wl, sample_tokens: int):
    """The fp64 oracle, unsplit, on all heads of the first `sample_tokens`
    tokens of the same inputs (bf16 values upcast to fp64)."""
    import numpy as np
    import torch
    import oracle
    sl = slice(0, sample_tokens)
    f64 = lambda t: np.ascontiguousarray(t[:, :, sl].to("cpu", torch.float64).numpy())  # noqa: E731
    q, k, v, dO = f64(inp.q), f64(inp.k), f64(inp.v), f64(inp.dO)
    a = inp.decay.to("cpu", torch.float64).numpy()
    available = len(os.sched_getaffinity(0))
    threads = min(wl.B * wl.H, available)
    t0 = time.perf_counter()
    oracle.fwd(q, k, v, a, None, nthreads=threads)
    t1 = time.perf_counter()
    oracle.bwd(q, k, v, a, None, dO, None, nthreads=threads)
    dt = time.perf_counter() - t0
    return {"value": wl.B * sample_tokens / dt, "unit": "tokens/s", "cores": threads,
            "cores_available": available, "cpu_count": os.cpu_count(), "kind": "oracle",
            "sample": f"fwd+bwd, unsplit, all {wl.B * wl.H} heads, first {sample_tokens} of "
                      f"{wl.T} tokens ({dt:.1f} s)",
            "fwd_tokens_per_s": wl.B * sample_tokens / (t1 - t0)}


def delta_bench(linrec, dev, args):
    """Gated delta rule on its 16-head, 16K-token workload (4 pieces of 4096,
    per-token gate, d = 128, bf16): forward over the pieces (keeping what the
    backward needs), then the backward in reverse, carrying dS, through the
    sequence drivers (the backward runs a piece's per-chunk gradient kernels
    beside the next piece's serial walk); the per-piece calls beside them."""
    import torch
    from state_passing_amd.workloads import DELTA_WORKLOADS, make_inputs
    wl = DELTA_WORKLOADS[6]
    inp = make_inputs(wl, device=dev)
    lengths = wl.pieces()
    B, H, T, D = wl.B, wl.H, wl.T, wl.dk
    o = torch.empty(B, H, T, D, dtype=torch.bfloat16, device=dev)
    dq, dk, dv = (torch.empty(B, H, T, D, dtype=torch.bfloat16, device=dev) for _ in range(3))
    db = torch.empty(B, H, T, dtype=torch.float32, device=dev)
    pd = linrec.desc(B, H, lengths[0], D, D, linrec.BF16, linrec.DECAY_TOKEN)
    saved = [torch.empty(linrec.delta_saved_bytes(pd), dtype=torch.uint8, device=dev) for _ in lengths]
    wsf = torch.empty(linrec.delta_workspace_bytes(pd), dtype=torch.uint8, device=dev)
    wsb = torch.empty(linrec.delta_bwd_workspace_bytes(pd), dtype=torch.uint8, device=dev)
    S = torch.empty(B, H, D, D, dtype=torch.float32, device=dev)
    dS = torch.empty_like(S)
    bounds = [0]
    for L in lengths:
        bounds.append(bounds[-1] + L)

    def fwd():
        for i in range(len(lengths)):
            sl = slice(bounds[i], bounds[i + 1])
            linrec.delta_fwd(inp.q[:, :, sl], inp.k[:, :, sl], inp.v[:, :, sl], inp.beta[:, :, sl],
                             inp.decay[:, :, sl], None if i == 0 else S, o=o[:, :, sl], S_out=S,
                             saved=saved[i], workspace=wsf)

    def bwd():
        for i in reversed(range(len(lengths))):
            sl = slice(bounds[i], bounds[i + 1])
            linrec.delta_bwd(inp.q[:, :, sl], inp.k[:, :, sl], inp.v[:, :, sl], inp.beta[:, :, sl],
                             inp.decay[:, :, sl], saved[i], inp.dO[:, :, sl],
                             None if i == len(lengths) - 1 else dS, dq=dq[:, :, sl],
                             dk=dk[:, :, sl], dv=dv[:, :, sl], dbeta=db[:, :, sl], dS_in=dS,
                             workspace=wsb)

    seq_saved = torch.empty(linrec.delta_seq_saved_bytes(
        linrec.desc(B, H, T, D, D, linrec.BF16, linrec.DECAY_TOKEN), lengths), dtype=torch.uint8,
        device=dev)

    def fwd_seq():
        linrec.delta_fwd_seq(inp.q, inp.k, inp.v, inp.beta, inp.decay, lengths, None, o=o, S_out=S,
                             saved=seq_saved)

    def bwd_seq():
        linrec.delta_bwd_seq(inp.q, inp.k, inp.v, inp.beta, inp.decay, lengths, seq_saved, inp.dO,
                             None, dq=dq, dk=dk, dv=dv, dbeta=db, dS_in=dS)

    def timed(fn, steps):
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            fn()
        b_.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b_) / steps

    if args.profile_delta:
        # only the sequence drivers' dispatches, for a profiler
        fwd_seq()
        bwd_seq()
        torch.cuda.synchronize()
        return {"profile": "delta-rule sequence drivers", "steps": 1}
    for _ in range(max(args.warmup, 1)):
        fwd()
        bwd()
        fwd_seq()
        bwd_seq()
    steps = max(1, min(args.steps, 5))
    ms_fwd = timed(fwd_seq, steps)
    ms_bwd = timed(bwd_seq, steps)
    ms_fwd_pp = timed(fwd, steps)
    ms_bwd_pp = timed(bwd, steps)
    tokens = B * T
    # algorithmic bytes per head-token (bf16, d = 128): forward reads q, k, v,
    # beta, gate and writes o; backward reads q, k, v, dO, beta, gate and
    # writes dq, dk, dv, dbeta
    fwd_b, bwd_b = DELTA_BYTES["fwd"] * B * H * T, DELTA_BYTES["bwd"] * B * H * T
    fwd_gbs, bwd_gbs = fwd_b / (ms_fwd * 1e-3) / 1e9, bwd_b / (ms_bwd * 1e-3) / 1e9
    return {"workload": wl.name, "B": B, "H": H, "T": T, "d": D,
            "pieces": f"{len(lengths)} x {lengths[0]}", "decay": "per-token gate",
            "fwd_ms": ms_fwd, "bwd_ms": ms_bwd, "fwd_tokens_per_s": tokens / (ms_fwd * 1e-3),
            "fwd_plus_bwd_tokens_per_s": tokens / ((ms_fwd + ms_bwd) * 1e-3),
            "roofline": {"bound": "latency (serial chunk walks on half the CUs)",
                         "algorithmic_bytes_per_head_token": DELTA_BYTES,
                         "fwd_GBs": fwd_gbs, "bwd_GBs": bwd_gbs, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "fwd_frac": fwd_gbs / PEAK_HBM_GBS,
                         "bwd_frac": bwd_gbs / PEAK_HBM_GBS},
            "per_piece_calls": {"fwd_ms": ms_fwd_pp, "bwd_ms": ms_bwd_pp}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported; this build measures one GPU "
              "(the layer's one-GPU share; see the sharding design)", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_probe:
        print(json.dumps({"copy_probe_bytes": args.copy_probe,
                          "read_plus_write_GBs": copy_probe(args.copy_probe)}))
        return
    if args.profile_delta:
        from state_passing_amd import linrec
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        print(json.dumps(delta_bench(linrec, dev, args)))
        return

    from state_passing_amd import linrec
    from state_passing_amd.workloads import WORKLOADS, make_inputs

    wl = WORKLOADS[3]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_inputs(wl, device=dev)
    lengths = wl.pieces()
    B, H, T, DK, DV = wl.B, wl.H, wl.T, wl.dk, wl.dv

    o = torch.empty(B, H, T, DV, dtype=torch.bfloat16, device=dev)
    dq, dk, dv = (torch.empty(B, H, T, d, dtype=torch.bfloat16, device=dev) for d in (DK, DK, DV))
    S_out = torch.empty(B, H, DK, DV, dtype=torch.float32, device=dev)
    dS_in = torch.empty_like(S_out)
    d = linrec.desc(B, H, T, DK, DV, linrec.BF16, linrec.DECAY_HEAD)
    states = torch.empty(linrec.seq_states_bytes(d, lengths), dtype=torch.uint8, device=dev)
    ws = torch.empty(linrec.bwd_seq_workspace_bytes(d, lengths), dtype=torch.uint8, device=dev)
    bounds = [0]
    for L in lengths:
        bounds.append(bounds[-1] + L)

    def step_seq(record=None):
        ev = None
        if record is not None:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            ev[0].record()
        linrec.fwd_seq(inp.q, inp.k, inp.v, inp.decay, lengths, inp.S_in, o=o, S_out=S_out,
                       states=states)
        if ev is not None:
            ev[1].record()
        linrec.bwd_seq(inp.q, inp.k, inp.v, inp.decay, lengths, states, inp.dO, None, dq=dq,
                       dk=dk, dv=dv, dS_in=dS_in, workspace=ws)
        if ev is not None:
            ev[2].record()
            record.append(ev)

    def timed(fn, steps):
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            fn()
        b_.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b_) / steps

    for _ in range(args.warmup):
        step_seq()
    torch.cuda.synchronize()
    if args.profile:
        # only the timed region's dispatches, for a profiler
        for _ in range(args.steps):
            step_seq()
        torch.cuda.synchronize()
        print(json.dumps({"profile": "sequence drivers", "steps": args.steps}))
        return

    # timed region: K whole steps, bracketed by synchronisation
    fwd_ev = []
    t0 = time.perf_counter()
    ms_step = timed(lambda: step_seq(fwd_ev), args.steps)
    wall = time.perf_counter() - t0
    fwd_only_ms = sum(e[0].elapsed_time(e[1]) for e in fwd_ev) / len(fwd_ev)
    per_step = sorted(e[0].elapsed_time(e[2]) for e in fwd_ev)

    # the same steps again with per-kernel events on each kernel's own stream
    linrec.set_kernel_timing(True)
    ms_events = timed(step_seq, args.steps)
    ktimes = linrec.kernel_times()
    linrec.set_kernel_timing(False)

    tokens = B * T
    token_heads_piece = B * H * lengths[0]
    kernels = {}
    for name, (n, ms) in ktimes.items():
        if n == 0 or name not in KERNEL_BYTES:
            continue
        avg_ms = ms / n
        kernels[name] = {
            "launches_per_step": n // args.steps, "avg_us": avg_ms * 1e3,
            "ms_per_step": ms / args.steps,
            "algorithmic_GBs": KERNEL_BYTES[name] * token_heads_piece / (avg_ms * 1e-3) / 1e9,
            "design_GBs": KERNEL_DESIGN_BYTES[name] * token_heads_piece / (avg_ms * 1e-3) / 1e9,
        }
    dominant = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dom = kernels[dominant]
    achieved = dom["algorithmic_GBs"]
    traffic = traffic_from_profile(dominant, token_heads_piece)
    roofline = {"kernel": dominant, "symbol": KERNEL_SYMBOL[dominant], "bound": "hbm",
                "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                "algorithmic_bytes_per_launch": KERNEL_BYTES[dominant] * token_heads_piece,
                "design_bytes_per_launch": KERNEL_DESIGN_BYTES[dominant] * token_heads_piece,
                "avg_launch_us": dom["avg_us"],
                # what a plain streaming copy reaches on this GPU, beside the spec peak
                "copy_probe_GBs": copy_probe(1 << 30)}

    # The backward variants, each over the 64 pieces in reverse with dS
    # carried through the per-piece calls, against the plain per-piece
    # backward; the per-piece forward below leaves the piece states, the
    # boundary states and o in place.
    pd = linrec.desc(B, H, lengths[0], DK, DV, linrec.BF16, linrec.DECAY_HEAD)
    piece_states = [torch.empty(linrec.states_bytes(pd), dtype=torch.uint8, device=dev)
                    for _ in lengths]
    piece_ws = torch.empty(linrec.bwd_workspace_bytes(pd), dtype=torch.uint8, device=dev)
    bnd = torch.zeros(len(lengths) + 1, B, H, DK, DV, dtype=torch.float32, device=dev)
    if inp.S_in is not None:
        bnd[0].copy_(inp.S_in)
    for i in range(len(lengths)):
        sl = slice(bounds[i], bounds[i + 1])
        linrec.fwd(inp.q[:, :, sl], inp.k[:, :, sl], inp.v[:, :, sl], inp.decay, bnd[i],
                   o=o[:, :, sl], S_out=bnd[i + 1], states=piece_states[i])
    ws_rc = torch.empty(linrec.bwd_recompute_workspace_bytes(pd), dtype=torch.uint8, device=dev)
    ws_da = torch.empty(linrec.bwd_da_workspace_bytes(pd), dtype=torch.uint8, device=dev)
    da = torch.empty(B, H, T, dtype=torch.float32, device=dev)
    carry = torch.zeros(B, H, dtype=torch.float32, device=dev)

    def pieces_bwd(kind):
        dS = None
        if kind == "da":
            carry.zero_()
        for i in reversed(range(len(lengths))):
            sl = slice(bounds[i], bounds[i + 1])
            a = (inp.q[:, :, sl], inp.k[:, :, sl], inp.v[:, :, sl], inp.decay)
            outs = dict(dq=dq[:, :, sl], dk=dk[:, :, sl], dv=dv[:, :, sl], dS_in=dS_in)
            if kind == "plain":
                linrec.bwd(*a, piece_states[i], inp.dO[:, :, sl], dS, workspace=piece_ws, **outs)
            elif kind == "recompute":
                linrec.bwd_recompute(*a, bnd[i], inp.dO[:, :, sl], dS, workspace=ws_rc, **outs)
            else:
                linrec.bwd_da(*a, piece_states[i], inp.dO[:, :, sl], dS, carry, da=da[:, :, sl],
                              da_carry_out=carry, workspace=ws_da, **outs)
            dS = dS_in

    variants = {}
    for kind in ("plain", "recompute", "da"):
        pieces_bwd(kind)
        variants[kind] = timed(lambda: pieces_bwd(kind), args.steps)
    next_rows = {
        "bwd_per_piece_ms": variants["plain"],
        "bwd_recompute_ms": variants["recompute"],
        "bwd_recompute_tokens_per_s_fwd_plus_bwd": tokens / ((fwd_only_ms + variants["recompute"]) * 1e-3),
        "bwd_da_ms": variants["da"],
        "kept_between_passes_bytes": {
            "stored_states": linrec.seq_states_bytes(d, lengths),
            "boundary_states_only": (len(lengths) + 1) * B * H * DK * DV * 4},
    }

    flops_step = (FWD_FLOPS + BWD_FLOPS) * B * H * T
    result = {
        "metric": "fwd+bwd tokens/s at T=256K,H=16,d=128 bf16; MFMA util % of peak",
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_median": per_step[len(per_step) // 2],
        "ms_per_step_min": per_step[0],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "H": H, "T": T, "d_k": DK, "d_v": DV,
                   "chunk": 64, "pieces": f"{len(lengths)} x {lengths[0]}",
                   "decay": "per-head", "outputs": "bf16"},
        "fwd_tokens_per_s": tokens / (fwd_only_ms * 1e-3),
        "fwd_ms": fwd_only_ms,
        "mfma_util_pct": 100.0 * flops_step / (ms_step * 1e-3) / (PEAK_BF16_TFLOPS * 1e12),
        "mfma_busy_pct_counters": {k: mfma_busy_from_profile(k) for k in ("fwd_seg", "bwd_seg")},
        "hbm_roof_pct_minimal_bytes": 100.0 * (FWD_BYTES + BWD_BYTES) * B * H * T
                                      / (ms_step * 1e-3) / (PEAK_HBM_GBS * 1e9),
        "fwd_mfma_util_pct": 100.0 * FWD_FLOPS * B * H * T / (fwd_only_ms * 1e-3)
                             / (PEAK_BF16_TFLOPS * 1e12),
        "fwd_hbm_roof_pct_minimal_bytes": 100.0 * FWD_BYTES * B * H * T / (fwd_only_ms * 1e-3)
                                          / (PEAK_HBM_GBS * 1e9),
        "roofline": roofline,
        "ms_per_step_with_kernel_events": ms_events,
        "kernels": kernels,
        "backward_variants": next_rows,
        "delta_rule": delta_bench(linrec, dev, args),
        "wall_s_timed": wall,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, wl, sample_tokens=wl.T)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
