"""Benchmark of the chunkwise linear-recurrence layer on one MI355X.

One step is one pass of the whole path over the 256K-token sequence: the
forward over 64 sub-sequences of 4096 tokens in order, carrying S, then the
backward over them in reverse, carrying dS (sequence accumulation), through
the library's native sequence drivers.  Workload: B=1, H=16, T=262144,
d_k=d_v=128, bf16 inputs and outputs, per-head decay a_h = 1 - 2^-(5+8h/H),
chunk 64; inputs are seeded synthetic tensors resident in HBM before timing.

Prints one JSON line: fwd+bwd tokens/s (B*T / step time), the roofline of
the dominant kernel (algorithmic bytes per launch over its mean duration,
timed with HIP events on its own stream during a second timed pass), the
MFMA utilisation implied by the algorithmic flop count, and the fp64 CPU
oracle's rate on a bounded sample of the same workload.

Flags: --gpus N (only 1 is supported: one GPU), --steps K, --warmup W,
--no-cpu-baseline, --copy-probe BYTES (run only a device copy of that size,
for calibrating rocprofv3 byte counters), --profile (fewer side legs; for
runs under rocprofv3).
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
    "fwd_scan": 512,       # reads k, v
    "fwd_intra": 1024,     # reads q, k, v, writes o
    "bwd_scan": 512,       # reads q, dO
    "bwd_intra": 1792,     # reads q, k, v, dO, writes dq, dk, dv
}
KERNEL_SYMBOL = {
    "fwd_scan": "state_scan_kernel",
    "fwd_intra": "fwd_intra_kernel",
    "bwd_scan": "state_scan_kernel",
    "bwd_intra": "bwd_intra_kernel",
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bwd_intra_sa256k_traffic.txt")
KERNEL_SOURCE = os.path.join(ROOT, "state_passing_amd", "csrc", "kernels.hip")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-probe", type=int, default=0)
    p.add_argument("--profile", action="store_true")
    return p.parse_args()


def kernel_source_hash() -> str:
    return hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()[:16]


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


def copy_probe(nbytes: int) -> None:
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    reps = 10
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"copy_probe_bytes": nbytes, "read_plus_write_GBs": 2 * nbytes / dt / 1e9}))


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
    threads = min(wl.B * wl.H, len(os.sched_getaffinity(0)))
    t0 = time.perf_counter()
    oracle.fwd(q, k, v, a, None, nthreads=threads)
    oracle.bwd(q, k, v, a, None, dO, None, nthreads=threads)
    dt = time.perf_counter() - t0
    return {"value": wl.B * sample_tokens / dt, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"fwd+bwd, unsplit, all {wl.B * wl.H} heads, first {sample_tokens} of "
                      f"{wl.T} tokens ({dt:.1f} s)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported; this build measures one GPU "
              "(the layer's one-GPU share; see the sharding design)", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_probe:
        copy_probe(args.copy_probe)
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
    states = torch.empty(linrec.states_bytes(d), dtype=torch.uint8, device=dev)
    ws = torch.empty(linrec.bwd_seq_workspace_bytes(d, lengths), dtype=torch.uint8, device=dev)

    fwd_ms = []

    def step(record_fwd=False):
        e0 = e1 = None
        if record_fwd:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        linrec.fwd_seq(inp.q, inp.k, inp.v, inp.decay, lengths, inp.S_in, o=o, S_out=S_out,
                       states=states)
        if record_fwd:
            e1.record()
            fwd_ms.append((e0, e1))
        linrec.bwd_seq(inp.q, inp.k, inp.v, inp.decay, lengths, states, inp.dO, None, dq=dq,
                       dk=dk, dv=dv, dS_in=dS_in, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps, bracketed by synchronisation
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        step(record_fwd=True)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(stop) / args.steps
    fwd_only_ms = sum(a.elapsed_time(b) for a, b in fwd_ms) / len(fwd_ms)

    # second timed pass with per-kernel events on each kernel's own stream
    linrec.set_kernel_timing(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ktimes = linrec.kernel_times()
    linrec.set_kernel_timing(False)

    tokens = B * T
    token_heads_piece = B * H * lengths[0]
    kernels = {}
    for name, (n, ms) in ktimes.items():
        if n == 0:
            continue
        avg_ms = ms / n
        kernels[name] = {
            "launches_per_step": n // args.steps, "avg_us": avg_ms * 1e3,
            "ms_per_step": ms / args.steps,
            "algorithmic_GBs": KERNEL_BYTES[name] * token_heads_piece / (avg_ms * 1e-3) / 1e9,
        }
    dominant = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dom = kernels[dominant]
    achieved = dom["algorithmic_GBs"]
    flops_step = (FWD_FLOPS + BWD_FLOPS) * B * H * T
    traffic = traffic_from_profile(dominant, token_heads_piece)

    result = {
        "metric": "fwd+bwd tokens/s at T=256K,H=16,d=128 bf16; MFMA util % of peak",
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
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
        "hbm_roof_pct_minimal_bytes": 100.0 * (FWD_BYTES + BWD_BYTES) * B * H * T
                                      / (ms_step * 1e-3) / (PEAK_HBM_GBS * 1e9),
        "roofline": {"kernel": dominant, "symbol": KERNEL_SYMBOL[dominant], "bound": "hbm",
                     "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic},
        "kernels": kernels,
        "wall_s_timed": wall,
    }
    if not args.no_cpu_baseline and not args.profile:
        result["cpu_baseline"] = cpu_baseline(inp, wl, sample_tokens=wl.T)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
