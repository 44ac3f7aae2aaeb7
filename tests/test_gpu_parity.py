"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle,
at sizes the oracle finishes in seconds: several chunks and tiles, every
decay kind, d_k != d_v, fp32, a nonzero S_in / dS_out, and uniform,
non-uniform and single-chunk splits."""
import sys

import numpy as np
import pytest
import torch

from parity_util import TOL, compare, oracle_run, rne_mismatch
from state_passing_amd import linrec
from state_passing_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def small(name, B, H, T, dk, dv, dtype, decay, s_in=0.0):
    return Workload(900, name, B, H, T, dk, dv, dtype, decay, s_in_std=s_in, piece=T)


SMALL = [
    small("bf16-head", 1, 2, 256, 128, 128, "bf16", "head"),
    small("bf16-token", 2, 3, 384, 128, 128, "bf16", "token", s_in=0.1),
    small("bf16-none", 1, 2, 192, 128, 128, "bf16", "none"),
    small("bf16-64x64", 2, 2, 320, 64, 64, "bf16", "token", s_in=0.1),
    small("bf16-64x128", 1, 3, 256, 64, 128, "bf16", "head", s_in=0.1),
    small("bf16-128x64", 1, 3, 256, 128, 64, "bf16", "token", s_in=0.1),
    small("f32-64", 1, 2, 1024, 64, 64, "f32", "none"),
    small("f32-64-token", 2, 2, 256, 64, 64, "f32", "token", s_in=0.1),
    small("bf16-one-chunk", 1, 1, 64, 128, 128, "bf16", "token", s_in=0.1),
    # 36 chunks = 9 segments of 4: three scan rounds, the last one partial
    small("bf16-long", 1, 2, 2304, 128, 128, "bf16", "token", s_in=0.1),
    small("bf16-long-head", 2, 1, 2240, 128, 128, "bf16", "head"),
]


def gpu_inputs(wl, seed=7, with_dS_out=True):
    inp = make_inputs(wl, device="cpu", seed=seed, with_dS_out=with_dS_out)
    for name in ("q", "k", "v", "dO", "S_in", "decay", "dS_out"):
        x = getattr(inp, name)
        if x is not None:
            setattr(inp, name, x.to(DEV))
    return inp


def run_unsplit(inp, out_dtype=None):
    o, S_out, st = linrec.fwd(inp.q, inp.k, inp.v, inp.decay, inp.S_in, out_dtype=out_dtype)
    dq, dk, dv, dS_in = linrec.bwd(inp.q, inp.k, inp.v, inp.decay, st, inp.dO, inp.dS_out,
                                   out_dtype=out_dtype)
    torch.cuda.synchronize()
    return dict(o=o, S_out=S_out, dq=dq, dk=dk, dv=dv, dS_in=dS_in)


def run_seq(inp, lengths, out_dtype=None):
    o, S_out, st = linrec.fwd_seq(inp.q, inp.k, inp.v, inp.decay, lengths, inp.S_in,
                                  out_dtype=out_dtype)
    dq, dk, dv, dS_in = linrec.bwd_seq(inp.q, inp.k, inp.v, inp.decay, lengths, st, inp.dO,
                                       inp.dS_out, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return dict(o=o, S_out=S_out, dq=dq, dk=dk, dv=dv, dS_in=dS_in)


def run_loop(inp, lengths, out_dtype=None):
    o, S_out, dq, dk, dv, dS_in = linrec.piece_loop(inp.q, inp.k, inp.v, inp.decay, lengths,
                                                    inp.S_in, inp.dO, inp.dS_out,
                                                    out_dtype=out_dtype)
    torch.cuda.synchronize()
    return dict(o=o, S_out=S_out, dq=dq, dk=dk, dv=dv, dS_in=dS_in)


def check(got, ref, heads, wl, label):
    tol = TOL[wl.torch_dtype]
    errs, bad, report = compare(got, ref, heads, tol)
    print(f"[{label}] {wl.name}: {report}", flush=True)
    assert not bad, f"{label} {wl.name}: over tolerance {tol}: {bad}"


def check_rne(got16, got32, label):
    """bf16 outputs are the fp32 results of the same kernels rounded to
    nearest even."""
    for name in ("o", "dq", "dk", "dv"):
        frac, ulps = rne_mismatch(got16[name], got32[name])
        print(f"  [{label}] {name}: bf16 store vs rne(fp32 store): {frac:.2e} differ, "
              f"max {ulps} ulp", flush=True)
        assert frac <= 1e-4 and ulps <= 1, (label, name, frac, ulps)


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_small_unsplit(wl):
    """fp32 outputs against the plain bar, and the activation-dtype outputs
    (bf16 beyond its half-ulp representation limit, or fp32)."""
    print(f"case {wl}", flush=True)
    inp = gpu_inputs(wl)
    ref = oracle_run(inp)
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    got32 = run_unsplit(inp, torch.float32)
    check(got32, ref, heads, wl, "unsplit/f32-out")
    if wl.dtype == "bf16":
        got16 = run_unsplit(inp)
        check(got16, ref, heads, wl, "unsplit/bf16-out")
        check_rne(got16, got32, "unsplit")


SPLIT_CASES = SMALL[:2] + SMALL[6:8] + SMALL[9:10]


@pytest.mark.parametrize("wl", SPLIT_CASES, ids=[w.name for w in SPLIT_CASES])
def test_small_split_matches_oracle_and_unsplit(wl):
    """Uniform and non-uniform splits (seq driver and per-piece loop) against
    the oracle.  Cuts on segment boundaries (multiples of 256 tokens) leave
    the order of every fp32 operation unchanged, so those splits must also
    equal the GPU unsplit result bitwise; other cuts regroup the segment
    folds and are held to the oracle bar only."""
    inp = gpu_inputs(wl)
    ref = oracle_run(inp)
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    base = run_unsplit(inp, torch.float32)
    N = wl.T // 64
    splits = {"uniform": [wl.T // 2] * 2 if N % 2 == 0 else [64] * N,
              "ragged": [64] + [wl.T - 128] + [64] if N >= 3 else [wl.T]}
    if N >= 12:
        splits["five"] = [320, 64, wl.T - 640, 192, 64]
    if wl.T % 256 == 0 and wl.T >= 512:
        splits["segment-aligned"] = [256, wl.T - 512, 256] if wl.T >= 768 else [256, 256]
    for sname, lengths in splits.items():
        aligned = all(L % 256 == 0 for L in lengths[:-1])
        for runner in (run_seq, run_loop):
            got = runner(inp, lengths, torch.float32)
            check(got, ref, heads, wl, f"{runner.__name__}/{sname}")
            same = {k: bool(torch.equal(got[k], base[k])) for k in got}
            print(f"  segment-aligned={aligned} bitwise equal to unsplit: {same}", flush=True)
            if aligned:
                assert all(same.values()), same


@pytest.mark.parametrize("decay", ["token", "head"])
def test_strong_decay_unfactored_mask(decay):
    """Decays strong enough that a chunk's total log-decay falls below the
    threshold under which the mask factor is no longer taken as a product of
    two table entries (the later one would overflow): there the kernels take
    one exp per mask entry.  Per-token decays drawn in [0.3, 1) mix both
    paths chunk by chunk; a per-head decay of 0.5 (chunk decay 2^-64) takes
    the per-entry path everywhere.  Unsplit and split against the oracle."""
    wl = small(f"strong-{decay}", 2, 2, 768, 128, 128, "bf16", decay, s_in=0.1)
    inp = gpu_inputs(wl)
    g = torch.Generator().manual_seed(31)
    if decay == "token":
        a = 0.3 + 0.7 * torch.rand(tuple(inp.decay.shape), generator=g)
    else:
        a = torch.full(tuple(inp.decay.shape), 0.5)
    inp.decay = a.to(torch.float32).to(DEV)
    ref = oracle_run(inp)
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    check(run_unsplit(inp, torch.float32), ref, heads, wl, "unsplit/f32-out")
    check(run_seq(inp, [256, 448, 64], torch.float32), ref, heads, wl, "run_seq/f32-out")


RECOMPUTE_CASES = [SMALL[1], SMALL[4], SMALL[6], SMALL[9]]


@pytest.mark.parametrize("wl", RECOMPUTE_CASES, ids=[w.name for w in RECOMPUTE_CASES])
def test_recompute_equals_stored_states(wl):
    """The backward that rebuilds the segment states from S_in gives the
    backward over stored states bit for bit."""
    inp = gpu_inputs(wl)
    o, S_out, st = linrec.fwd(inp.q, inp.k, inp.v, inp.decay, inp.S_in)
    ref = linrec.bwd(inp.q, inp.k, inp.v, inp.decay, st, inp.dO, inp.dS_out)
    got = linrec.bwd_recompute(inp.q, inp.k, inp.v, inp.decay, inp.S_in, inp.dO, inp.dS_out)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv", "dS_in"), got, ref):
        assert torch.equal(a, b), name


def test_recompute_sequence_keeps_boundary_states_only():
    """Sequence accumulation that keeps one boundary state per piece: the
    forward reuses one state store, the backward rebuilds each piece's
    states; results against the oracle."""
    wl = SMALL[9]
    inp = gpu_inputs(wl)
    ref = oracle_run(inp)
    lengths = [256, 768, 512, 768]
    bounds = np.cumsum([0] + lengths)
    q, k, v, dO = inp.q, inp.k, inp.v, inp.dO
    o = torch.empty(v.shape, dtype=torch.float32, device=DEV)
    store = torch.empty(linrec.states_bytes(linrec.desc(wl.B, wl.H, max(lengths), wl.dk, wl.dv,
                                                        linrec.BF16, linrec.DECAY_TOKEN)),
                        dtype=torch.uint8, device=DEV)
    S = inp.S_in
    boundary = []
    for i, L in enumerate(lengths):
        sl = slice(int(bounds[i]), int(bounds[i + 1]))
        boundary.append(S)
        pd = linrec.desc(wl.B, wl.H, L, wl.dk, wl.dv, linrec.BF16, linrec.DECAY_TOKEN)
        _, S, _ = linrec.fwd(q[:, :, sl], k[:, :, sl], v[:, :, sl], inp.decay[:, :, sl], S,
                             o=o[:, :, sl], states=store[:linrec.states_bytes(pd)])
    S_out = S
    dq, dk, dv = (torch.empty(x.shape, dtype=torch.float32, device=DEV) for x in (q, k, v))
    dS = inp.dS_out
    for i in reversed(range(len(lengths))):
        sl = slice(int(bounds[i]), int(bounds[i + 1]))
        _, _, _, dS = linrec.bwd_recompute(q[:, :, sl], k[:, :, sl], v[:, :, sl],
                                           inp.decay[:, :, sl], boundary[i], dO[:, :, sl], dS,
                                           dq=dq[:, :, sl], dk=dk[:, :, sl], dv=dv[:, :, sl])
    torch.cuda.synchronize()
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    check(dict(o=o, S_out=S_out, dq=dq, dk=dk, dv=dv, dS_in=dS), ref, heads, wl, "recompute-seq")


def test_deterministic_run_to_run():
    wl = SMALL[1]
    inp = gpu_inputs(wl)
    a, b = run_unsplit(inp), run_unsplit(inp)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_aliasing_carry_in_place():
    """S_out may alias S_in and dS_in may alias dS_out."""
    wl = SMALL[1]
    inp = gpu_inputs(wl)
    base = run_unsplit(inp)
    S = inp.S_in.clone()
    o, S2, st = linrec.fwd(inp.q, inp.k, inp.v, inp.decay, S, S_out=S)
    dS = inp.dS_out.clone()
    _, _, _, dS2 = linrec.bwd(inp.q, inp.k, inp.v, inp.decay, st, inp.dO, dS, dS_in=dS)
    torch.cuda.synchronize()
    assert torch.equal(S, base["S_out"]) and torch.equal(dS, base["dS_in"])


def test_strided_piece_views():
    """Pieces passed as strided views of a [B,T,H,d]-major buffer."""
    wl = SMALL[0]
    inp = gpu_inputs(wl)
    base = run_unsplit(inp)
    # same values, memory laid out [B, T, H, d] and viewed as [B, H, T, d]
    rel = lambda x: x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)  # noqa: E731
    q, k, v, dO = (rel(x) for x in (inp.q, inp.k, inp.v, inp.dO))
    assert q.stride(2) == wl.H * wl.dk
    o, S_out, st = linrec.fwd(q, k, v, inp.decay, inp.S_in)
    dq, dk, dv, dS_in = linrec.bwd(q, k, v, inp.decay, st, dO, inp.dS_out)
    torch.cuda.synchronize()
    for name, x in dict(o=o, S_out=S_out, dq=dq, dk=dk, dv=dv, dS_in=dS_in).items():
        assert torch.equal(x, base[name]), name


if __name__ == "__main__":
    sys.exit(pytest.main([__file__, "-v", "-s"]))
