"""GPU parity of the gated delta rule (linrec_delta_fwd / linrec_delta_bwd,
through the C ABI) against the fp64 delta-rule oracle: small cases over every
decay kind, d = 64 and 128, fp32 and bf16 inputs, a nonzero S_in and dS_out,
pieces chained through S_out -> S_in and dS_in -> dS_out, and the 16-head,
16K-token gated workload on sampled heads.

Error measure as for the linear recurrence: max|X_gpu - X_oracle| / RMS(X_oracle)
per tensor, fp32 outputs, bar 2e-2 for bf16 inputs and 1e-4 for fp32."""
import os

import numpy as np
import pytest
import torch

import oracle
from parity_util import np64, select_heads
from state_passing_amd import linrec
from state_passing_amd.workloads import DELTA_WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"bf16": 2e-2, "f32": 1e-4}


def small(name, B, H, T, d, dtype, decay, s_in=0.0):
    return Workload(960, name, B, H, T, d, d, dtype, decay, s_in_std=s_in, piece=T, delta=True)


SMALL = [
    small("delta-bf16-token", 1, 2, 256, 128, "bf16", "token", s_in=0.1),
    small("delta-bf16-head", 2, 2, 384, 128, "bf16", "head"),
    small("delta-bf16-none", 1, 3, 192, 128, "bf16", "none", s_in=0.1),
    small("delta-bf16-64", 2, 2, 320, 64, "bf16", "token", s_in=0.1),
    small("delta-f32-64", 1, 2, 256, 64, "f32", "token", s_in=0.1),
    small("delta-one-chunk", 1, 1, 64, 128, "bf16", "token", s_in=0.1),
]


def to_dev(inp):
    for name in ("q", "k", "v", "dO", "S_in", "dS_out", "decay", "beta"):
        x = getattr(inp, name)
        if x is not None:
            setattr(inp, name, x.to(DEV))
    return inp


def oracle_delta(inp, heads=None, backward=False):
    wl = inp.wl
    if heads is None:
        heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    pick = lambda x: None if x is None else np.ascontiguousarray(np64(select_heads(x, heads)))  # noqa: E731
    a = None
    if inp.decay is not None:
        a = (np.array([float(inp.decay[h]) for _, h in heads]) if inp.decay.dim() == 1
             else pick(inp.decay))
    o, S_out = oracle.delta_fwd(pick(inp.q), pick(inp.k), pick(inp.v), pick(inp.beta), a,
                                pick(inp.S_in))
    out = {"o": o, "S_out": S_out}
    if backward:
        dq, dk, dv, db, dS_in = oracle.delta_bwd(pick(inp.q), pick(inp.k), pick(inp.v),
                                                 pick(inp.beta), a, pick(inp.S_in), pick(inp.dO),
                                                 pick(inp.dS_out))
        out.update(dq=dq, dk=dk, dv=dv, dbeta=db, dS_in=dS_in)
    return out


def errors(got, ref, heads):
    out = {}
    for name, r in ref.items():
        g = np64(select_heads(got[name], heads))
        rms = float(np.sqrt(np.mean(r * r)))
        out[name] = float(np.max(np.abs(g - r))) / rms
    return out


def run_pieces(inp, lengths, backward=False):
    """The pieces one after another, S carried through S_out -> S_in, then
    (backward) in reverse with dS carried through dS_in -> dS_out."""
    S = inp.S_in
    o = torch.empty(inp.v.shape, dtype=torch.float32, device=DEV)
    bounds, saved = [0], []
    for L in lengths:
        bounds.append(bounds[-1] + L)
    dsl = lambda x, sl: x if x is None or x.dim() == 1 else x[:, :, sl]  # noqa: E731
    for i in range(len(lengths)):
        sl = slice(bounds[i], bounds[i + 1])
        _, S, sv = linrec.delta_fwd(inp.q[:, :, sl], inp.k[:, :, sl], inp.v[:, :, sl],
                                    inp.beta[:, :, sl], dsl(inp.decay, sl), S, o=o[:, :, sl],
                                    save=backward)
        saved.append(sv)
    out = {"o": o, "S_out": S}
    if backward:
        dq, dk, dv = (torch.empty(x.shape, dtype=torch.float32, device=DEV) for x in (inp.q, inp.k, inp.v))
        db = torch.empty(inp.beta.shape, dtype=torch.float32, device=DEV)
        dS = inp.dS_out
        for i in reversed(range(len(lengths))):
            sl = slice(bounds[i], bounds[i + 1])
            _, _, _, _, dS = linrec.delta_bwd(inp.q[:, :, sl], inp.k[:, :, sl], inp.v[:, :, sl],
                                              inp.beta[:, :, sl], dsl(inp.decay, sl), saved[i],
                                              inp.dO[:, :, sl], dS, dq=dq[:, :, sl], dk=dk[:, :, sl],
                                              dv=dv[:, :, sl], dbeta=db[:, :, sl], out_dtype=torch.float32)
        out.update(dq=dq, dk=dk, dv=dv, dbeta=db, dS_in=dS)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_delta_backward_small(wl):
    """Forward with the saved states, backward against the oracle's gradients
    (q, k, v, beta, S_in) with a nonzero dS_out; whole piece and chained."""
    print(f"case {wl}", flush=True)
    inp = to_dev(make_inputs(wl, device="cpu", seed=11, with_dS_out=True))
    ref = oracle_delta(inp, backward=True)
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    splits = [[wl.T]] + ([[64, wl.T - 192, 128]] if wl.T >= 256 else [])
    for lens in splits:
        errs = errors(run_pieces(inp, lens, backward=True), ref, heads)
        print(f"[{wl.name} pieces {lens}] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
              flush=True)
        assert all(v <= TOL[wl.dtype] for v in errs.values()), errs


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_delta_forward_small(wl):
    print(f"case {wl}", flush=True)
    inp = to_dev(make_inputs(wl, device="cpu", seed=9))
    ref = oracle_delta(inp)
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    got = run_pieces(inp, [wl.T])
    errs = errors(got, ref, heads)
    print(f"[{wl.name}] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert all(v <= TOL[wl.dtype] for v in errs.values()), errs
    if wl.T >= 256:
        lens = [64, wl.T - 192, 128]
        errs2 = errors(run_pieces(inp, lens), ref, heads)
        print(f"[{wl.name} pieces {lens}] " + " ".join(f"{k}={v:.2e}" for k, v in errs2.items()),
              flush=True)
        assert all(v <= TOL[wl.dtype] for v in errs2.values()), errs2


def test_delta_unit_key_overwrite_exact():
    """|k| = 1 and beta = 1 at a token whose query is its key: the output there
    is v_t (the oracle's special case, through the GPU path)."""
    wl = small("delta-overwrite", 1, 2, 256, 128, "bf16", "token", s_in=0.1)
    inp = make_inputs(wl, device="cpu", seed=10)
    hits = [5, 70, 130, 255]
    inp.beta[:, :, hits] = 1.0
    inp.q[:, :, hits] = inp.k[:, :, hits]
    inp = to_dev(inp)
    got = run_pieces(inp, [wl.T])
    ref = oracle_delta(inp)
    o_hits = got["o"][:, :, hits].double().cpu().numpy()
    v_hits = np64(inp.v[:, :, hits])
    # the oracle reproduces v exactly up to the bf16 rounding of k (|k| != 1 exactly)
    print("max|o - v| at the hits: gpu %.2e oracle %.2e"
          % (np.abs(o_hits - v_hits).max(), np.abs(ref["o"][:, :, hits] - v_hits).max()), flush=True)
    assert np.abs(o_hits - ref["o"][:, :, hits]).max() <= 1e-3 * np.abs(v_hits).max()


def test_delta_gated_16k_sampled_heads():
    """Forward and backward over the 4 pieces of the 16-head, 16K-token gated
    workload; the oracle runs unsplit on three heads."""
    wl = DELTA_WORKLOADS[6]
    heads = [(0, 0), (0, 7), (0, 15)]
    inp = make_inputs(wl, device=DEV)
    ref = oracle_delta(inp, heads, backward=True)
    got = run_pieces(inp, wl.pieces(), backward=True)
    errs = errors(got, ref, heads)
    print(f"[{wl.name} {len(wl.pieces())} pieces] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
          flush=True)
    assert all(v <= TOL[wl.dtype] for v in errs.values()), errs


RAGGED = [
    small("delta-one-token", 1, 2, 1, 128, "bf16", "token", s_in=0.1),
    small("delta-ragged-100", 1, 2, 100, 128, "bf16", "token", s_in=0.1),
    small("delta-ragged-333-head", 2, 2, 333, 128, "bf16", "head"),
    small("delta-ragged-200-64", 1, 3, 200, 64, "bf16", "token", s_in=0.1),
    small("delta-ragged-130-f32", 1, 2, 130, 64, "f32", "token", s_in=0.1),
]


@pytest.mark.parametrize("wl", RAGGED, ids=[w.name for w in RAGGED])
def test_delta_ragged(wl):
    """Lengths that are not whole chunks: the piece's last chunk holds 1..63
    tokens.  Forward and backward against the oracle, as one piece and as
    pieces that end mid-chunk; outputs past the last token are untouched."""
    print(f"case {wl}", flush=True)
    inp = to_dev(make_inputs(wl, device="cpu", seed=12, with_dS_out=True))
    ref = oracle_delta(inp, backward=True)
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    splits = [[wl.T]]
    if wl.T >= 100:
        splits.append([37, wl.T - 37 - 50, 50])
    for lens in splits:
        errs = errors(run_pieces(inp, lens, backward=True), ref, heads)
        print(f"[{wl.name} pieces {lens}] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
              flush=True)
        assert all(v <= TOL[wl.dtype] for v in errs.values()), errs
    # nothing is written past the piece: views into longer buffers keep their fill
    T, fill = wl.T, 7.0
    o = torch.full((wl.B, wl.H, T + 64, wl.dv), fill, dtype=torch.float32, device=DEV)
    dq = torch.full((wl.B, wl.H, T + 64, wl.dk), fill, dtype=torch.float32, device=DEV)
    db = torch.full((wl.B, wl.H, T + 64), fill, dtype=torch.float32, device=DEV)
    _, _, sv = linrec.delta_fwd(inp.q, inp.k, inp.v, inp.beta, inp.decay, inp.S_in, o=o[:, :, :T],
                                save=True)
    linrec.delta_bwd(inp.q, inp.k, inp.v, inp.beta, inp.decay, sv, inp.dO, inp.dS_out,
                     dq=dq[:, :, :T], dbeta=db[:, :, :T], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert bool((o[:, :, T:] == fill).all()) and bool((dq[:, :, T:] == fill).all())
    assert bool((db[:, :, T:] == fill).all())


def run_seq(inp, lengths):
    """The native sequence drivers (linrec_delta_fwd_seq / linrec_delta_bwd_seq),
    fp32 outputs."""
    o, S, saved = linrec.delta_fwd_seq(inp.q, inp.k, inp.v, inp.beta, inp.decay, lengths, inp.S_in,
                                       save=True, out_dtype=torch.float32)
    dq, dk, dv, db, dS = linrec.delta_bwd_seq(inp.q, inp.k, inp.v, inp.beta, inp.decay, lengths, saved,
                                              inp.dO, inp.dS_out, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return {"o": o, "S_out": S, "dq": dq, "dk": dk, "dv": dv, "dbeta": db, "dS_in": dS}


SEQ = [
    (SMALL[0], [64, 64, 128]),
    (SMALL[3], [128, 64, 128]),
    (SMALL[4], [256]),
    (RAGGED[2], [37, 246, 50]),
    (RAGGED[1], [1, 63, 36]),
    (small("delta-seq-many", 1, 2, 640, 128, "bf16", "head", s_in=0.1), [64] * 7 + [100, 92]),
]


@pytest.mark.parametrize("wl,lens", SEQ, ids=[f"{w.name}-{len(l)}" for w, l in SEQ])
def test_delta_sequence_drivers(wl, lens):
    """The sequence drivers overlap the next piece's per-chunk kernels with
    the current piece's serial walk on a second stream; their results equal
    those of the per-piece calls bit for bit, and the oracle's."""
    print(f"case {wl.name} pieces {lens}", flush=True)
    inp = to_dev(make_inputs(wl, device="cpu", seed=13, with_dS_out=True))
    got = run_seq(inp, lens)
    ref = run_pieces(inp, lens, backward=True)
    same = {k: torch.equal(got[k], ref[k]) for k in ref}
    assert all(same.values()), same
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    errs = errors(got, oracle_delta(inp, backward=True), heads)
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert all(v <= TOL[wl.dtype] for v in errs.values()), errs


def test_delta_sequence_drivers_gated_16k():
    """The 16-head, 16K-token gated workload through the sequence drivers, as
    timed: bitwise equal to the per-piece calls, twice in a row (the
    workspace slots reused), and against the oracle on sampled heads."""
    wl = DELTA_WORKLOADS[6]
    lens = wl.pieces()
    inp = make_inputs(wl, device=DEV, with_dS_out=True)
    ref = run_pieces(inp, lens, backward=True)
    for rep in range(2):
        got = run_seq(inp, lens)
        same = {k: torch.equal(got[k], ref[k]) for k in ref}
        print(f"[{wl.name} run {rep}] bitwise equal: {same}", flush=True)
        assert all(same.values()), same
    heads = [(0, 2), (0, 13)]
    errs = errors(got, oracle_delta(inp, heads, backward=True), heads)
    print("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert all(v <= TOL[wl.dtype] for v in errs.values()), errs
