"""GPU parity at lengths that are not a multiple of the 64-token chunk: a
piece's last chunk holds 1..63 tokens, the rest of it does not exist (its
rows are neither read nor written).  Against the fp64 oracle, which has no
chunks: one token, less than a chunk, several chunks and segments with a
ragged tail, every decay kind, fp32 and bf16, d_k != d_v; pieces with
ragged ends inside a sequence (sequence drivers and the per-piece loop);
splits on segment boundaries bitwise equal to the unsplit run; the
recompute backward bitwise equal to the stored-state one; the decay
gradient with its carry."""
import numpy as np
import pytest
import torch

from parity_util import TOL, compare, oracle_run, rel_err, rne_mismatch
from state_passing_amd import linrec
from state_passing_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def small(name, B, H, T, dk, dv, dtype, decay, s_in=0.0):
    return Workload(902, name, B, H, T, dk, dv, dtype, decay, s_in_std=s_in, piece=T)


RAGGED = [
    small("one-token", 1, 2, 1, 128, 128, "bf16", "token", s_in=0.1),
    small("sub-chunk-63", 2, 2, 63, 64, 64, "f32", "token", s_in=0.1),
    small("two-chunks-100", 1, 3, 100, 128, 128, "bf16", "head", s_in=0.1),
    small("segment-plus-1", 1, 2, 257, 128, 128, "bf16", "none", s_in=0.1),
    small("tail-40-1000", 2, 2, 1000, 128, 128, "bf16", "token", s_in=0.1),
    small("tail-1-2305", 1, 2, 2305, 64, 128, "bf16", "head"),
    small("tail-17-465-128x64", 1, 2, 465, 128, 64, "bf16", "token", s_in=0.1),
]


def gpu_inputs(wl, seed=5):
    inp = make_inputs(wl, device="cpu", seed=seed, with_dS_out=True)
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


def check(got, ref, wl, label):
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    tol = TOL[wl.torch_dtype]
    errs, bad, report = compare(got, ref, heads, tol)
    print(f"[{label}] {wl.name} T={wl.T}: {report}", flush=True)
    assert not bad, f"{label} {wl.name}: over tolerance {tol}: {bad}"


@pytest.mark.parametrize("wl", RAGGED, ids=[w.name for w in RAGGED])
def test_ragged_unsplit(wl):
    print(f"case {wl}", flush=True)
    inp = gpu_inputs(wl)
    ref = oracle_run(inp)
    got32 = run_unsplit(inp, torch.float32)
    check(got32, ref, wl, "unsplit/f32-out")
    if wl.dtype == "bf16":
        got16 = run_unsplit(inp)
        check(got16, ref, wl, "unsplit/bf16-out")
        for name in ("o", "dq", "dk", "dv"):
            frac, ulps = rne_mismatch(got16[name], got32[name])
            assert frac <= 1e-4 and ulps <= 1, (name, frac, ulps)


def test_ragged_outputs_stop_at_the_last_token():
    """Rows past the end of a ragged piece are never written: an output
    buffer one chunk longer keeps its fill there."""
    wl = RAGGED[4]
    inp = gpu_inputs(wl)
    T = wl.T
    pad = 64
    fill = 7.0
    o = torch.full((wl.B, wl.H, T + pad, wl.dv), fill, dtype=torch.float32, device=DEV)
    dq = torch.full((wl.B, wl.H, T + pad, wl.dk), fill, dtype=torch.float32, device=DEV)
    _, _, st = linrec.fwd(inp.q, inp.k, inp.v, inp.decay, inp.S_in, o=o[:, :, :T])
    linrec.bwd(inp.q, inp.k, inp.v, inp.decay, st, inp.dO, inp.dS_out, dq=dq[:, :, :T])
    torch.cuda.synchronize()
    assert bool((o[:, :, T:] == fill).all()) and bool((dq[:, :, T:] == fill).all())
    assert not bool((o[:, :, :T] == fill).any())


SPLITS = {
    "tail-40-1000": {"ragged-pieces": [37, 500, 463], "aligned": [256, 744], "aligned2": [512, 488],
                     "many": [100, 156, 1, 63, 680]},
    "tail-1-2305": {"ragged-pieces": [1000, 1, 1304], "aligned": [768, 1024, 513]},
    "tail-17-465-128x64": {"ragged-pieces": [65, 400], "aligned": [256, 209]},
    "two-chunks-100": {"ragged-pieces": [1, 99], "two": [50, 50]},
}


@pytest.mark.parametrize("name", sorted(SPLITS))
def test_ragged_splits(name):
    """Pieces that end mid-chunk inside the sequence, through the sequence
    drivers and the per-piece loop, against the oracle; splits whose cuts
    fall on segment boundaries (multiples of 256) equal the unsplit run bit
    for bit."""
    wl = next(w for w in RAGGED if w.name == name)
    inp = gpu_inputs(wl)
    ref = oracle_run(inp)
    base = run_unsplit(inp, torch.float32)
    for sname, lengths in SPLITS[name].items():
        assert sum(lengths) == wl.T
        aligned = all(L % 256 == 0 for L in lengths[:-1])
        for runner in (run_seq, run_loop):
            got = runner(inp, lengths, torch.float32)
            check(got, ref, wl, f"{runner.__name__}/{sname}")
            same = {k: bool(torch.equal(got[k], base[k])) for k in got}
            print(f"  segment-aligned={aligned} bitwise equal to unsplit: {same}", flush=True)
            if aligned:
                assert all(same.values()), same


@pytest.mark.parametrize("wl", [RAGGED[2], RAGGED[4], RAGGED[5]], ids=lambda w: w.name)
def test_ragged_recompute_equals_stored_states(wl):
    inp = gpu_inputs(wl)
    o, S_out, st = linrec.fwd(inp.q, inp.k, inp.v, inp.decay, inp.S_in)
    ref = linrec.bwd(inp.q, inp.k, inp.v, inp.decay, st, inp.dO, inp.dS_out)
    got = linrec.bwd_recompute(inp.q, inp.k, inp.v, inp.decay, inp.S_in, inp.dO, inp.dS_out)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv", "dS_in"), got, ref):
        assert torch.equal(a, b), name


@pytest.mark.parametrize("wl", [RAGGED[0], RAGGED[2], RAGGED[4], RAGGED[6]], ids=lambda w: w.name)
def test_ragged_decay_gradient(wl):
    """The decay gradient at a ragged length and, for the longer case, over
    ragged pieces with the carry handed back."""
    import oracle
    from parity_util import np64
    inp = gpu_inputs(wl)
    f = lambda x: None if x is None else np.ascontiguousarray(np64(x))  # noqa: E731
    q, k, v, a, S_in, dO, dS_out = (f(x) for x in (inp.q, inp.k, inp.v, inp.decay, inp.S_in,
                                                   inp.dO, inp.dS_out))
    _, S_out = oracle.fwd(q, k, v, a, S_in)
    *_, da_ref = oracle.bwd(q, k, v, a, S_in, dO, dS_out, want_da=True)
    carry = torch.tensor(np.sum(dS_out * S_out, axis=(-2, -1)), dtype=torch.float32, device=DEV)
    lengths = [wl.T] if wl.T < 300 else [37, wl.T - 37 - 300, 300]
    bounds = np.cumsum([0] + lengths)
    S, stores = inp.S_in, []
    for i in range(len(lengths)):
        sl = slice(int(bounds[i]), int(bounds[i + 1]))
        _, S, st = linrec.fwd(inp.q[:, :, sl], inp.k[:, :, sl], inp.v[:, :, sl],
                              inp.decay[:, :, sl] if inp.decay.dim() == 3 else inp.decay, S,
                              out_dtype=torch.float32)
        stores.append(st)
    da = torch.empty(wl.B, wl.H, wl.T, dtype=torch.float32, device=DEV)
    dS, c = inp.dS_out, carry
    for i in reversed(range(len(lengths))):
        sl = slice(int(bounds[i]), int(bounds[i + 1]))
        dec = inp.decay[:, :, sl] if inp.decay.dim() == 3 else inp.decay
        _, _, _, dS, _, c = linrec.bwd_da(inp.q[:, :, sl], inp.k[:, :, sl], inp.v[:, :, sl], dec,
                                          stores[i], inp.dO[:, :, sl], dS, c, da=da[:, :, sl],
                                          da_carry_out=c, out_dtype=torch.float32)
    torch.cuda.synchronize()
    err = rel_err(da, da_ref)
    print(f"[ragged-da] {wl.name} pieces {lengths}: da={err:.2e}", flush=True)
    assert err <= TOL[wl.torch_dtype], err


def test_empty_piece_passes_the_carry_through():
    """T = 0: S_out = S_in, dS_in = dS_out, the decay-gradient carry passes
    unchanged (a NULL input gives zeros), for every per-piece call; a
    zero-length piece inside the per-piece loop changes nothing."""
    B, H, dk, dv = 2, 3, 128, 128
    g = torch.Generator().manual_seed(11)
    S = torch.randn(B, H, dk, dv, generator=g).to(DEV)
    dS = torch.randn(B, H, dk, dv, generator=g).to(DEV)
    carry = torch.randn(B, H, generator=g).to(DEV)
    q = torch.empty(B, H, 0, dk, dtype=torch.bfloat16, device=DEV)
    v = torch.empty(B, H, 0, dv, dtype=torch.bfloat16, device=DEV)
    dec = torch.empty(B, H, 0, dtype=torch.float32, device=DEV)
    print("case empty piece B=2 H=3 d=128", flush=True)
    o, S_out, st = linrec.fwd(q, q, v, dec, S)
    _, S_zero, _ = linrec.fwd(q, q, v, dec, None)
    dq, dk_, dv_, dS_in = linrec.bwd(q, q, v, dec, st, v, dS)
    _, _, _, dS_rec = linrec.bwd_recompute(q, q, v, dec, S, v, dS)
    _, _, _, dS_na = linrec.bwd_noalloc(q, q, v, dec, st, v, dS)
    _, _, _, dS_da, da, c_out = linrec.bwd_da(q, q, v, dec, st, v, dS, carry)
    _, _, _, _, _, c_zero = linrec.bwd_da(q, q, v, dec, st, v, None, None)
    beta = torch.empty(B, H, 0, dtype=torch.float32, device=DEV)
    _, S_delta, saved = linrec.delta_fwd(q, q, v, beta, dec, S, save=True)
    *_, dS_delta = linrec.delta_bwd(q, q, v, beta, dec, saved, v, dS)
    torch.cuda.synchronize()
    assert o.numel() == 0 and dq.numel() == 0 and da.numel() == 0
    for got in (S_out, S_delta):
        assert torch.equal(got, S)
    for got in (dS_in, dS_rec, dS_na, dS_da, dS_delta):
        assert torch.equal(got, dS)
    assert torch.equal(c_out, carry)
    assert not bool(S_zero.any()) and not bool(c_zero.any())

    wl = RAGGED[4]
    inp = gpu_inputs(wl)
    base = run_loop(inp, [256, 744], torch.float32)
    got = run_loop(inp, [256, 0, 744], torch.float32)
    same = {k: bool(torch.equal(got[k], base[k])) for k in got}
    print(f"  loop with an empty piece bitwise equal: {same}", flush=True)
    assert all(same.values()), same
