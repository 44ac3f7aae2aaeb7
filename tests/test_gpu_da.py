"""GPU parity of the decay gradient (linrec_bwd_da) against the fp64 oracle:
per-token and per-head decay, nonzero S_in and dS_out, d_k != d_v, fp32,
one piece and a sequence of pieces with the carry passed back."""
import numpy as np
import pytest
import torch

import oracle
from parity_util import TOL, np64, rel_err
from state_passing_amd import linrec
from state_passing_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def small(name, B, H, T, dk, dv, dtype, decay, s_in=0.0):
    return Workload(901, name, B, H, T, dk, dv, dtype, decay, s_in_std=s_in, piece=T)


CASES = [
    small("da-token", 2, 3, 384, 128, 128, "bf16", "token", s_in=0.1),
    small("da-head", 1, 2, 512, 128, 128, "bf16", "head", s_in=0.1),
    small("da-f32-token", 1, 2, 256, 64, 64, "f32", "token", s_in=0.1),
    small("da-long", 1, 2, 2304, 128, 128, "bf16", "token"),
    small("da-64x128", 1, 2, 320, 64, 128, "bf16", "token", s_in=0.1),
    small("da-128x64", 1, 2, 320, 128, 64, "bf16", "token", s_in=0.1),
]


def inputs(wl, seed=17):
    inp = make_inputs(wl, device="cpu", seed=seed, with_dS_out=True)
    for name in ("q", "k", "v", "dO", "S_in", "decay", "dS_out"):
        x = getattr(inp, name)
        if x is not None:
            setattr(inp, name, x.to(DEV))
    return inp


def oracle_da(inp):
    f = lambda x: None if x is None else np.ascontiguousarray(np64(x))  # noqa: E731
    q, k, v, a, S_in, dO, dS_out = (f(x) for x in (inp.q, inp.k, inp.v, inp.decay, inp.S_in,
                                                   inp.dO, inp.dS_out))
    _, S_out = oracle.fwd(q, k, v, a, S_in)
    dq, dk, dv, dS_in, da = oracle.bwd(q, k, v, a, S_in, dO, dS_out, want_da=True)
    carry = np.sum(dS_out * S_out, axis=(-2, -1)) if dS_out is not None else None
    return dict(dq=dq, dk=dk, dv=dv, dS_in=dS_in, da=da), carry, a


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_decay_gradient_one_piece(wl):
    print(f"case {wl}", flush=True)
    inp = inputs(wl)
    ref, carry, a = oracle_da(inp)
    carry_t = torch.tensor(carry, dtype=torch.float32, device=DEV)
    o, S_out, st = linrec.fwd(inp.q, inp.k, inp.v, inp.decay, inp.S_in, out_dtype=torch.float32)
    dq, dk, dv, dS_in, da, cout = linrec.bwd_da(inp.q, inp.k, inp.v, inp.decay, st, inp.dO,
                                                inp.dS_out, carry_t, out_dtype=torch.float32)
    base = linrec.bwd(inp.q, inp.k, inp.v, inp.decay, st, inp.dO, inp.dS_out,
                      out_dtype=torch.float32)
    torch.cuda.synchronize()
    for name, x, y in zip(("dq", "dk", "dv", "dS_in"), (dq, dk, dv, dS_in), base):
        assert torch.equal(x, y), name
    tol = TOL[wl.torch_dtype]
    err = rel_err(da, ref["da"])
    # the carry for an earlier piece is a_0 da_0 (the sum of g over the whole
    # piece and the carry in), measured against the scale of a_t da_t
    af = a if a.ndim == 3 else np.broadcast_to(a[None, :, None], ref["da"].shape)
    ada = af * ref["da"]
    cerr = float(np.max(np.abs(np64(cout) - ada[:, :, 0])) / np.sqrt(np.mean(ada * ada)))
    print(f"[{wl.name}] da={err:.2e} carry_out={cerr:.2e}", flush=True)
    assert err <= tol and cerr <= tol, (err, cerr)


def test_decay_gradient_strong_decay():
    """Per-token decays in [0.3, 1): chunks on both sides of the threshold
    below which the mask is taken one exp per entry."""
    wl = small("da-strong", 1, 2, 512, 128, 128, "bf16", "token", s_in=0.1)
    inp = inputs(wl)
    g = torch.Generator().manual_seed(37)
    inp.decay = (0.3 + 0.7 * torch.rand(tuple(inp.decay.shape), generator=g)).to(DEV)
    ref, carry, a = oracle_da(inp)
    _, _, st = linrec.fwd(inp.q, inp.k, inp.v, inp.decay, inp.S_in, out_dtype=torch.float32)
    carry_t = torch.tensor(carry, dtype=torch.float32, device=DEV)
    da, cout = linrec.bwd_da(inp.q, inp.k, inp.v, inp.decay, st, inp.dO, inp.dS_out, carry_t,
                             out_dtype=torch.float32)[4:]
    torch.cuda.synchronize()
    err = rel_err(da, ref["da"])
    ada = a * ref["da"]
    cerr = float(np.max(np.abs(np64(cout) - ada[:, :, 0])) / np.sqrt(np.mean(ada * ada)))
    print(f"[da-strong] da={err:.2e} carry_out={cerr:.2e}", flush=True)
    assert err <= TOL[torch.bfloat16] and cerr <= TOL[torch.bfloat16], (err, cerr)


def test_decay_gradient_sequence_with_carry():
    """Pieces in reverse with dS and the decay-gradient carry handed back give
    the unsplit oracle's da over the whole sequence."""
    wl = small("da-seq", 1, 2, 2048, 128, 128, "bf16", "token", s_in=0.1)
    inp = inputs(wl)
    ref, carry, _ = oracle_da(inp)
    lengths = [512, 1024, 256, 256]
    bounds = np.cumsum([0] + lengths)
    q, k, v, dO, a = inp.q, inp.k, inp.v, inp.dO, inp.decay
    S = inp.S_in
    stores = []
    for i in range(len(lengths)):
        sl = slice(int(bounds[i]), int(bounds[i + 1]))
        _, S, st = linrec.fwd(q[:, :, sl], k[:, :, sl], v[:, :, sl], a[:, :, sl], S,
                              out_dtype=torch.float32)
        stores.append(st)
    da = torch.empty(wl.B, wl.H, wl.T, dtype=torch.float32, device=DEV)
    dS = inp.dS_out
    c = torch.tensor(carry, dtype=torch.float32, device=DEV)
    for i in reversed(range(len(lengths))):
        sl = slice(int(bounds[i]), int(bounds[i + 1]))
        _, _, _, dS, _, c = linrec.bwd_da(q[:, :, sl], k[:, :, sl], v[:, :, sl], a[:, :, sl],
                                          stores[i], dO[:, :, sl], dS, c, da=da[:, :, sl],
                                          da_carry_out=c, out_dtype=torch.float32)
    torch.cuda.synchronize()
    err = rel_err(da, ref["da"])
    print(f"[da-seq] da={err:.2e}", flush=True)
    assert err <= TOL[torch.bfloat16], err


def test_decay_gradient_gated_32k():
    """The gated-batch shape (per-token gate, 8 pieces of 4096) on two (b, h)
    pairs, whole sequence against the oracle."""
    wl = Workload(905, "da-gated-32k", 2, 1, 32768, 128, 128, "bf16", "token")
    inp = inputs(wl, seed=5)
    ref, carry, _ = oracle_da(inp)
    L = 4096
    q, k, v, dO, a = inp.q, inp.k, inp.v, inp.dO, inp.decay
    S = inp.S_in
    stores = []
    for i in range(wl.T // L):
        sl = slice(i * L, (i + 1) * L)
        _, S, st = linrec.fwd(q[:, :, sl], k[:, :, sl], v[:, :, sl], a[:, :, sl], S)
        stores.append(st)
    da = torch.empty(wl.B, wl.H, wl.T, dtype=torch.float32, device=DEV)
    dS = inp.dS_out
    c = torch.tensor(carry, dtype=torch.float32, device=DEV)
    for i in reversed(range(wl.T // L)):
        sl = slice(i * L, (i + 1) * L)
        _, _, _, dS, _, c = linrec.bwd_da(q[:, :, sl], k[:, :, sl], v[:, :, sl], a[:, :, sl],
                                          stores[i], dO[:, :, sl], dS, c, da=da[:, :, sl],
                                          da_carry_out=c)
    torch.cuda.synchronize()
    err = rel_err(da, ref["da"])
    print(f"[da-gated-32k] da={err:.2e}", flush=True)
    assert err <= TOL[torch.bfloat16], err
