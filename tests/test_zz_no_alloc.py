"""The no-allocation backward (linrec_bwd_noalloc, fixed device scratch)
against linrec_bwd with a caller workspace: identical results on two calls
in a row, the second on a smaller piece, so that the scratch still holds the
first call's records when the second starts."""
import pytest
import torch

from state_passing_amd import linrec
from state_passing_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def case(B, H, T, decay, seed):
    wl = Workload(950, "noalloc", B, H, T, 128, 128, "bf16", decay, s_in_std=0.1, piece=T)
    inp = make_inputs(wl, device="cpu", seed=seed, with_dS_out=True)
    for name in ("q", "k", "v", "dO", "S_in", "decay", "dS_out"):
        x = getattr(inp, name)
        if x is not None:
            setattr(inp, name, x.to(DEV))
    return inp


def test_noalloc_matches_workspace_backward_twice():
    # 16 heads x 4096 tokens (16.8 MB of records), then 2 x 3 heads x 1280
    for B, H, T, decay, seed in ((1, 16, 4096, "head", 3), (2, 3, 1280, "token", 4)):
        print(f"case B={B} H={H} T={T} decay={decay}", flush=True)
        inp = case(B, H, T, decay, seed)
        _, _, st = linrec.fwd(inp.q, inp.k, inp.v, inp.decay, inp.S_in)
        ref = linrec.bwd(inp.q, inp.k, inp.v, inp.decay, st, inp.dO, inp.dS_out)
        out = [torch.empty_like(x) for x in ref]
        got = linrec.bwd_noalloc(inp.q, inp.k, inp.v, inp.decay, st, inp.dO, inp.dS_out,
                                 dq=out[0], dk=out[1], dv=out[2], dS_in=out[3])
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv", "dS_in"), got, ref):
            assert torch.equal(a, b), (T, name)


def test_noalloc_rejects_pieces_over_the_scratch():
    inp = case(1, 16, 8192, "head", 5)
    _, _, st = linrec.fwd(inp.q, inp.k, inp.v, inp.decay, inp.S_in)
    with pytest.raises(linrec.LinrecError, match="LINREC_E_SCRATCH"):
        linrec.bwd_noalloc(inp.q, inp.k, inp.v, inp.decay, st, inp.dO, inp.dS_out)
    torch.cuda.synchronize()
