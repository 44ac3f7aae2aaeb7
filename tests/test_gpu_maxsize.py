"""GPU parity past 2^31 elements per tensor.

One head of T = 2^24 + 37 tokens at d_k = d_v = 128 bf16: q, k, v, dO and
every output hold 2^31 + 4736 elements, and one head's T * d alone passes
2^31, so every token offset the kernels form is beyond 32 bits for most of
the sequence.  One unsplit piece with a ragged last chunk (37 tokens),
fp32 outputs.

The oracle checks both ends of every output.  With the per-head decay
a = 1 - 2^-5 of a one-head workload, a token 1024 positions away weighs
a^1024 ~ 8e-15 against the near ones, so the first 2048 tokens (from
S_in = 0) and the last 2048 (from a zero state, ending at dS_out) are
problems the oracle solves exactly up to that weight: o and dq of the
last 1024 tokens, dk and dv of all of the last 2048, S_out; o and dq of
the first 2048 tokens, dk and dv of the first 1024, dS_in.  The whole
sequence would take the oracle minutes, so only these samples are
compared."""
import numpy as np
import pytest
import torch

import oracle
from parity_util import TOL, np64, rel_err
from state_passing_amd import linrec
from state_passing_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
T = (1 << 24) + 37
WIN = 2048


def test_one_head_past_2_31_elements():
    wl = Workload(910, "one-head-16m", 1, 1, T, 128, 128, "bf16", "head", piece=T)
    print(f"case {wl.name}: B=1 H=1 T={T} d=128 bf16, fp32 outputs, per-head decay", flush=True)
    inp = make_inputs(wl, device=DEV, seed=7, with_dS_out=True)
    assert abs(float(inp.decay[0]) - (1 - 2 ** -5)) < 1e-7
    assert inp.q.numel() > 2 ** 31 and T * 128 > 2 ** 31
    o, S_out, st = linrec.fwd(inp.q, inp.k, inp.v, inp.decay, None, out_dtype=torch.float32)
    dq, dk, dv, dS_in = linrec.bwd(inp.q, inp.k, inp.v, inp.decay, st, inp.dO, inp.dS_out,
                                   out_dtype=torch.float32)
    torch.cuda.synchronize()
    print("gpu done", flush=True)
    del st

    a = np.ascontiguousarray(np64(inp.decay))
    win = lambda x, sl: np.ascontiguousarray(np64(x[:, :, sl]))  # noqa: E731
    tol = TOL[torch.float32]
    errs = {}

    # the first WIN tokens, from S_in = 0, gradient beyond them neglected
    head = slice(0, WIN)
    q, k, v, dO = (win(x, head) for x in (inp.q, inp.k, inp.v, inp.dO))
    ro, _ = oracle.fwd(q, k, v, a, None)
    rdq, rdk, rdv, rdS = oracle.bwd(q, k, v, a, None, dO, None)
    errs["o[head]"] = rel_err(o[:, :, head], ro)
    errs["dq[head]"] = rel_err(dq[:, :, head], rdq)
    errs["dk[head/2]"] = rel_err(dk[:, :, :WIN // 2], rdk[:, :, :WIN // 2])
    errs["dv[head/2]"] = rel_err(dv[:, :, :WIN // 2], rdv[:, :, :WIN // 2])
    errs["dS_in"] = rel_err(dS_in, rdS)

    # the last WIN tokens, from a zero state, ending at dS_out
    tail = slice(T - WIN, T)
    q, k, v, dO = (win(x, tail) for x in (inp.q, inp.k, inp.v, inp.dO))
    dS_out = np.ascontiguousarray(np64(inp.dS_out))
    ro, rS = oracle.fwd(q, k, v, a, None)
    rdq, rdk, rdv, _ = oracle.bwd(q, k, v, a, None, dO, dS_out)
    late = slice(T - WIN // 2, T)
    errs["o[tail/2]"] = rel_err(o[:, :, late], ro[:, :, WIN // 2:])
    errs["dq[tail/2]"] = rel_err(dq[:, :, late], rdq[:, :, WIN // 2:])
    errs["dk[tail]"] = rel_err(dk[:, :, tail], rdk)
    errs["dv[tail]"] = rel_err(dv[:, :, tail], rdv)
    errs["S_out"] = rel_err(S_out, rS)

    print("  " + "  ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"over {tol}: {bad}"
