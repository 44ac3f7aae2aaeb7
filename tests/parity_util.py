"""Helpers shared by the GPU parity tests: oracle runs on sampled heads and
the error measures.

err(X) = max |X_gpu - X_oracle| / RMS(X_oracle), per returned tensor; the
bar is 2e-2 for bf16 activations and 1e-4 for fp32 ones.  The oracle eats
the GPU's inputs exactly as stored (bf16 values upcast to fp64), so input
quantisation is not counted as error.

bf16 outputs.  An output stored as bf16 cannot hold the exact result:
rounding the oracle's own fp64 values to bf16 (round to nearest even) already
gives max|err|/RMS of 2.2e-2 to 3.4e-2 on the bf16 workloads, because their
largest elements are 10 to 13 times the RMS and half an ulp is 2^-8 |x|.  No
bf16-output result can meet the plain bar, so three figures are reported for
bf16 outputs:
    plain  = max |X_gpu - X_oracle| / RMS                      (printed)
    floor  = max |rne_bf16(X_oracle) - X_oracle| / RMS         (printed: the
             plain error of a perfect bf16 result)
    excess = max( |X_gpu - X_oracle| - 2^-8 |X_oracle| ) / RMS (asserted <= bar)
and fp32 outputs of the same kernels (no final rounding) are held to the
plain bar.  That the bf16 store itself rounds to nearest even is checked
separately (rne_mismatch): bf16 outputs must equal the fp32 outputs of the
same kernels cast with round to nearest even.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


BF16_HALF_ULP = 2.0 ** -8


def _rms(ref: np.ndarray) -> float:
    return float(np.sqrt(np.mean(ref * ref)))


def rel_err(got: torch.Tensor, ref: np.ndarray) -> float:
    """The asserted measure: plain for fp32 outputs, excess beyond half a
    bf16 ulp for bf16 outputs."""
    g = np64(got)
    allow = BF16_HALF_ULP * np.abs(ref) if got.dtype == torch.bfloat16 else 0.0
    excess = np.maximum(np.abs(g - ref) - allow, 0.0)
    rms = _rms(ref)
    if rms == 0.0:
        return float(np.max(excess))
    return float(np.max(excess) / rms)


def plain_err(got: torch.Tensor, ref: np.ndarray) -> float:
    rms = _rms(ref)
    e = float(np.max(np.abs(np64(got) - ref)))
    return e / rms if rms else e


def bf16_floor(ref: np.ndarray) -> float:
    """max|rne_bf16(ref) - ref| / RMS: what a correctly rounded bf16 result scores."""
    r = torch.from_numpy(ref).to(torch.bfloat16).to(torch.float64).numpy()
    rms = _rms(ref)
    e = float(np.max(np.abs(r - ref)))
    return e / rms if rms else e


def rne_mismatch(out_bf16: torch.Tensor, out_f32: torch.Tensor):
    """Compare a bf16 output with the fp32 output of the same kernels cast to
    bf16 (round to nearest even).  Returns (fraction of elements that differ,
    largest difference in bf16 ulps of the fp32 value)."""
    want = out_f32.to(torch.bfloat16)
    diff = out_bf16.view(torch.int16).to(torch.int32) - want.view(torch.int16).to(torch.int32)
    same_sign = (out_bf16.float() * want.float()) >= 0
    nz = diff != 0
    frac = float(nz.float().mean())
    # bit patterns of same-sign finite bf16 values differ by the ulp count
    ulps = int(diff.abs()[same_sign].max()) if bool(same_sign.any()) else 0
    if bool((nz & ~same_sign).any()):
        ulps = max(ulps, 1 << 16)
    return frac, ulps


def select_heads(x: torch.Tensor | None, heads):
    """x[b, h] for the (b, h) pairs in `heads`, stacked as [1, len(heads), ...]."""
    if x is None:
        return None
    return torch.stack([x[b, h] for b, h in heads]).unsqueeze(0)


def oracle_run(inp, heads=None, want_bwd=True, nthreads=None):
    """Run the oracle on the inputs of the (b, h) pairs in `heads` (all if None).

    Returns dict of float64 arrays shaped [1, len(heads), ...]."""
    wl = inp.wl
    if heads is None:
        heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    pick = lambda x: None if x is None else np.ascontiguousarray(np64(select_heads(x, heads)))  # noqa: E731
    q, k, v, dO = pick(inp.q), pick(inp.k), pick(inp.v), pick(inp.dO)
    S_in = pick(inp.S_in)
    dS_out = pick(inp.dS_out)
    a = None
    if inp.decay is not None:
        if inp.decay.dim() == 1:
            a = np.ascontiguousarray(np.array([float(inp.decay[h]) for _, h in heads]))
        else:
            a = pick(inp.decay)
    o, S_out = oracle.fwd(q, k, v, a, S_in, nthreads=nthreads)
    out = {"o": o, "S_out": S_out}
    if want_bwd:
        dq, dk, dv, dS_in = oracle.bwd(q, k, v, a, S_in, dO, dS_out, nthreads=nthreads)
        out.update(dq=dq, dk=dk, dv=dv, dS_in=dS_in)
    return out


def compare(got: dict, ref: dict, heads, tol: float):
    """Per-tensor errors of GPU outputs (full [B,H,...] tensors) vs oracle.

    Returns (errs, bad, report): errs holds the asserted measure per tensor
    (rel_err), bad those over tol, report a printable line that also gives
    the plain error and, for bf16 outputs, the bf16 floor."""
    errs, parts = {}, []
    for name, r in ref.items():
        g = select_heads(got[name], heads)
        errs[name] = rel_err(g, r)
        if g.dtype == torch.bfloat16:
            parts.append(f"{name}: plain={plain_err(g, r):.2e} floor={bf16_floor(r):.2e} "
                         f"excess={errs[name]:.2e}")
        else:
            parts.append(f"{name}={errs[name]:.2e}")
    bad = {k: v for k, v in errs.items() if not (v <= tol)}
    return errs, bad, " ".join(parts)
