"""Seeded synthetic workloads for the linear-recurrence layer.

This module only draws inputs: it holds none of the layer's arithmetic, so
both the HIP path and the CPU oracle can be fed from it.  The pages train
linear-recurrence models on a public text corpus; neither data nor trained
weights are used here.  Gaussian activations with the shapes below stand in
for a layer's q, k, v and upstream gradient.

Workloads (sizes from the five configurations this layer is measured on):

  1 tiny-fp32      B=1 H=2  T=1024   d=64  fp32, a_t = 1, split 4 x 256
  2 decay-16k      B=1 H=16 T=16384  d=128 bf16, per-head decay, 4 x 4096
  3 sa-256k        B=1 H=16 T=262144 d=128 bf16, per-head decay, 64 x 4096
  4 nonuniform     B=1 H=32 T=262144 d=128 bf16, per-head decay, S_in~N(0,0.1^2),
                   seeded random piece lengths (multiples of 64 in [2048, 32768])
  5 gated-batch    B=8 H=32 T=32768  d=128 bf16, per-token gate, 8 x 4096

Recipe (all draws seeded, in this order: q, k, v, dO, S_in, gate logits,
dS_out when asked for, beta logits for the delta rule):
  q, k  ~ N(0, I) per token in fp32, divided by their L2 norm, then cast to
        the workload dtype (round to nearest even);
  v, dO ~ N(0, 1), cast the same way;
  S_in  ~ N(0, s^2) fp32 with s = 0.1 for workload 4, else zeros;
  per-head decay a_h = 1 - 2^-(5 + 8h/H), h = 0..H-1, stored as fp32;
  per-token gate a = 0.9 + 0.1 * sigmoid(x), x ~ N(2, 1), fp32;
  delta rule: beta = sigmoid(y), y ~ N(0, 1), fp32 [B,H,T].
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

CHUNK = 64


@dataclass(frozen=True)
class Workload:
    idx: int
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    dtype: str            # "bf16" | "f32"
    decay: str            # "none" | "head" | "token"
    s_in_std: float = 0.0
    piece: int = 4096     # uniform piece length (ignored when random_split)
    random_split: bool = False
    delta: bool = False   # gated delta rule: also draw the write strengths beta

    @property
    def seed(self) -> int:
        return 1000 + self.idx

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def pieces(self) -> List[int]:
        """Sub-sequence lengths, in order; they sum to T."""
        if self.random_split:
            return random_split(self.T, self.seed)
        return [self.piece] * (self.T // self.piece)

    def scaled(self, **kw) -> "Workload":
        """A copy with some fields replaced (smaller parity cases)."""
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    1: Workload(1, "tiny-fp32", 1, 2, 1024, 64, 64, "f32", "none", piece=256),
    2: Workload(2, "decay-16k", 1, 16, 16384, 128, 128, "bf16", "head", piece=4096),
    3: Workload(3, "sa-256k", 1, 16, 262144, 128, 128, "bf16", "head", piece=4096),
    4: Workload(4, "nonuniform-256k", 1, 32, 262144, 128, 128, "bf16", "head",
                s_in_std=0.1, random_split=True),
    5: Workload(5, "gated-batch", 8, 32, 32768, 128, 128, "bf16", "token", piece=4096),
}

# Gated delta rule (the Gated DeltaNet recurrence StateFlow trains): the
# gated-batch recipe per head at the 16-head, 16K-token shape, plus write
# strengths beta = sigmoid(y), y ~ N(0, 1), drawn last.
DELTA_WORKLOADS = {
    6: Workload(6, "delta-gated-16k", 1, 16, 16384, 128, 128, "bf16", "token", piece=4096,
                delta=True),
}


def random_split(T: int, seed: int, lo: int = 2048, hi: int = 32768) -> List[int]:
    """Seeded piece lengths: multiples of 64 in [lo, hi] that sum to T.

    While more than `hi` tokens remain, draw a length uniformly among the
    multiples of 64 that leave at least `lo` tokens; the remainder is the
    last piece.
    """
    assert T % CHUNK == 0 and T >= lo
    rng = np.random.default_rng(seed)
    out, R = [], T
    while R > hi:
        top = min(hi // CHUNK, (R - lo) // CHUNK)
        L = CHUNK * int(rng.integers(lo // CHUNK, top, endpoint=True))
        out.append(L)
        R -= L
    out.append(R)
    return out


def head_decay(H: int) -> torch.Tensor:
    """a_h = 1 - 2^-(5 + 8h/H) for h = 0..H-1, rounded to fp32."""
    h = np.arange(H, dtype=np.float64)
    return torch.from_numpy(1.0 - np.exp2(-(5.0 + 8.0 * h / H))).to(torch.float32)


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)


@dataclass
class Inputs:
    wl: Workload
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    dO: torch.Tensor
    S_in: Optional[torch.Tensor]          # fp32 [B,H,dk,dv] or None (zeros)
    decay: Optional[torch.Tensor]         # fp32 [H] or [B,H,T], None for a_t = 1
    dS_out: Optional[torch.Tensor] = None  # fp32 [B,H,dk,dv] or None (zeros)
    beta: Optional[torch.Tensor] = None    # fp32 [B,H,T] (delta rule) or None
    extra: dict = field(default_factory=dict)


def make_inputs(wl: Workload, device="cpu", seed: Optional[int] = None,
                with_dS_out: bool = False) -> Inputs:
    """Draw one workload's inputs on `device` with a seeded generator.

    `with_dS_out` adds a seeded N(0,1) dS_out (tests of that input); the
    workloads themselves end with dS_out = 0.
    """
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed if seed is None else seed)
    B, H, T, dk, dv = wl.B, wl.H, wl.T, wl.dk, wl.dv
    dt = wl.torch_dtype

    def randn(*shape):
        return torch.randn(*shape, generator=g, device=dev, dtype=torch.float32)

    q = _unit_rows(randn(B, H, T, dk)).to(dt)
    k = _unit_rows(randn(B, H, T, dk)).to(dt)
    v = randn(B, H, T, dv).to(dt)
    dO = randn(B, H, T, dv).to(dt)
    S_in = None
    if wl.s_in_std > 0:
        S_in = randn(B, H, dk, dv) * wl.s_in_std
    decay = None
    if wl.decay == "head":
        decay = head_decay(H).to(dev)
    elif wl.decay == "token":
        x = randn(B, H, T) + 2.0
        decay = 0.9 + 0.1 * torch.sigmoid(x)
    dS_out = randn(B, H, dk, dv) if with_dS_out else None
    beta = torch.sigmoid(randn(B, H, T)) if wl.delta else None
    return Inputs(wl, q, k, v, dO, S_in, decay, dS_out, beta)
