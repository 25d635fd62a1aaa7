"""Seeded synthetic inputs for the AG+GEMM and GEMM+RS workloads.

This module only draws random numbers and lays them out: it holds none of the operations'
arithmetic, and both the HIP path and the CPU oracle consume what it makes.  Everything is drawn on
the CPU from torch.Generator('cpu').manual_seed(seed), in a fixed order: the weight first (A or W),
then the activation chunks in rank order 0..tp-1 (or X), then the peer partials in increasing rank.
Values are drawn in fp32 and rounded to bf16 (nearest even), or quantised to OCP E4M3 with one
fp32 scale per tensor (scale = amax / 448, codes = the value / scale clamped to +-448 and rounded to
nearest even by torch's cast).

The named workloads are the five shapes this library is measured and checked on:
  ag_tiny   AG+GEMM tp=2 self=0: A [256, 256], 2 chunks [256, 256], U[-1, 1], D [512, 256] bf16
  ag_4k     AG+GEMM tp=4 self=1: M=K=N=4096, 4 chunks [1024, 4096], N(0,1)/sqrt(K), bf16
  rs_8k     GEMM+RS one rank of tp=8: X [8192, 1024], W [8192, 1024] bf16, N(0,1)/sqrt(8192);
            7 peer partials [8192, 8192] fp32 N(0,1)/256 whose rows outside this rank's chunk are
            NaN; D [1024, 8192] bf16
  ag_qkv    AG+GEMM tp=8 self=5: 8 chunks [1024, 8192], A [3072, 8192], N(0,1)/sqrt(8192), bf16
  ag_fc1_f8 AG+GEMM tp=8 self=0, E4M3: 8 chunks [2048, 8192], A [3584, 8192], N(0,1) quantised
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch

E4M3_MAX = 448.0


@dataclass(frozen=True)
class AGShape:
    name: str
    tp: int
    self_rank: int
    nc: int           # rows per chunk
    K: int
    M: int            # output columns (weight rows)
    dtype: str        # "bf16" | "fp8"
    dist: str         # "uniform1" | "normal_sqrtk" | "normal" | "int3"
    seed: int

    @property
    def N(self) -> int:
        return self.tp * self.nc

    @property
    def flops(self) -> float:
        return 2.0 * self.N * self.M * self.K


@dataclass(frozen=True)
class RSShape:
    name: str
    tp: int
    self_rank: int
    T: int            # tokens (rows of X), T = tp * nc
    Kl: int           # local contraction dim
    Mo: int           # output columns
    dist: str         # "normal_rs" | "int3"
    seed: int

    @property
    def nc(self) -> int:
        return self.T // self.tp

    @property
    def flops(self) -> float:
        return 2.0 * self.T * self.Mo * self.Kl


WORKLOADS = {
    "ag_tiny": AGShape("ag_tiny", tp=2, self_rank=0, nc=256, K=256, M=256, dtype="bf16",
                       dist="uniform1", seed=1001),
    "ag_4k": AGShape("ag_4k", tp=4, self_rank=1, nc=1024, K=4096, M=4096, dtype="bf16",
                     dist="normal_sqrtk", seed=1002),
    "rs_8k": RSShape("rs_8k", tp=8, self_rank=0, T=8192, Kl=1024, Mo=8192, dist="normal_rs",
                     seed=1003),
    "ag_qkv": AGShape("ag_qkv", tp=8, self_rank=5, nc=1024, K=8192, M=3072, dtype="bf16",
                      dist="normal_sqrtk", seed=1004),
    "ag_fc1_f8": AGShape("ag_fc1_f8", tp=8, self_rank=0, nc=2048, K=8192, M=3584, dtype="fp8",
                         dist="normal", seed=1005),
}


def _draw(g: torch.Generator, shape, dist: str, k_for_scale: int) -> torch.Tensor:
    if dist == "uniform1":
        return torch.rand(shape, generator=g, dtype=torch.float32) * 2.0 - 1.0
    if dist == "normal_sqrtk":
        return torch.randn(shape, generator=g, dtype=torch.float32) / math.sqrt(k_for_scale)
    if dist == "normal":
        return torch.randn(shape, generator=g, dtype=torch.float32)
    if dist == "int3":
        return torch.randint(-3, 4, shape, generator=g).to(torch.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def quantize_e4m3(x: torch.Tensor):
    """Per-tensor E4M3 quantisation of an fp32 tensor: (codes as torch.float8_e4m3fn, scale).
    dequantised value = float(code) * scale."""
    amax = float(x.abs().max()) if x.numel() else 0.0
    scale = amax / E4M3_MAX if amax > 0 else 1.0
    q = (x / scale).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q, float(scale)


@dataclass
class AGInputs:
    shape: AGShape
    A: torch.Tensor                       # [M, K] bf16, or float8_e4m3fn
    chunks: List[torch.Tensor]            # tp x [nc, K]
    scale_A: Optional[float] = None       # fp8 only
    scale_B: Optional[float] = None       # fp8 only (one scale for the gathered tensor)


def make_ag(shape: AGShape) -> AGInputs:
    g = torch.Generator("cpu").manual_seed(shape.seed)
    a = _draw(g, (shape.M, shape.K), shape.dist, shape.K)
    b = [_draw(g, (shape.nc, shape.K), shape.dist, shape.K) for _ in range(shape.tp)]
    if shape.dtype == "bf16":
        return AGInputs(shape, a.to(torch.bfloat16), [c.to(torch.bfloat16) for c in b])
    if shape.dtype == "fp8":
        if shape.dist == "int3":
            # small integers are exact E4M3 codes with scale 1
            return AGInputs(shape, a.to(torch.float8_e4m3fn),
                            [c.to(torch.float8_e4m3fn) for c in b], 1.0, 1.0)
        qa, sa = quantize_e4m3(a)
        # one scale for the whole gathered input: every rank quantises with the tensor's amax
        amax_b = max(float(c.abs().max()) for c in b)
        sb = amax_b / E4M3_MAX if amax_b > 0 else 1.0
        qb = [(c / sb).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn) for c in b]
        return AGInputs(shape, qa, qb, sa, sb)
    raise ValueError(shape.dtype)


@dataclass
class RSInputs:
    shape: RSShape
    X: torch.Tensor                       # [T, Kl] bf16
    W: torch.Tensor                       # [Mo, Kl] bf16
    partials: List[Optional[torch.Tensor]] = field(default_factory=list)  # [T, Mo] fp32, self None


def make_rs(shape: RSShape, poison_outside_chunk: bool = True) -> RSInputs:
    """Peer partials: rank p's fp32 [T, Mo] partial output.  Only rows of this rank's chunk are read
    by a reduce-scatter; the other rows are filled with NaN so that reading them shows up."""
    g = torch.Generator("cpu").manual_seed(shape.seed)
    if shape.dist == "normal_rs":
        w = torch.randn((shape.Mo, shape.Kl), generator=g) / math.sqrt(shape.tp * shape.Kl)
        x = torch.randn((shape.T, shape.Kl), generator=g) / math.sqrt(shape.tp * shape.Kl)
    else:
        w = _draw(g, (shape.Mo, shape.Kl), shape.dist, shape.Kl)
        x = _draw(g, (shape.T, shape.Kl), shape.dist, shape.Kl)
    nc = shape.nc
    s = shape.self_rank
    partials: List[Optional[torch.Tensor]] = []
    for p in range(shape.tp):
        if p == s:
            partials.append(None)
            continue
        if poison_outside_chunk:
            part = torch.full((shape.T, shape.Mo), float("nan"), dtype=torch.float32)
            rows = (nc, shape.Mo)
        else:
            part = torch.empty((shape.T, shape.Mo), dtype=torch.float32)
            rows = None
        if shape.dist == "normal_rs":
            blk = torch.randn(rows or (shape.T, shape.Mo), generator=g) / 256.0
        else:
            blk = _draw(g, rows or (shape.T, shape.Mo), shape.dist, shape.Kl)
        if rows:
            part[s * nc:(s + 1) * nc] = blk
        else:
            part.copy_(blk)
        partials.append(part)
    return RSInputs(shape, x.to(torch.bfloat16), w.to(torch.bfloat16), partials)


@dataclass
class RSRingInputs:
    shape: RSShape
    X: torch.Tensor                       # [T, Kl] bf16
    W: torch.Tensor                       # [Mo, Kl] bf16
    incoming: List[torch.Tensor] = field(default_factory=list)   # tp x [nc, Mo] fp32, by chunk


def make_rs_ring(shape: RSShape) -> RSRingInputs:
    """Inputs of one ring-accumulate reduce-scatter step: X and W drawn as in make_rs, then one
    fp32 [nc, Mo] incoming running sum per chunk, in increasing chunk index (the step ignores the
    entry of the chain that starts at this rank; it is drawn like the others)."""
    g = torch.Generator("cpu").manual_seed(shape.seed)
    if shape.dist == "normal_rs":
        w = torch.randn((shape.Mo, shape.Kl), generator=g) / math.sqrt(shape.tp * shape.Kl)
        x = torch.randn((shape.T, shape.Kl), generator=g) / math.sqrt(shape.tp * shape.Kl)
        inc = [torch.randn((shape.nc, shape.Mo), generator=g) / 256.0 for _ in range(shape.tp)]
    else:
        w = _draw(g, (shape.Mo, shape.Kl), shape.dist, shape.Kl)
        x = _draw(g, (shape.T, shape.Kl), shape.dist, shape.Kl)
        inc = [_draw(g, (shape.nc, shape.Mo), shape.dist, shape.Kl) for _ in range(shape.tp)]
    return RSRingInputs(shape, x.to(torch.bfloat16), w.to(torch.bfloat16),
                        [t.to(torch.float32) for t in inc])


def make_reduced_chunks(shape: RSShape) -> List[torch.Tensor]:
    """The owners' reduced output chunks that an all-gather brings to this rank: tp bf16
    [nc, Mo] tensors in increasing chunk index (the own entry is drawn too and ignored), from a
    generator of their own so that make_rs's draws stay as they are."""
    g = torch.Generator("cpu").manual_seed(shape.seed + 7919)
    out = []
    for _ in range(shape.tp):
        if shape.dist == "normal_rs":
            out.append((torch.randn((shape.nc, shape.Mo), generator=g) / 16.0).to(torch.bfloat16))
        else:
            out.append(_draw(g, (shape.nc, shape.Mo), shape.dist, shape.Kl).to(torch.bfloat16))
    return out


def ag_shape(tp, self_rank, nc, K, M, dtype="bf16", dist="uniform1", seed=7) -> AGShape:
    return AGShape(f"ag_tp{tp}_s{self_rank}_nc{nc}_k{K}_m{M}_{dtype}_{dist}", tp, self_rank, nc, K,
                   M, dtype, dist, seed)


def rs_shape(tp, self_rank, T, Kl, Mo, dist="normal_rs", seed=11) -> RSShape:
    return RSShape(f"rs_tp{tp}_s{self_rank}_t{T}_k{Kl}_m{Mo}_{dist}", tp, self_rank, T, Kl, Mo,
                   dist, seed)


def bits_u16(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (CPU)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")


def bits_u8(t: torch.Tensor):
    """float8_e4m3fn tensor -> numpy uint8 codes (CPU)."""
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()
