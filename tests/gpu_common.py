"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and the CPU oracle
on the same seeded inputs, and compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import ringag_oracle as O
from ring_all_gather_amd import binding as B
from ring_all_gather_amd import workloads as W

DEV = "cuda:0"
TOL_BF16 = 2e-2     # max|D - ref| <= TOL * max|ref| for bf16 inputs
TOL_FP8 = 5e-2      # ... for fp8 inputs, ref on the dequantised values
TOL_SEND = 1e-3     # fp32 outgoing RS chunks
_ctx = None


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def ctx() -> B.Context:
    global _ctx
    if _ctx is None:
        _ctx = B.Context(0, max_tp=16)
    return _ctx


def reset_options(c: B.Context):
    c.set_option(B.RAG_OPT_COPY_ENGINE, 0)
    c.set_option(B.RAG_OPT_COMM_WGS, 32)
    c.set_option(B.RAG_OPT_SPIN_LIMIT_US, 2_000_000)
    c.set_option(B.RAG_OPT_ARRIVAL_DELAY_US, 0)
    c.set_option(B.RAG_OPT_WITHHOLD_MASK, 0)
    c.set_option(B.RAG_OPT_TILE, 0)
    c.set_option(B.RAG_OPT_COMM_CUS, 0)
    c.set_option(B.RAG_OPT_SDMA_STREAMS, 1)
    c.set_option(B.RAG_OPT_AG_GATE, B.RAG_GATE_CHUNK)
    c.set_option(B.RAG_OPT_SLAB_HELP_US, 20)


def scale_tensor(s):
    return torch.tensor([s], dtype=torch.float32, device=DEV)


def bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return W.bits_u16(t)
    if t.dtype == torch.float8_e4m3fn:
        return W.bits_u8(t)
    raise TypeError(t.dtype)


class AGRun:
    """Device copies of one AG+GEMM input set plus output buffers.  own_in_g: the own chunk lives
    in its slot of G (as the local shard does in a ring all-gather's output buffer, and as the
    benchmark places it), so the call copies only the peers' chunks."""

    def __init__(self, inp: W.AGInputs, with_G: bool = True, own_in_g: bool = False):
        self.inp = inp
        s = inp.shape
        self.A = inp.A.to(DEV)
        self.chunks = [c.to(DEV) for c in inp.chunks]
        self.D = torch.empty((s.N, s.M), dtype=torch.bfloat16, device=DEV)
        self.G = torch.empty((s.N, s.K), dtype=inp.A.dtype, device=DEV) if with_G else None
        if own_in_g:
            assert with_G
            r0 = s.self_rank * s.nc
            self.G[r0:r0 + s.nc].copy_(self.chunks[s.self_rank])
            self.chunks[s.self_rank] = self.G[r0:r0 + s.nc]
        self.sA = scale_tensor(inp.scale_A) if s.dtype == "fp8" else None
        self.sB = scale_tensor(inp.scale_B) if s.dtype == "fp8" else None

    def run(self, c: B.Context, flags: int = 0, self_rank=None, tp=None):
        s = self.inp.shape
        B.ag_gemm(c, self.A, self.chunks, s.tp if tp is None else tp,
                  s.self_rank if self_rank is None else self_rank, self.D, G=self.G,
                  scale_A=self.sA, scale_B=self.sB, flags=flags)
        torch.cuda.synchronize()
        return self

    def D_bits(self) -> np.ndarray:
        return W.bits_u16(self.D.cpu())


def oracle_ag(inp: W.AGInputs):
    """(G bit patterns / codes, fp32 reference D)."""
    if inp.shape.dtype == "fp8":
        return O.ag_gemm_fp8(bits(inp.A), inp.scale_A, [bits(c) for c in inp.chunks], inp.scale_B)
    return O.ag_gemm(bits(inp.A), [bits(c) for c in inp.chunks])


_full_cache = {}


def cached(key, fn):
    """fn() computed once per test session under `key` (the full oracle of a full-size workload
    takes seconds on the host; several GPU variants are compared with the same result)."""
    if key not in _full_cache:
        _full_cache[key] = fn()
    return _full_cache[key]


def oracle_ag_rows(inp: W.AGInputs, rows):
    if inp.shape.dtype == "fp8":
        return O.ag_gemm_fp8_rows(bits(inp.A), inp.scale_A, [bits(c) for c in inp.chunks],
                                  inp.scale_B, rows)
    return O.ag_gemm_rows(bits(inp.A), [bits(c) for c in inp.chunks], rows)


def rel_err(got_bits: np.ndarray, ref: np.ndarray) -> float:
    got = O.bf16_to_f32(got_bits).astype(np.float64)
    ref = ref.astype(np.float64)
    scale = np.abs(ref).max()
    if not np.isfinite(got).all():
        return float("inf")
    return float(np.abs(got - ref).max() / (scale if scale > 0 else 1.0))


def sampled_rows(tp: int, nc: int, seed: int, per_chunk: int = 62):
    """First, last and `per_chunk` seeded-random rows of every chunk (indices into N)."""
    g = np.random.default_rng(seed)
    rows = []
    for r in range(tp):
        mid = g.choice(np.arange(1, nc - 1), size=min(per_chunk, max(nc - 2, 0)), replace=False) \
            if nc > 2 else np.array([], dtype=np.int64)
        rows.extend([r * nc, r * nc + nc - 1, *(r * nc + mid)])
    return np.unique(np.asarray(rows, dtype=np.int64))
