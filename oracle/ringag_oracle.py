"""CPU oracle for the ring-decomposed all-gather + GEMM (AG+GEMM) and GEMM + reduce-scatter (GEMM+RS).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It shares no code with the HIP library and never imports it; the two meet only
on the seeded inputs that the tests generate.

Each function below cites the passage it follows.  Pages (by title):
  [TE-1583]  TransformerEngine issue #1583, "curious about atomic_gemm_overlap_ag" — the question
             and the C++ listing of CommOverlapP2PBase::atomic_gemm_overlap_ag.
  [NVF-3392] nvFuser PR #3392, "Ring-based decomposition for Allgather+GEMM overlap ATen
             implementation" — description and the nsys experiment.
  [TE-2443]  TransformerEngine PR #2443, "Comm+GEMM overlap API updated to support cuBlasMp
             backend" — summary, sequence diagram, review comments.
  [NVF-5742] nvFuser PR #5742, "Reference implementation for Linear+Allreduce with overlapping" —
             trace, walkthrough, sequence diagram, discussion.

Conventions (all row-major, K-contiguous):
  A  weight shard [M, K]          B_r  chunk of rank r [nc, K]        G  gathered [tp*nc, K]
  D = G A^T  [tp*nc, M]           X  activation shard [T, Kl]         W  weight shard [Mo, Kl]
bf16 tensors travel as numpy uint16 bit patterns, e4m3 tensors as uint8 codes, fp32 as float32.
Products and sums are fp32 with k ascending and no fused multiply-add (the workloads fix fp32
accumulation); the C library under this directory does the loops.

Pins: every function here is checked by the CPU tests against exact integer products, float64
brute force within the fp32 error bound, hand-worked fixtures and library conversions; the
sampled-row forms (ag_gemm_rows, ag_gemm_fp8_rows, gemm_rs_rows, gemm_rs_ring_step_rows) are also
checked against exact integer products at rows that span every chunk and bit for bit against rows
of their full forms, and planted row-index mistakes are shown to fail those pins.  No function is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Sequence, Tuple

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        lib = ctypes.CDLL(path)
        f32p = ctypes.POINTER(ctypes.c_float)
        lib.oracle_gemm_tn_f32.argtypes = [f32p, ctypes.c_long, f32p, ctypes.c_long, f32p,
                                           ctypes.c_long, ctypes.c_long, ctypes.c_long,
                                           ctypes.c_long]
        lib.oracle_gemm_tn_rows_f32.argtypes = [f32p, ctypes.c_long, f32p, ctypes.c_long,
                                                ctypes.POINTER(ctypes.c_long), ctypes.c_long,
                                                f32p, ctypes.c_long, ctypes.c_long, ctypes.c_long]
        lib.oracle_bf16_to_f32.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long]
        lib.oracle_f32_to_bf16_rne.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long]
        lib.oracle_e4m3fn_to_f32.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long]
        lib.oracle_f32_to_e4m3fn_sat.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long]
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    """Threads the oracle's loops run on (OpenMP's count for this process)."""
    return int(_load().oracle_num_threads())


def _f32p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


# ----------------------------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------------------------

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 (bf16 is the top half of an fp32 word)."""
    src = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(src.shape, dtype=np.float32)
    _load().oracle_bf16_to_f32(src.ctypes.data, out.ctypes.data, src.size)
    return out


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (the output rounding of D: the pages do not
    state it; nearest-even is IEEE's default rounding)."""
    src = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(src.shape, dtype=np.uint16)
    _load().oracle_f32_to_bf16_rne(src.ctypes.data, out.ctypes.data, src.size)
    return out


def e4m3fn_to_f32(codes: np.ndarray) -> np.ndarray:
    """Decode OCP FP8 E4M3 (no-infinity variant) codes to fp32 (exact).  The fp8 workload names
    "fp8 e4m3"; the [TE-1583] listing carries the dequantisation factor (scale_inv) with the
    input tensor, so inputs are the codes plus one fp32 scale per tensor."""
    src = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(src.shape, dtype=np.float32)
    _load().oracle_e4m3fn_to_f32(src.ctypes.data, out.ctypes.data, src.size)
    return out


def f32_to_e4m3fn_sat(x: np.ndarray) -> np.ndarray:
    """fp32 -> OCP E4M3 (no-infinity variant) codes, saturating to +-448 and rounding to nearest
    with ties to even: the fp8 output of the GEMM ([TE-1583] listing: the output tensor carries its
    own scale and amax, so D can be fp8).  Written from the format's definition in oracle.c."""
    src = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(src.shape, dtype=np.uint8)
    _load().oracle_f32_to_e4m3fn_sat(src.ctypes.data, out.ctypes.data, src.size)
    return out


def dequantize_e4m3(codes: np.ndarray, scale: float) -> np.ndarray:
    """Dequantised fp32 values float(q) * scale: the operand values the GEMM multiplies, with the
    per-tensor scale of [TE-1583]'s input tensor applied (one fp32 multiply per element)."""
    return (e4m3fn_to_f32(codes) * np.float32(scale)).astype(np.float32)


# ----------------------------------------------------------------------------------------------
# The ring: who holds what, in which order chunks arrive
# ----------------------------------------------------------------------------------------------

def ring_neighbours(rank: int, tp: int) -> Tuple[int, int]:
    """(next, prev) of a rank.  [TE-1583] listing: each ring step sends to the next rank and
    receives from the previous one; their values are not printed.  Reading taken: next = rank+1,
    prev = rank-1 (mod tp)."""
    return (rank + 1) % tp, (rank - 1) % tp


def ring_exchange(tp: int) -> List[List[int]]:
    """Simulate the tp-1 steps of the ring all-gather and return, for every rank, the origin ranks
    of the chunks in the order they become available there (own chunk first).

    [TE-1583] listing: in step i a rank forwards the chunk it holds in slot i (its own chunk at
    i = 0, afterwards the one it received in the step before) to the next rank and receives the
    previous rank's chunk into slot i+1.  [NVF-3392] describes the same tp-1 step decomposition.
    """
    held = [[r] for r in range(tp)]          # per rank: origins in arrival order
    for step in range(tp - 1):
        outgoing = [held[r][step] for r in range(tp)]
        for r in range(tp):
            _, prev = ring_neighbours(r, tp)
            held[r].append(outgoing[prev])
    return held


def ring_order(tp: int, self_rank: int) -> List[int]:
    """Arrival order of chunks at self_rank (derived by running the ring, not by formula)."""
    if not (1 <= tp and 0 <= self_rank < tp):
        raise ValueError("need 1 <= tp and 0 <= self_rank < tp")
    return ring_exchange(tp)[self_rank]


# ----------------------------------------------------------------------------------------------
# All-gather + GEMM
# ----------------------------------------------------------------------------------------------

def gather(chunks: Sequence[np.ndarray]) -> np.ndarray:
    """Explicit all-gather result: chunk r copied to rows [r*nc, (r+1)*nc) of one contiguous buffer.
    [TE-1583] listing comment: the AG output is contiguous in every rank after the exchanges, each
    chunk at its rank's offset (n_chunk = n / tp rows per chunk)."""
    tp = len(chunks)
    nc, k = chunks[0].shape
    out = np.empty((tp * nc, k), dtype=chunks[0].dtype)
    for r, c in enumerate(chunks):
        if c.shape != (nc, k):
            raise ValueError("all chunks must have the same shape")
        out[r * nc:(r + 1) * nc] = c
    return out


def gemm_tn(G: np.ndarray, A: np.ndarray) -> np.ndarray:
    """D[n][m] = sum_k G[n][k] * A[m][k], fp32, k ascending.  [TE-1583] listing: TN layout, m taken
    from the weight's rows, n from the gathered buffer's rows."""
    G = np.ascontiguousarray(G, dtype=np.float32)
    A = np.ascontiguousarray(A, dtype=np.float32)
    (n, k), (m, k2) = G.shape, A.shape
    if k != k2:
        raise ValueError("K mismatch")
    out = np.empty((n, m), dtype=np.float32)
    if n and m:
        _load().oracle_gemm_tn_f32(_f32p(G), k, _f32p(A), k, _f32p(out), m, n, m, k)
    return out


def gemm_tn_rows(G: np.ndarray, A: np.ndarray, rows: Sequence[int]) -> np.ndarray:
    """Rows `rows` of gemm_tn(G, A) only (same loop, same order)."""
    G = np.ascontiguousarray(G, dtype=np.float32)
    A = np.ascontiguousarray(A, dtype=np.float32)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if rows.size and (rows.min() < 0 or rows.max() >= G.shape[0]):
        raise IndexError("row out of range")
    m, k = A.shape
    out = np.empty((rows.size, m), dtype=np.float32)
    if rows.size and m:
        _load().oracle_gemm_tn_rows_f32(_f32p(G), G.shape[1], _f32p(A), k,
                                        rows.ctypes.data_as(ctypes.POINTER(ctypes.c_long)),
                                        rows.size, _f32p(out), m, m, k)
    return out


def ag_gemm(A_bits: np.ndarray, chunk_bits: Sequence[np.ndarray]) -> Tuple[np.ndarray, np.ndarray]:
    """bf16 AG+GEMM: returns (G bit patterns, D in fp32 before output rounding).
    G = explicit rank-ordered concatenation of the chunks; D = G A^T (fp32 accumulate)."""
    G = gather(chunk_bits)
    return G, gemm_tn(bf16_to_f32(G), bf16_to_f32(A_bits))


def ag_gemm_rows(A_bits: np.ndarray, chunk_bits: Sequence[np.ndarray], rows) -> np.ndarray:
    """Rows `rows` (indices into the gathered N) of the bf16 AG+GEMM result, fp32."""
    G = gather(chunk_bits)
    return gemm_tn_rows(bf16_to_f32(G), bf16_to_f32(A_bits), rows)


def ag_gemm_fp8(A_q: np.ndarray, scale_A: float, chunk_q: Sequence[np.ndarray],
                scale_B: float) -> Tuple[np.ndarray, np.ndarray]:
    """fp8 (E4M3) AG+GEMM on dequantised values: (G codes, D fp32).  Each operand is dequantised
    with its per-tensor scale, then the same fp32 GEMM runs."""
    G = gather(chunk_q)
    return G, gemm_tn(dequantize_e4m3(G, scale_B), dequantize_e4m3(A_q, scale_A))


def ag_gemm_fp8_rows(A_q, scale_A, chunk_q, scale_B, rows) -> np.ndarray:
    """Rows `rows` (indices into the gathered N) of the fp8 AG+GEMM result on dequantised values,
    fp32 (same loop and order as ag_gemm_fp8)."""
    G = gather(chunk_q)
    return gemm_tn_rows(dequantize_e4m3(G, scale_B), dequantize_e4m3(A_q, scale_A), rows)


def ag_gemm_ring(A: np.ndarray, chunks: Sequence[np.ndarray], self_rank: int) -> np.ndarray:
    """The ring-decomposed computation at one rank, on fp32 operands: chunks are taken in their
    arrival order and each chunk's product is written at that chunk's rank offset.
    [TE-1583] listing (GEMM split into tp pieces along n, consuming chunk after chunk as the ring
    delivers it) and [NVF-3392] (ring-based decomposition of AG+GEMM)."""
    tp = len(chunks)
    nc = chunks[0].shape[0]
    out = np.full((tp * nc, A.shape[0]), np.nan, dtype=np.float32)
    for r in ring_order(tp, self_rank):
        out[r * nc:(r + 1) * nc] = gemm_tn(chunks[r], A)
    return out


def staged_output_rotation(slot_outputs: Sequence[np.ndarray]) -> np.ndarray:
    """The output placement printed in the [TE-1583] listing, taken literally: the GEMM writes its
    tp output chunks into a buffer of tp+1 chunks (slot j = the j-th chunk the GEMM consumed), then
    slot 0 is copied to slot tp and D is slots 1..tp."""
    tp = len(slot_outputs)
    nc, m = slot_outputs[0].shape
    buf = np.empty(((tp + 1) * nc, m), dtype=slot_outputs[0].dtype)
    for j, o in enumerate(slot_outputs):
        buf[j * nc:(j + 1) * nc] = o
    buf[tp * nc:(tp + 1) * nc] = buf[0:nc]
    return buf[nc:(tp + 1) * nc].copy()


def staged_output_by_rank(slot_outputs: Sequence[np.ndarray], order: Sequence[int]) -> np.ndarray:
    """The staged placement as this library realises it: slot j (j-th chunk consumed, origin rank
    order[j]) is copied to D rows [order[j]*nc, ...).  D is then rank-ordered for every self rank,
    which is what the listing's comment promises (contiguous AG output in all ranks)."""
    tp = len(slot_outputs)
    nc, m = slot_outputs[0].shape
    out = np.empty((tp * nc, m), dtype=slot_outputs[0].dtype)
    for j, r in enumerate(order):
        out[r * nc:(r + 1) * nc] = slot_outputs[j]
    return out


# ----------------------------------------------------------------------------------------------
# GEMM + reduce-scatter (row-parallel linear)
# ----------------------------------------------------------------------------------------------

def local_partial(X_bits: np.ndarray, W_bits: np.ndarray) -> np.ndarray:
    """This rank's partial product P = X W^T over all T rows (fp32).  In a row-parallel linear the
    contraction dimension is sharded ([TE-2443] review: global k = local k * tp), so every rank
    holds a partial sum of the whole [T, Mo] output ([NVF-5742] walkthrough)."""
    return gemm_tn(bf16_to_f32(X_bits), bf16_to_f32(W_bits))


def reduce_chunk(partials: Sequence[np.ndarray], chunk: int, nc: int) -> np.ndarray:
    """Reduce-scatter result for one output chunk: sum over ranks p = 0..tp-1 (ascending) of rows
    [chunk*nc, (chunk+1)*nc) of partial p, fp32 adds.  [TE-2443] sequence diagram (GEMM then
    reduce-scatter) and [NVF-5742] (the all-reduce sums each chunk over ranks)."""
    acc = np.zeros((nc, partials[0].shape[1]), dtype=np.float32)
    for p in range(len(partials)):
        acc = (acc + partials[p][chunk * nc:(chunk + 1) * nc]).astype(np.float32)
    return acc


def gemm_rs(X_bits: np.ndarray, W_bits: np.ndarray, peer_partials: Sequence[np.ndarray],
            tp: int, self_rank: int):
    """One rank's GEMM+RS.  peer_partials[p] is rank p's fp32 [T, Mo] partial (entry self_rank is
    ignored and may be None).  Returns (D fp32 [nc, Mo] before output rounding,
    send [tp, nc, Mo] fp32 with send[c] = rows of chunk c of this rank's partial (slot self_rank is
    not part of the result), the local partial P [T, Mo])."""
    T = X_bits.shape[0]
    if T % tp:
        raise ValueError("T must be a multiple of tp")
    nc = T // tp
    P = local_partial(X_bits, W_bits)
    full = [P if p == self_rank else np.asarray(peer_partials[p], dtype=np.float32)
            for p in range(tp)]
    D = reduce_chunk(full, self_rank, nc)
    send = np.stack([P[c * nc:(c + 1) * nc] for c in range(tp)])
    return D, send, P


def gemm_rs_rows(X_bits, W_bits, peer_partials, tp, self_rank, local_rows):
    """Rows `local_rows` (indices within this rank's output chunk) of gemm_rs's D, fp32."""
    T = X_bits.shape[0]
    nc = T // tp
    rows = np.asarray(local_rows, dtype=np.int64)
    P_rows = gemm_tn_rows(bf16_to_f32(X_bits), bf16_to_f32(W_bits), self_rank * nc + rows)
    acc = np.zeros_like(P_rows)
    for p in range(tp):
        part = P_rows if p == self_rank else \
            np.asarray(peer_partials[p], dtype=np.float32)[self_rank * nc + rows]
        acc = (acc + part).astype(np.float32)
    return acc


def rs_ring_order(self_rank: int, tp: int) -> List[int]:
    """Chunks in the order one rank works on them in a ring reduce-scatter whose running sums go
    to rank s+1 (the same direction as the all-gather ring: send to next, receive from prev).
    Chunk c's sum starts at rank c+1 and travels c+1 -> c+2 -> ... -> c, so rank s holds it at
    step k = (s - c - 1) mod tp: at step k it works on c_k = (s - 1 - k) mod tp, its own chunk
    last.  [TE-2443] sequence diagram (split GEMM, then reduce-scatter);
    [TE-1583] listing (ring neighbours)."""
    return [(self_rank - 1 - k) % tp for k in range(tp)]


def gemm_rs_ring_step(X_bits: np.ndarray, W_bits: np.ndarray,
                      incoming: Sequence[np.ndarray], tp: int, self_rank: int):
    """One rank's share of a ring-accumulate reduce-scatter.  P = X W^T over all T rows; for
    every chunk c, out[c] = incoming[c] + P[rows of c] (one fp32 add), where incoming[c] is the
    running sum of chunk c that arrives from rank s-1, and incoming[(s-1) mod tp] is None (that
    chain starts here: out = P's rows).  The own chunk's out[s] is the reduced result.
    Returns (D fp32 [nc, Mo] = out[s], send [tp, nc, Mo] with send[c] = out[c] for c != s, P).
    [TE-2443] sequence diagram (reduce-scatter of the split GEMM's output); [NVF-5742]
    walkthrough (each output chunk is a sum over ranks)."""
    T = X_bits.shape[0]
    if T % tp:
        raise ValueError("T must be a multiple of tp")
    nc = T // tp
    P = local_partial(X_bits, W_bits)
    start = (self_rank - 1) % tp
    out = []
    for c in range(tp):
        mine = P[c * nc:(c + 1) * nc]
        if c == start:
            out.append(mine.copy())
        else:
            out.append((np.asarray(incoming[c], dtype=np.float32) + mine).astype(np.float32))
    return out[self_rank], np.stack(out), P


def gemm_rs_ring_step_rows(X_bits, W_bits, incoming, tp, self_rank, chunk, local_rows):
    """Rows `local_rows` of out[chunk] of gemm_rs_ring_step, fp32 (sampled checks)."""
    T = X_bits.shape[0]
    nc = T // tp
    rows = np.asarray(local_rows, dtype=np.int64)
    mine = gemm_tn_rows(bf16_to_f32(X_bits), bf16_to_f32(W_bits), chunk * nc + rows)
    if chunk == (self_rank - 1) % tp:
        return mine
    return (np.asarray(incoming[chunk], dtype=np.float32)[rows] + mine).astype(np.float32)


def linear_allreduce_step(X_bits: np.ndarray, W_bits: np.ndarray,
                          peer_partials: Sequence[np.ndarray], reduced_bits: Sequence[np.ndarray],
                          tp: int, self_rank: int):
    """One rank's share of a row-parallel linear whose output is all-reduced as a reduce-scatter
    followed by an all-gather of the reduced chunks.  The reduce-scatter is gemm_rs (this rank
    reduces its own chunk over all ranks' partials); the all-gather brings in every other chunk
    c as its owner reduced it (reduced_bits[c], bf16 [nc, Mo]; entry self_rank ignored).
    Returns (Y fp32 [T, Mo]: rows of chunk c = reduced chunk c widened, rows of the own chunk =
    the fp32 sum before output rounding; send as gemm_rs).
    [NVF-5742] walkthrough and sequence diagram (row-parallel linear: per-chunk matmul, then the
    chunk's all-reduce); [TE-2443] sequence diagram (reduce-scatter of the split GEMM)."""
    T = X_bits.shape[0]
    nc = T // tp
    D, send, _ = gemm_rs(X_bits, W_bits, peer_partials, tp, self_rank)
    Mo = D.shape[1]
    Y = np.empty((T, Mo), dtype=np.float32)
    for c in range(tp):
        Y[c * nc:(c + 1) * nc] = D if c == self_rank else bf16_to_f32(reduced_bits[c])
    return Y, send


def quantize_output_e4m3(D: np.ndarray, scale_D: float) -> Tuple[np.ndarray, float]:
    """fp8 output epilogue: codes = E4M3(D * scale_D) with one fp32 multiply per element, and
    amax = max |D| over the output before the scale.  [TE-1583] listing: the GEMM's output
    buffer is built with D's amax and scale, so the GEMM quantises its own output and records the
    absolute maximum for the next scaling."""
    D = np.asarray(D, dtype=np.float32)
    codes = f32_to_e4m3fn_sat((D * np.float32(scale_D)).astype(np.float32))
    amax = float(np.max(np.abs(D))) if D.size else 0.0
    return codes, amax
