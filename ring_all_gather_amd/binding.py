"""Thin ctypes binding of libringag.so (include/ringag.h).

Argument marshalling only: tensors are turned into device pointers and sizes, the caller's current
torch stream is passed as the stream, and a non-zero return becomes a RuntimeError carrying
rag_last_error().  Every step of the operations runs in the library's HIP kernels; there is no
other code path.  If the library has not been built, the first call raises.

Environment overrides applied when a Context is created (all optional):
  RAG_COPY_ENGINE=kernel|sdma   RAG_COMM_WGS=n   RAG_SPIN_LIMIT_US=n   RAG_TILE=auto|128x128|256x128|256x256
"""
from __future__ import annotations

import atexit
import ctypes
import os
import re
import sys
import weakref
from typing import Optional, Sequence

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libringag.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "ringag.h")

# constants of include/ringag.h
RAG_OK, RAG_EINVAL, RAG_EHIP, RAG_ETIMEOUT, RAG_ENOMEM = 0, -1, -2, -3, -4
RAG_BF16, RAG_FP8_E4M3 = 0, 1
RAG_STAGED_OUT, RAG_NO_COPY, RAG_COPY_ONLY, RAG_PER_CHUNK, RAG_RS_ARRIVE = 1, 2, 4, 8, 16
RAG_OPT_COPY_ENGINE, RAG_OPT_COMM_WGS, RAG_OPT_SPIN_LIMIT_US = 1, 2, 3
RAG_OPT_ARRIVAL_DELAY_US, RAG_OPT_WITHHOLD_MASK, RAG_OPT_TIMING, RAG_OPT_TILE = 4, 5, 6, 7
RAG_OPT_TRACE_BUF, RAG_OPT_TRACE_BYTES, RAG_OPT_WGS_PER_CU, RAG_OPT_COPY_PRIORITY = 8, 9, 10, 11
RAG_OPT_GEMM_COPY_WGS, RAG_OPT_COMM_CUS, RAG_OPT_SDMA_STREAMS, RAG_OPT_AG_GATE = 12, 13, 14, 15
RAG_OPT_SLAB_HELP_US = 16
RAG_GATE_CHUNK, RAG_GATE_SLAB = 0, 1
RAG_COPY_KERNEL, RAG_COPY_SDMA, RAG_COPY_IN_GEMM, RAG_COPY_IN_GEMM_ASSIST = 0, 1, 2, 3
RAG_COPY_IN_GEMM_SDMA = 4
ENGINES = {"kernel": RAG_COPY_KERNEL, "sdma": RAG_COPY_SDMA, "in-gemm": RAG_COPY_IN_GEMM,
           "assist": RAG_COPY_IN_GEMM_ASSIST, "in-gemm-sdma": RAG_COPY_IN_GEMM_SDMA}
TRACE_HEADER, TRACE_START, TRACE_TILE_WORDS = 64, 32, 5
TILES = {"auto": 0, "128x128": 1, "256x128": 2, "256x256": 3, "256x256w8": 4, "256x256w8s4": 5,
         "256x192w8": 6}
RAG_MAX_TP = 16

_lib = None
_live = weakref.WeakSet()     # open contexts, closed at exit before the runtime shuts down


@atexit.register
def _close_all():
    for c in list(_live):
        try:
            c.close()
        except Exception:
            pass


class RagError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"ringag error {code}: {msg}")
        self.code = code


def lib():
    """Load libringag.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -m "
                           "ring_all_gather_amd.build or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, ll = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong
    L.rag_create.argtypes = [ctypes.POINTER(vp), i, i, i]
    L.rag_destroy.argtypes = [vp]
    L.rag_set_option.argtypes = [vp, i, ll]
    L.ag_gemm.argtypes = [vp, vp, i, i, ctypes.POINTER(vp), i, i, i, vp, vp, i, vp, vp, i, vp]
    L.gemm_rs.argtypes = [vp, vp, i, i, vp, i, ctypes.POINTER(vp), ll, i, i, vp, vp, i, vp]
    L.ag_gemm_noalloc.argtypes = [vp, vp, i, i, ctypes.POINTER(vp), i, i, i, vp, vp, i, vp, vp,
                                  i, vp]
    L.ag_gemm_ex.argtypes = [vp, vp, i, i, ctypes.POINTER(vp), i, i, i, vp, vp, i, vp, vp, i,
                             vp, vp, vp, i, vp]
    L.gemm_rs_ring.argtypes = [vp, vp, i, i, vp, i, ctypes.POINTER(vp), ll, i, i, vp, vp, i, vp]
    L.linear_allreduce.argtypes = [vp, vp, i, i, vp, i, ctypes.POINTER(vp), ll,
                                   ctypes.POINTER(vp), i, i, vp, vp, i, vp]
    L.rag_check.argtypes = [vp]
    L.rag_kernel_times.argtypes = [vp, ctypes.POINTER(ctypes.c_float), i]
    L.rag_ag_kernel_name.argtypes = [vp, i, i, i, i, ctypes.c_char_p, i]
    L.rag_rs_kernel_name.argtypes = [vp, i, i, i, ctypes.c_char_p, i]
    L.rag_last_error.restype = ctypes.c_char_p
    L.rag_version.restype = i
    for f in ("rag_create", "rag_destroy", "rag_set_option", "ag_gemm", "ag_gemm_ex", "gemm_rs",
              "gemm_rs_ring", "ag_gemm_noalloc",
              "linear_allreduce",
              "rag_check",
              "rag_kernel_times", "rag_ag_kernel_name", "rag_rs_kernel_name"):
        getattr(L, f).restype = i
    _lib = L
    return L


def declared_functions():
    """Names of the functions include/ringag.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*RAG_API\s+(?:const\s+)?\w+\s*\**\s*(\w+)\s*\(", text,
                                 flags=re.M)))


def kernels_fingerprint() -> str:
    """SHA-256 of the gfx950 code object embedded in the loaded library."""
    return (ctypes.c_char * 65).in_dll(lib(), "ringag_kernels_sha256").value.decode()


def last_error() -> str:
    return lib().rag_last_error().decode()


def _check(rc: int):
    if rc != RAG_OK:
        raise RagError(rc, last_error())
    return rc


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to libringag must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libringag must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class Context:
    """Owns a rag_ctx (side stream, events, counters, epoch, cached buffers)."""

    def __init__(self, device: int = 0, max_tp: int = 8):
        h = ctypes.c_void_p()
        _check(lib().rag_create(ctypes.byref(h), device, max_tp, 0))
        self.h = h
        self.device = device
        self.max_tp = max_tp
        _live.add(self)
        env = os.environ
        if "RAG_COPY_ENGINE" in env:
            self.set_option(RAG_OPT_COPY_ENGINE, ENGINES[env["RAG_COPY_ENGINE"]])
        if "RAG_COMM_WGS" in env:
            self.set_option(RAG_OPT_COMM_WGS, int(env["RAG_COMM_WGS"]))
        if "RAG_SPIN_LIMIT_US" in env:
            self.set_option(RAG_OPT_SPIN_LIMIT_US, int(env["RAG_SPIN_LIMIT_US"]))
        if "RAG_TILE" in env:
            self.set_option(RAG_OPT_TILE, TILES[env["RAG_TILE"]])

    def set_option(self, key: int, value: int):
        _check(lib().rag_set_option(self.h, key, int(value)))

    def set_trace(self, buf: Optional[torch.Tensor]):
        """Diagnostics: record wall-clock stamps of the next ag_gemm calls into `buf` (an int64 GPU
        tensor; layout in ringag.h under RAG_OPT_TRACE_BUF), or stop with None."""
        if buf is None:
            self.set_option(RAG_OPT_TRACE_BUF, 0)
            self.set_option(RAG_OPT_TRACE_BYTES, 0)
            return
        if buf.dtype != torch.int64 or not buf.is_cuda or not buf.is_contiguous():
            raise ValueError("trace buffer must be a contiguous int64 GPU tensor")
        self.set_option(RAG_OPT_TRACE_BYTES, buf.numel() * 8)
        self.set_option(RAG_OPT_TRACE_BUF, buf.data_ptr())

    def ag_kernel_name(self, nc: int, M: int, tp: int, fp8: bool = False) -> str:
        """Entry point ag_gemm would launch for these sizes (diagnostics)."""
        buf = ctypes.create_string_buffer(128)
        _check(lib().rag_ag_kernel_name(self.h, nc, M, tp, RAG_FP8_E4M3 if fp8 else RAG_BF16,
                                        buf, 128))
        return buf.value.decode()

    def rs_kernel_name(self, nc: int, Mo: int, tp: int) -> str:
        """Entry point gemm_rs would launch for these sizes (diagnostics)."""
        buf = ctypes.create_string_buffer(128)
        _check(lib().rag_rs_kernel_name(self.h, nc, Mo, tp, buf, 128))
        return buf.value.decode()

    def check(self):
        """Synchronise and raise RagError(RAG_ETIMEOUT) if a chunk never arrived."""
        _check(lib().rag_check(self.h))

    def kernel_times(self, max_n: int = 4096):
        buf = (ctypes.c_float * max_n)()
        n = lib().rag_kernel_times(self.h, buf, max_n)
        if n < 0:
            _check(n)
        return [buf[i] for i in range(min(n, max_n))]

    def close(self):
        if getattr(self, "h", None):
            lib().rag_destroy(self.h)
            self.h = None

    def __del__(self, _finalizing=sys.is_finalizing):
        # During interpreter shutdown the HIP runtime may already be going away: leave the
        # context to the process exit (atexit above closes it earlier in a normal exit).  The
        # check is bound as a default argument: module globals may already be gone by then.
        try:
            if _finalizing() or not getattr(self, "h", None):
                return
            self.close()
        except Exception:
            pass


def ag_gemm(ctx: Context, A: torch.Tensor, B_chunks: Sequence[torch.Tensor], tp: int,
            self_rank: int, D: torch.Tensor, G: Optional[torch.Tensor] = None,
            scale_A: Optional[torch.Tensor] = None, scale_B: Optional[torch.Tensor] = None,
            flags: int = 0, stream=None, scale_D: Optional[torch.Tensor] = None,
            amax_D: Optional[torch.Tensor] = None, B_copy: Optional[torch.Tensor] = None) -> int:
    """D = [B_0; ...; B_{tp-1}] A^T for rank self_rank of a tp-rank ring (see ringag.h).  D is
    bfloat16, or float8_e4m3fn with scale_D (and optionally amax_D); B_copy, if given, receives
    this rank's chunk (these go through ag_gemm_ex)."""
    if len(B_chunks) != tp:
        raise ValueError(f"need tp={tp} chunks, got {len(B_chunks)}")
    fp8 = A.dtype == torch.float8_e4m3fn
    if not fp8 and A.dtype != torch.bfloat16:
        raise ValueError("A must be bfloat16 or float8_e4m3fn")
    M, K = A.shape
    nc = B_chunks[0].shape[0]
    for b in B_chunks:
        if b.dtype != A.dtype or tuple(b.shape) != (nc, K):
            raise ValueError("every chunk must be [nc, K] with A's dtype")
    out8 = D.dtype == torch.float8_e4m3fn
    if (D.dtype != torch.bfloat16 and not out8) or tuple(D.shape) != (tp * nc, M):
        raise ValueError(f"D must be bfloat16 or float8_e4m3fn [{tp * nc}, {M}]")
    if G is not None and (G.dtype != A.dtype or tuple(G.shape) != (tp * nc, K)):
        raise ValueError(f"G must be [{tp * nc}, {K}] with A's dtype")
    if B_copy is not None and (B_copy.dtype != A.dtype or tuple(B_copy.shape) != (nc, K)):
        raise ValueError(f"B_copy must be [{nc}, {K}] with A's dtype")
    ptrs = (ctypes.c_void_p * tp)(*[_ptr(b) for b in B_chunks])
    dt = RAG_FP8_E4M3 if fp8 else RAG_BF16
    if not out8 and scale_D is None and amax_D is None and B_copy is None:
        return _check(lib().ag_gemm(ctx.h, _ptr(A), M, K, ptrs, nc, tp, self_rank, _ptr(G),
                                    _ptr(D), dt, _ptr(scale_A), _ptr(scale_B), flags,
                                    _stream(stream)))
    return _check(lib().ag_gemm_ex(ctx.h, _ptr(A), M, K, ptrs, nc, tp, self_rank, _ptr(G), _ptr(D),
                                   dt, _ptr(scale_A), _ptr(scale_B),
                                   RAG_FP8_E4M3 if out8 else RAG_BF16, _ptr(scale_D),
                                   _ptr(amax_D), _ptr(B_copy), flags, _stream(stream)))


def ag_gemm_noalloc(ctx: Context, A: torch.Tensor, B_chunks: Sequence[torch.Tensor], tp: int,
                    self_rank: int, D: torch.Tensor, G: torch.Tensor,
                    scale_A: Optional[torch.Tensor] = None,
                    scale_B: Optional[torch.Tensor] = None, flags: int = 0, stream=None) -> int:
    """ag_gemm with the call's device words in the library's fixed scratch array (ringag.h):
    G is required; D is bfloat16."""
    if len(B_chunks) != tp:
        raise ValueError(f"need tp={tp} chunks, got {len(B_chunks)}")
    fp8 = A.dtype == torch.float8_e4m3fn
    M, K = A.shape
    nc = B_chunks[0].shape[0]
    ptrs = (ctypes.c_void_p * tp)(*[_ptr(b) for b in B_chunks])
    return _check(lib().ag_gemm_noalloc(ctx.h, _ptr(A), M, K, ptrs, nc, tp, self_rank, _ptr(G),
                                        _ptr(D), RAG_FP8_E4M3 if fp8 else RAG_BF16,
                                        _ptr(scale_A), _ptr(scale_B), flags, _stream(stream)))


def _rs(fn, ctx: Context, X: torch.Tensor, W: torch.Tensor, entries, rows: int, skip: int,
        tp: int, self_rank: int, D: torch.Tensor, send, flags: int, stream) -> int:
    T, Kl = X.shape
    Mo = W.shape[0]
    if X.dtype != torch.bfloat16 or W.dtype != torch.bfloat16 or W.shape[1] != Kl:
        raise ValueError("X [T, Kl] and W [Mo, Kl] must be bfloat16")
    if len(entries) != tp:
        raise ValueError(f"need tp={tp} entries (the ignored one may be None)")
    nc = T // tp
    if D.dtype != torch.bfloat16 or tuple(D.shape) != (nc, Mo):
        raise ValueError(f"D must be bfloat16 [{nc}, {Mo}]")
    if send is not None and (send.dtype != torch.float32 or tuple(send.shape) != (tp, nc, Mo)):
        raise ValueError(f"send must be float32 [{tp}, {nc}, {Mo}]")
    ld = None
    arr = []
    for i, t in enumerate(entries):
        if i == skip or t is None:
            arr.append(None)
            continue
        if t.dtype != torch.float32 or t.dim() != 2 or t.shape[0] != rows or t.shape[1] < Mo \
                or t.stride(1) != 1 or not t.is_cuda:
            raise ValueError(f"each entry must be a float32 GPU tensor [{rows}, >={Mo}], unit "
                             "column stride")
        if ld is not None and t.stride(0) != ld:
            raise ValueError("all entries must share one row stride")
        ld = t.stride(0)
        arr.append(ctypes.c_void_p(t.data_ptr()))
    ptrs = (ctypes.c_void_p * tp)(*arr)
    return _check(fn(ctx.h, _ptr(X), T, Kl, _ptr(W), Mo, ptrs, Mo if ld is None else ld, tp,
                     self_rank, _ptr(send), _ptr(D), flags, _stream(stream)))


def gemm_rs(ctx: Context, X: torch.Tensor, W: torch.Tensor,
            partials: Sequence[Optional[torch.Tensor]], tp: int, self_rank: int,
            D: torch.Tensor, send: Optional[torch.Tensor] = None, flags: int = 0,
            stream=None) -> int:
    """D = sum over ranks of the rows of chunk self_rank of X W^T (peers' [T, Mo] partials given;
    entry self_rank ignored); send[c] = this rank's rows of chunk c."""
    return _rs(lib().gemm_rs, ctx, X, W, partials, X.shape[0], self_rank, tp, self_rank, D, send,
               flags, stream)


def gemm_rs_ring(ctx: Context, X: torch.Tensor, W: torch.Tensor,
                 incoming: Sequence[Optional[torch.Tensor]], tp: int, self_rank: int,
                 D: torch.Tensor, send: Optional[torch.Tensor] = None, flags: int = 0,
                 stream=None) -> int:
    """One ring-accumulate reduce-scatter step: send[c] = incoming[c] + this rank's rows of chunk
    c, D = incoming[self_rank] + its own rows (incoming [nc, Mo] running sums by chunk; the entry
    of the chain that starts here, (self_rank - 1) mod tp, is ignored)."""
    nc = X.shape[0] // tp
    return _rs(lib().gemm_rs_ring, ctx, X, W, incoming, nc, (self_rank - 1) % tp, tp, self_rank,
               D, send, flags, stream)


def linear_allreduce(ctx: Context, X: torch.Tensor, W: torch.Tensor,
                     partials: Sequence[Optional[torch.Tensor]],
                     reduced: Sequence[Optional[torch.Tensor]], tp: int, self_rank: int,
                     Y: torch.Tensor, send: Optional[torch.Tensor] = None, flags: int = 0,
                     stream=None) -> int:
    """Row-parallel linear with its output all-reduced (reduce-scatter + all-gather of the reduced
    chunks): Y's own chunk = the sum over ranks of that chunk's partials, Y's chunk c = reduced[c]
    (the owners' bf16 [nc, Mo] results, entry self_rank ignored)."""
    T, Kl = X.shape
    Mo = W.shape[0]
    if Y.dtype != torch.bfloat16 or tuple(Y.shape) != (T, Mo) or not Y.is_contiguous():
        raise ValueError(f"Y must be a contiguous bfloat16 [{T}, {Mo}] tensor")
    if len(reduced) != tp:
        raise ValueError(f"need tp={tp} reduced entries (entry self_rank may be None)")
    nc = T // tp
    rarr = []
    for r, t in enumerate(reduced):
        if r == self_rank or t is None:
            rarr.append(None)
            continue
        if t.dtype != torch.bfloat16 or tuple(t.shape) != (nc, Mo) or not t.is_contiguous() \
                or not t.is_cuda:
            raise ValueError(f"each reduced chunk must be a contiguous bfloat16 GPU [{nc}, {Mo}]")
        rarr.append(ctypes.c_void_p(t.data_ptr()))
    rptrs = (ctypes.c_void_p * tp)(*rarr)
    arr = []
    ldp = Mo
    for p, t in enumerate(partials):
        if p == self_rank or t is None:
            arr.append(None)
            continue
        if t.dtype != torch.float32 or t.dim() != 2 or t.shape[0] != T or t.stride(1) != 1:
            raise ValueError("each peer partial must be a float32 GPU tensor [T, >=Mo]")
        ldp = t.stride(0)
        arr.append(ctypes.c_void_p(t.data_ptr()))
    ptrs = (ctypes.c_void_p * tp)(*arr)
    return _check(lib().linear_allreduce(ctx.h, _ptr(X), T, Kl, _ptr(W), Mo, ptrs, ldp, rptrs, tp,
                                         self_rank, _ptr(send), _ptr(Y), flags, _stream(stream)))
