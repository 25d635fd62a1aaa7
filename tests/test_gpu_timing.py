"""GPU kernel timing of the C ABI (RAG_OPT_TIMING, rag_kernel_times): one duration per GEMM call,
each positive and inside the wall-clock interval of the calls, for the one-launch calls (whose
launch records its own events) and for the split form (events around its launches)."""
import time

import pytest
import torch

from ring_all_gather_amd import binding as B
from ring_all_gather_amd import workloads as W

from gpu_common import DEV, ctx, reset_options, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _fresh_options():
    reset_options(ctx())
    yield
    ctx().set_option(B.RAG_OPT_TIMING, 0)
    ctx().kernel_times()
    reset_options(ctx())


def _timed(c, fn, n):
    torch.cuda.synchronize()
    c.kernel_times()
    c.set_option(B.RAG_OPT_TIMING, 1)
    t0 = time.perf_counter()
    for _ in range(n):
        fn()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    c.set_option(B.RAG_OPT_TIMING, 0)
    kt = c.kernel_times()
    return kt, wall_ms


@pytest.mark.parametrize("flags", [0, B.RAG_NO_COPY, B.RAG_PER_CHUNK])
def test_ag_kernel_times(flags):
    c = ctx()
    shape = W.ag_shape(4, 1, 512, 1024, 1024, seed=5)
    say(f"case ag timing flags={flags}")
    inp = W.make_ag(shape)
    A = inp.A.to(DEV)
    ch = [x.to(DEV) for x in inp.chunks]
    D = torch.empty((shape.N, shape.M), dtype=torch.bfloat16, device=DEV)
    kt, wall = _timed(c, lambda: B.ag_gemm(c, A, ch, shape.tp, shape.self_rank, D, flags=flags),
                      5)
    c.check()
    assert len(kt) == 5
    assert all(0.0 < t <= wall for t in kt), (kt, wall)
    assert sum(kt) <= wall


def test_rs_kernel_times():
    c = ctx()
    shape = W.rs_shape(4, 2, 4 * 256, 256, 512, seed=9)
    say("case rs timing")
    inp = W.make_rs(shape)
    X, Wt = inp.X.to(DEV), inp.W.to(DEV)
    parts = [None if p is None else p.to(DEV) for p in inp.partials]
    D = torch.empty((shape.nc, shape.Mo), dtype=torch.bfloat16, device=DEV)
    kt, wall = _timed(c, lambda: B.gemm_rs(c, X, Wt, parts, shape.tp, shape.self_rank, D), 4)
    assert len(kt) == 4
    assert all(0.0 < t <= wall for t in kt), (kt, wall)


def test_timing_off_records_nothing():
    c = ctx()
    shape = W.ag_shape(2, 0, 256, 256, 256, seed=6)
    inp = W.make_ag(shape)
    A = inp.A.to(DEV)
    ch = [x.to(DEV) for x in inp.chunks]
    D = torch.empty((shape.N, shape.M), dtype=torch.bfloat16, device=DEV)
    c.kernel_times()
    B.ag_gemm(c, A, ch, shape.tp, shape.self_rank, D)
    torch.cuda.synchronize()
    assert c.kernel_times() == []
