"""The per-tile wall-clock trace (RAG_OPT_TRACE_BUF) of ag_gemm: consistent stamps (start <= go <=
end for every tile, no tile of a peer's chunk before that chunk's release), a traced call's
result unchanged, and a buffer too small for the call left untouched."""
import math

import pytest
import torch

from ring_all_gather_amd import binding as B
from ring_all_gather_amd import workloads as W

from gpu_common import DEV, TOL_BF16, ctx, oracle_ag, rel_err, reset_options, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _fresh_options():
    reset_options(ctx())
    yield
    ctx().set_trace(None)
    reset_options(ctx())


@pytest.mark.parametrize("engine", ["kernel", "in-gemm"])
def test_trace_stamps_are_consistent(engine):
    c = ctx()
    c.set_option(B.RAG_OPT_COPY_ENGINE, B.ENGINES[engine])
    c.set_option(B.RAG_OPT_TILE, B.TILES["128x128"])
    shape = W.ag_shape(4, 2, 256, 512, 384, seed=21)
    say(f"case trace engine={engine}")
    inp = W.make_ag(shape)
    A = inp.A.to(DEV)
    ch = [x.to(DEV) for x in inp.chunks]
    D = torch.empty((shape.N, shape.M), dtype=torch.bfloat16, device=DEV)
    per_chunk = math.ceil(shape.nc / 128) * math.ceil(shape.M / 128)
    total = per_chunk * shape.tp
    buf = torch.zeros(64 + 5 * total, dtype=torch.int64, device=DEV)
    c.set_trace(buf)
    B.ag_gemm(c, A, ch, shape.tp, shape.self_rank, D)
    torch.cuda.synchronize()
    c.set_trace(None)
    c.check()
    w = buf.cpu().numpy()
    tiles = w[64:64 + 5 * total].reshape(total, 5)
    assert (tiles[:, 0] > 0).all()
    assert (tiles[:, 0] <= tiles[:, 1]).all() and (tiles[:, 1] <= tiles[:, 2]).all()
    for j in range(1, shape.tp):
        release = w[j - 1]
        assert release > 0
        tj = tiles[j * per_chunk:(j + 1) * per_chunk]
        assert (tj[:, 1] >= release).all(), f"a tile of ring position {j} went before its release"
    _, ref = oracle_ag(inp)
    assert rel_err(W.bits_u16(D.cpu()), ref) <= TOL_BF16


def test_trace_buffer_too_small_records_nothing():
    c = ctx()
    c.set_option(B.RAG_OPT_COPY_ENGINE, B.ENGINES["in-gemm"])
    shape = W.ag_shape(2, 0, 256, 256, 256, seed=22)
    inp = W.make_ag(shape)
    A = inp.A.to(DEV)
    ch = [x.to(DEV) for x in inp.chunks]
    D = torch.empty((shape.N, shape.M), dtype=torch.bfloat16, device=DEV)
    buf = torch.zeros(64, dtype=torch.int64, device=DEV)
    c.set_trace(buf)
    B.ag_gemm(c, A, ch, shape.tp, shape.self_rank, D)
    torch.cuda.synchronize()
    c.set_trace(None)
    assert (buf.cpu().numpy() == 0).all()
