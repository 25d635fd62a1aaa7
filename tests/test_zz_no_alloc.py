"""The allocation-free AG+GEMM entry point (ag_gemm_noalloc, through the C ABI) against ag_gemm:
two calls in a row on the same device, the second with a smaller input, each bit for bit equal to
ag_gemm's output on the same inputs (the two share their kernels; only where the call's counters
and piece counts live differs)."""
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
    reset_options(ctx())


class _Case:
    def __init__(self, shape):
        inp = W.make_ag(shape)
        self.shape = shape
        self.A = inp.A.to(DEV)
        self.chunks = [t.to(DEV) for t in inp.chunks]
        self.G = torch.empty((shape.N, shape.K), dtype=inp.A.dtype, device=DEV)
        self.D = torch.full((shape.N, shape.M), float("nan"), dtype=torch.bfloat16, device=DEV)
        self.G_ref = torch.empty_like(self.G)
        self.D_ref = torch.full_like(self.D, float("nan"))
        self.sA = self.sB = None
        if shape.dtype == "fp8":
            self.sA = torch.tensor([inp.scale_A], dtype=torch.float32, device=DEV)
            self.sB = torch.tensor([inp.scale_B], dtype=torch.float32, device=DEV)

    def reference(self, c):
        s = self.shape
        B.ag_gemm(c, self.A, self.chunks, s.tp, s.self_rank, self.D_ref, G=self.G_ref,
                  scale_A=self.sA, scale_B=self.sB)

    def noalloc(self, c, flags=0):
        s = self.shape
        B.ag_gemm_noalloc(c, self.A, self.chunks, s.tp, s.self_rank, self.D, self.G,
                          scale_A=self.sA, scale_B=self.sB, flags=flags)

    def check(self, what):
        assert torch.equal(self.D.view(torch.int16), self.D_ref.view(torch.int16)), what
        assert torch.equal(self.G.view(torch.uint8), self.G_ref.view(torch.uint8)), what


@pytest.mark.parametrize("engine", ["in-gemm", "kernel", "sdma"])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_noalloc_matches_ag_gemm_two_calls_smaller_second(engine, dtype):
    c = ctx()
    c.set_option(B.RAG_OPT_COPY_ENGINE, B.ENGINES[engine])
    big = _Case(W.ag_shape(4, 1, 512, 1024, 768, dtype=dtype, dist="normal_sqrtk", seed=71))
    small = _Case(W.ag_shape(2, 1, 128, 512, 256, dtype=dtype, dist="normal_sqrtk", seed=72))
    say(f"case noalloc engine={engine} {big.shape.name} then {small.shape.name}")
    big.reference(c)
    small.reference(c)
    torch.cuda.synchronize()
    c.check()
    # the two calls back to back, no synchronisation between them
    big.noalloc(c)
    small.noalloc(c)
    torch.cuda.synchronize()
    c.check()
    big.check("first call")
    small.check("second call")


def test_noalloc_repeated_calls_allocate_nothing():
    """After a first call, further calls change neither the device's free memory nor torch's
    allocator state; outputs stay equal to ag_gemm's."""
    c = ctx()
    c.set_option(B.RAG_OPT_COPY_ENGINE, B.ENGINES["in-gemm"])
    case = _Case(W.ag_shape(4, 2, 256, 1024, 512, dist="int3", seed=73))
    case.reference(c)
    case.noalloc(c)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    alloc0 = torch.cuda.memory_allocated()
    for _ in range(20):
        case.noalloc(c)
    torch.cuda.synchronize()
    c.check()
    assert torch.cuda.mem_get_info()[0] == free0
    assert torch.cuda.memory_allocated() == alloc0
    case.check("repeated calls")


def test_noalloc_rejects_what_would_allocate():
    c = ctx()
    case = _Case(W.ag_shape(2, 0, 64, 256, 128, dist="int3", seed=74))
    s = case.shape
    with pytest.raises(RuntimeError, match="G must be given"):
        B.ag_gemm_noalloc(c, case.A, case.chunks, s.tp, s.self_rank, case.D, None)
    for flag in (B.RAG_STAGED_OUT, B.RAG_PER_CHUNK):
        with pytest.raises(RuntimeError, match="not available"):
            case.noalloc(c, flags=flag)
    chunks = case.chunks * 9
    with pytest.raises(RuntimeError, match="fixed scratch array"):
        B.ag_gemm_noalloc(c, case.A, chunks[:17], 17, 0, torch.empty(
            (17 * 64, 128), dtype=torch.bfloat16, device=DEV), torch.empty(
            (17 * 64, 256), dtype=torch.bfloat16, device=DEV))
