"""Argument validation of the C ABI with a real context (GPU): every bad argument is refused
with RAG_EINVAL and a message, and nothing is enqueued."""
import ctypes

import pytest
import torch

from ring_all_gather_amd import binding as B

from gpu_common import DEV, ctx, reset_options, say

pytestmark = pytest.mark.gpu


def _ag(c, A, M, K, chunks, nc, tp, s, G, D, dt=0, sa=None, sb=None, flags=0):
    ptrs = (ctypes.c_void_p * max(len(chunks), 1))(*[ctypes.c_void_p(x) for x in chunks])
    return B.lib().ag_gemm(c.h, A, M, K, ptrs, nc, tp, s, G, D, dt, sa, sb, flags, None)


def test_ag_gemm_rejects_bad_arguments():
    c = ctx()
    say("case abi validation")
    A = torch.zeros((64, 128), dtype=torch.bfloat16, device=DEV)
    b = [torch.zeros((32, 128), dtype=torch.bfloat16, device=DEV) for _ in range(2)]
    D = torch.zeros((64, 64), dtype=torch.bfloat16, device=DEV)
    Ap, Dp = A.data_ptr(), D.data_ptr()
    bp = [x.data_ptr() for x in b]
    good = dict(A=Ap, M=64, K=128, chunks=bp, nc=32, tp=2, s=0, G=None, D=Dp)
    assert _ag(c, **good) == B.RAG_OK
    torch.cuda.synchronize()
    bad = [
        (dict(tp=0), "tp="), (dict(tp=17), "tp="), (dict(s=2), "self_rank"), (dict(s=-1), "self_rank"),
        (dict(K=100), "multiple of 64"), (dict(M=0), ">= 1"), (dict(nc=0), ">= 1"),
        (dict(A=None), "NULL"), (dict(D=None), "NULL"), (dict(A=Ap + 2), "aligned"),
        (dict(D=Dp + 8), "aligned"), (dict(chunks=[bp[0], 0]), "B_chunks[1]"),
        (dict(flags=16), "flag"), (dict(flags=B.RAG_NO_COPY | B.RAG_COPY_ONLY), "exclude"),
        (dict(D=Ap), "overlap"), (dict(dt=5), "dtype"),
    ]
    for change, needle in bad:
        args = dict(good)
        args.update(change)
        rc = _ag(c, **args)
        assert rc == B.RAG_EINVAL, (change, rc)
        assert needle in B.last_error(), (change, B.last_error())
    # a host pointer must never reach a kernel
    host = (ctypes.c_char * (64 * 128 * 2))()
    args = dict(good, A=ctypes.addressof(host))
    assert _ag(c, **args) == B.RAG_EINVAL
    assert "device memory" in B.last_error()
    # fp8 needs both scales, bf16 takes none
    s = torch.ones(1, device=DEV)
    assert _ag(c, **good, dt=1) == B.RAG_EINVAL
    assert _ag(c, **good, sa=s.data_ptr(), sb=s.data_ptr()) == B.RAG_EINVAL
    # tp above the context's max_tp
    small = B.Context(0, max_tp=2)
    assert _ag(small, **dict(good, tp=3, chunks=bp + [bp[0]])) == B.RAG_EINVAL
    small.close()
    torch.cuda.synchronize()


def test_gemm_rs_rejects_bad_arguments():
    c = ctx()
    X = torch.zeros((64, 128), dtype=torch.bfloat16, device=DEV)
    Wt = torch.zeros((48, 128), dtype=torch.bfloat16, device=DEV)
    P = torch.zeros((64, 48), dtype=torch.float32, device=DEV)
    D = torch.zeros((32, 48), dtype=torch.bfloat16, device=DEV)
    parts = (ctypes.c_void_p * 2)(None, ctypes.c_void_p(P.data_ptr()))
    L = B.lib()

    def rs(T=64, Kl=128, Mo=48, ldp=48, tp=2, s=0, Dp=D.data_ptr(), flags=0, Xp=X.data_ptr()):
        return L.gemm_rs(c.h, Xp, T, Kl, Wt.data_ptr(), Mo, parts, ldp, tp, s, None, Dp, flags,
                         None)

    assert rs() == B.RAG_OK
    torch.cuda.synchronize()
    for kw, needle in [(dict(T=63), "multiple of tp"), (dict(Kl=100), "multiple of 64"),
                       (dict(ldp=40), "ldp"), (dict(s=2), "self_rank"), (dict(flags=1), "flags"),
                       (dict(Dp=0), "NULL"), (dict(Dp=P.data_ptr()), "overlap"),
                       (dict(Xp=X.data_ptr() + 4), "aligned"),
                       (dict(ldp=(1 << 20) + 4), "at most"),
                       (dict(Mo=(1 << 20) + 4, ldp=(1 << 20) + 4), "at most")]:
        assert rs(**kw) == B.RAG_EINVAL, kw
        assert needle in B.last_error(), (kw, B.last_error())


def test_automatic_tile_choice_by_shape():
    """The automatic tile: the largest that gives every compute unit a tile, and between the two
    8-wave sizes the one whose persistent rounds leave the least to do (whole rounds of 256x192
    where 256x256 would leave a partial one).  Checked on the measured workloads' shapes, on a
    GPU with 256 compute units."""
    c = ctx()
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    say(f"case automatic tiles, {n_cu} compute units")
    if n_cu != 256:
        pytest.skip("the expected choices assume 256 compute units")
    reset_options(c)   # automatic tile
    c.set_option(B.RAG_OPT_COPY_ENGINE, B.ENGINES["in-gemm"])   # (no copy kernel beside the GEMM)
    try:
        assert c.ag_kernel_name(1024, 4096, 4) == "rag_ag_bf16_t256x256w8"   # 256 tiles: 1 round
        assert c.ag_kernel_name(1024, 3072, 8) == "rag_ag_bf16_t256x192w8"   # 512 vs 384 tiles
        # (K-slab gating: the slab kernels of the same tiles)
        c.set_option(B.RAG_OPT_AG_GATE, B.RAG_GATE_SLAB)
        assert c.ag_kernel_name(1024, 4096, 4) == "rag_ag_bf16_slab_t256x256w8"
        assert c.ag_kernel_name(1024, 3072, 8) == "rag_ag_bf16_slab_t256x192w8"
        c.set_option(B.RAG_OPT_AG_GATE, B.RAG_GATE_CHUNK)
        assert c.ag_kernel_name(2048, 3584, 8, fp8=True) == "rag_ag_fp8_t256x256w8"
        assert c.rs_kernel_name(1024, 8192, 8) == "rag_rs_t256x256w8"        # 1024 tiles: 4 rounds
        assert c.ag_kernel_name(256, 1024, 2) == "rag_ag_bf16_t128x128"      # too few big tiles
        # engines whose copies or counter writes run beside the GEMM get a kernel that leaves them
        # room on every SIMD: the fp8 256x256 8-wave kernel (254 registers at two waves per SIMD)
        # gives way to the 4-stage one for the copy kernel and for SDMA, whose counters the
        # runtime's write-value kernel releases
        for engine in ("kernel", "sdma"):
            c.set_option(B.RAG_OPT_COPY_ENGINE, B.ENGINES[engine])
            assert c.ag_kernel_name(2048, 3584, 8, fp8=True) == "rag_ag_fp8_t256x256w8s4", engine
        # the assisting copy kernel runs only when a later round needs chunks: one round (ag_4k)
        # keeps the in-GEMM kernel
        c.set_option(B.RAG_OPT_COPY_ENGINE, B.ENGINES["assist"])
        assert c.ag_kernel_name(1024, 4096, 4) == "rag_ag_bf16_t256x256w8"
        # SDMA for the late chunks: the GEMM leaves the write-value kernel room where there are
        # late chunks (fp8 ag_fc1_f8: the 4-stage tile; bf16 ag_qkv: the 256x192 kernel has room),
        # and one round (ag_4k) is the in-GEMM call
        c.set_option(B.RAG_OPT_COPY_ENGINE, B.ENGINES["in-gemm-sdma"])
        assert c.ag_kernel_name(1024, 4096, 4) == "rag_ag_bf16_t256x256w8"
        assert c.ag_kernel_name(1024, 3072, 8) == "rag_ag_bf16_t256x192w8"
        assert c.ag_kernel_name(2048, 3584, 8, fp8=True) == "rag_ag_fp8_t256x256w8s4"
    finally:
        reset_options(c)


def test_set_option_rejects_bad_values():
    """Every option refuses out-of-range values with RAG_EINVAL and leaves the context usable."""
    c = ctx()
    say("case option validation")
    bad = [(B.RAG_OPT_COPY_ENGINE, 5), (B.RAG_OPT_COPY_ENGINE, -1), (B.RAG_OPT_COMM_CUS, 4),
           (B.RAG_OPT_COMM_CUS, 12), (B.RAG_OPT_COMM_CUS, 256), (B.RAG_OPT_SDMA_STREAMS, 0),
           (B.RAG_OPT_SDMA_STREAMS, 4), (B.RAG_OPT_TILE, 99), (B.RAG_OPT_COMM_WGS, 0),
           (B.RAG_OPT_AG_GATE, 2), (B.RAG_OPT_AG_GATE, -1), (B.RAG_OPT_SLAB_HELP_US, -1),
           (B.RAG_OPT_SLAB_HELP_US, 10_000_001), (999, 1)]
    for key, value in bad:
        rc = B.lib().rag_set_option(c.h, key, value)
        assert rc == B.RAG_EINVAL, (key, value, rc)
        assert B.last_error(), (key, value)
    for key, value in [(B.RAG_OPT_COMM_CUS, 8), (B.RAG_OPT_COMM_CUS, 0),
                       (B.RAG_OPT_SDMA_STREAMS, 3), (B.RAG_OPT_SDMA_STREAMS, 1),
                       (B.RAG_OPT_COPY_ENGINE, B.RAG_COPY_IN_GEMM_ASSIST)]:
        assert B.lib().rag_set_option(c.h, key, value) == B.RAG_OK, (key, value)
    reset_options(c)
