"""GPU parity of the AG+GEMM path (libringag.so through the C ABI) against the CPU oracle."""
import numpy as np
import pytest
import torch

from oracle import ringag_oracle as O
from ring_all_gather_amd import binding as B
from ring_all_gather_amd import workloads as W

from gpu_common import (DEV, AGRun, TOL_BF16, TOL_FP8, cached, ctx, oracle_ag, rel_err,
                        reset_options, say)

pytestmark = pytest.mark.gpu

TILE_NAMES = ["128x128", "256x128", "256x256", "256x256w8", "256x256w8s4", "256x192w8"]
# copy engines of the simulated arrival that run on compute units: the side-stream copy kernel, the
# GEMM's own workgroups (gating by chunk, or by K slab where that applies), and both on one queue
# (SDMA is covered in the flags test)
ENGINES = ["kernel", "in-gemm", "in-gemm-slab", "assist"]


def set_engine(c, engine):
    c.set_option(B.RAG_OPT_COPY_ENGINE, B.ENGINES[engine.replace("-slab", "")])
    c.set_option(B.RAG_OPT_AG_GATE,
                 B.RAG_GATE_SLAB if engine.endswith("-slab") else B.RAG_GATE_CHUNK)


@pytest.fixture(autouse=True)
def _fresh_options():
    reset_options(ctx())
    yield
    reset_options(ctx())


def test_ag_tiny_workload_full_parity():
    shape = W.WORKLOADS["ag_tiny"]
    say(f"case {shape}")
    inp = W.make_ag(shape)
    run = AGRun(inp).run(ctx())
    G_ref, ref = oracle_ag(inp)
    assert np.array_equal(W.bits_u16(run.G.cpu()), G_ref)
    assert rel_err(run.D_bits(), ref) <= TOL_BF16


def _int_case(tp, s, nc, K, M, seed, dtype="bf16"):
    return W.make_ag(W.ag_shape(tp, s, nc, K, M, dtype=dtype, dist="int3", seed=seed))


CASES = [(tp, s, nc) for tp in (1, 2, 3, 4, 8) for s in range(tp) for nc in (16, 48, 256)]


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("tp,s,nc", CASES)
def test_ag_exact_integers_every_rank(tp, s, nc, engine):
    """Small integers are exact in bf16 and their fp32 sums are exact in any order, so D must be
    the oracle's sum rounded to bf16, bit for bit; G must be the rank-ordered concatenation."""
    c = ctx()
    set_engine(c, engine)
    tile = TILE_NAMES[(tp + s + nc) % len(TILE_NAMES)]
    c.set_option(B.RAG_OPT_TILE, B.TILES[tile])
    inp = _int_case(tp, s, nc, K=128, M=80, seed=tp * 100 + s * 10 + nc)
    say(f"case tp={tp} s={s} nc={nc} K=128 M=80 tile={tile} engine={engine}")
    run = AGRun(inp).run(c)
    G_ref, ref = oracle_ag(inp)
    assert np.array_equal(W.bits_u16(run.G.cpu()), G_ref)
    assert np.array_equal(run.D_bits(), O.f32_to_bf16(ref))


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("tile", TILE_NAMES)
def test_ag_ragged_tiles_random(tile, engine):
    """Chunk rows and output columns that are not multiples of any tile (several tiles plus a
    ragged tail in both directions), normal data, every tile configuration."""
    c = ctx()
    set_engine(c, engine)
    c.set_option(B.RAG_OPT_TILE, B.TILES[tile])
    shape = W.ag_shape(3, 2, 300, 320, 333, dist="normal_sqrtk", seed=5)
    say(f"case {shape.name} tile={tile} engine={engine}")
    inp = W.make_ag(shape)
    run = AGRun(inp).run(c)
    G_ref, ref = oracle_ag(inp)
    assert np.array_equal(W.bits_u16(run.G.cpu()), G_ref)
    assert rel_err(run.D_bits(), ref) <= TOL_BF16


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("nsteps", [1, 2, 3])
@pytest.mark.parametrize("tile", TILE_NAMES)
def test_ag_short_k_every_tile(tile, nsteps, dtype):
    """K of one, two and three 128-byte k-steps: the K loop's first stage alone, one stage
    handover, and the DMA past the last stage that the loop drains; exact integers on a ragged
    shape, every tile."""
    c = ctx()
    c.set_option(B.RAG_OPT_TILE, B.TILES[tile])
    K = nsteps * (128 if dtype == "fp8" else 64)
    inp = _int_case(2, 1, 100, K=K, M=90, seed=900 + nsteps, dtype=dtype)
    say(f"case short K={K} dtype={dtype} tile={tile}")
    run = AGRun(inp).run(c)
    G_ref, ref = oracle_ag(inp)
    bits = W.bits_u8 if dtype == "fp8" else W.bits_u16
    assert np.array_equal(bits(run.G.cpu()), G_ref)
    assert np.array_equal(run.D_bits(), O.f32_to_bf16(ref))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("M", [1280, 3072, 2916], ids=["whole", "half", "half-ragged"])
def test_ag_rounds_whole_and_half_tiles(M, dtype):
    """The 8-wave 256x256 tile runs a round that is at most half full as twice as many 256x128
    half tiles.  tp=4 with 2048-row chunks gives 8 row blocks per chunk: M = 1280 gives 160 tiles
    on a grid of 256 workgroups (whole tiles), 3072 gives 384 (256 whole, then 128 split), and
    2916 gives 384 too, with a last column block 100 columns wide, so that its right halves have
    nothing to do; exact integers, D bit for bit."""
    c = ctx()
    c.set_option(B.RAG_OPT_TILE, B.TILES["256x256w8"])
    K = 256 if dtype == "fp8" else 128
    inp = _int_case(4, 1, 2048, K=K, M=M, seed=1300 + M, dtype=dtype)
    say(f"case rounds M={M} dtype={dtype}")
    run = AGRun(inp).run(c)
    G_ref, ref = oracle_ag(inp)
    bits = W.bits_u8 if dtype == "fp8" else W.bits_u16
    assert np.array_equal(bits(run.G.cpu()), G_ref)
    assert np.array_equal(run.D_bits(), O.f32_to_bf16(ref))


def test_ag_bitwise_invariant_across_ranks_and_modes():
    """Chunking splits the gathered rows, not K: the result must not depend on the self rank,
    on whether chunks arrive (counters) or are already there, or on the split at all (tp=1)."""
    c = ctx()
    shape = W.ag_shape(4, 0, 200, 256, 200, dist="normal_sqrtk", seed=9)
    inp = W.make_ag(shape)
    run = AGRun(inp)
    outs = []
    for s in range(4):
        say(f"case invariance s={s}")
        run.run(c, self_rank=s)
        outs.append(run.D_bits())
        assert np.array_equal(W.bits_u16(run.G.cpu()), O.gather([W.bits_u16(x) for x in inp.chunks]))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    run.D.zero_()
    run.run(c, flags=B.RAG_NO_COPY, self_rank=2)
    assert np.array_equal(run.D_bits(), outs[0])
    # tp = 1 on the gathered input
    G = run.G.clone()
    D1 = torch.empty_like(run.D)
    B.ag_gemm(c, run.A, [G], 1, 0, D1)
    torch.cuda.synchronize()
    assert np.array_equal(W.bits_u16(D1.cpu()), outs[0])
    _, ref = oracle_ag(inp)
    assert rel_err(outs[0], ref) <= TOL_BF16


@pytest.mark.parametrize("engine", ENGINES)
def test_ag_flags_staged_copy_only_sdma(engine):
    c = ctx()
    set_engine(c, engine)
    for tp, s in ((4, 1), (2, 1), (3, 0), (1, 0)):
        inp = W.make_ag(W.ag_shape(tp, s, 96, 192, 160, dist="int3", seed=tp + s))
        _, ref = oracle_ag(inp)
        want = O.f32_to_bf16(ref)
        G_ref = O.gather([W.bits_u16(x) for x in inp.chunks])
        run = AGRun(inp)
        say(f"case staged tp={tp} s={s}")
        run.run(c, flags=B.RAG_STAGED_OUT)
        assert np.array_equal(run.D_bits(), want)
        say(f"case copy-only tp={tp} s={s}")
        run.D.fill_(7.0)
        run.G.zero_()
        run.run(c, flags=B.RAG_COPY_ONLY)
        assert np.array_equal(W.bits_u16(run.G.cpu()), G_ref)
        assert bool((run.D.float() == 7.0).all())
        say(f"case sdma tp={tp} s={s}")
        set_engine(c, "sdma")
        run.G.zero_()
        run.run(c)
        assert np.array_equal(run.D_bits(), want)
        assert np.array_equal(W.bits_u16(run.G.cpu()), G_ref)
        set_engine(c, engine)


@pytest.mark.parametrize("engine", ["assist", "in-gemm-sdma"])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("tp,s,wgs_per_cu", [(8, 3, 0), (8, 0, 1), (4, 2, 1), (16, 9, 0)])
def test_ag_late_queue_exact(tp, s, wgs_per_cu, dtype, engine):
    """Shapes whose GEMM needs several persistent rounds, so that the late chunks are copied
    beside the first round (by the assisting copy kernel, or by SDMA) while the GEMM's waiting
    workgroups copy the early ones: exact integer parity, three calls back to back with fresh
    data, then an in-GEMM call."""
    c = ctx()
    set_engine(c, engine)
    c.set_option(B.RAG_OPT_TILE, B.TILES["128x128"])
    c.set_option(B.RAG_OPT_WGS_PER_CU, wgs_per_cu)
    runs = []
    for it in range(3):
        # 128x128 tiles: chunks of 4 x 32 tiles, so the persistent grid (512, or 256 with one
        # workgroup per CU) covers the first 4 (or 2) ring positions in its first round
        inp = W.make_ag(W.ag_shape(tp, s, 512, 256, 4096, dtype=dtype, dist="int3",
                                   seed=80 + it + tp))
        runs.append((AGRun(inp), inp))
    say(f"case late queue {engine} tp={tp} s={s} wgs/cu={wgs_per_cu} {dtype}")
    for run, inp in runs:
        sh = inp.shape
        B.ag_gemm(c, run.A, run.chunks, sh.tp, sh.self_rank, run.D, G=run.G, scale_A=run.sA,
                  scale_B=run.sB)
    set_engine(c, "in-gemm")
    run0, inp0 = runs[0]
    D2 = torch.empty_like(run0.D)
    B.ag_gemm(c, run0.A, run0.chunks, tp, s, D2, G=run0.G, scale_A=run0.sA, scale_B=run0.sB)
    torch.cuda.synchronize()
    c.check()
    for run, inp in runs:
        G_ref, ref = oracle_ag(inp)
        assert np.array_equal(run.D_bits(), O.f32_to_bf16(ref))
        Gb = W.bits_u8(run.G.cpu()) if dtype == "fp8" else W.bits_u16(run.G.cpu())
        assert np.array_equal(Gb, G_ref)
    assert torch.equal(D2.view(torch.int16), run0.D.view(torch.int16))


@pytest.mark.parametrize("streams", [1, 2, 3])
def test_ag_sdma_spread_over_streams(streams):
    """SDMA copies spread over 1-3 side streams: every chunk lands, D and G exact, with the own
    chunk copied into G, with B_copy (joined by events) and copy-only."""
    c = ctx()
    set_engine(c, "sdma")
    c.set_option(B.RAG_OPT_SDMA_STREAMS, streams)
    for tp, s in ((8, 5), (4, 1), (3, 2)):
        inp = W.make_ag(W.ag_shape(tp, s, 64, 128, 192, dist="int3", seed=40 + tp + s))
        _, ref = oracle_ag(inp)
        G_ref = O.gather([W.bits_u16(x) for x in inp.chunks])
        say(f"case sdma streams={streams} tp={tp} s={s}")
        run = AGRun(inp).run(c)
        assert np.array_equal(run.D_bits(), O.f32_to_bf16(ref))
        assert np.array_equal(W.bits_u16(run.G.cpu()), G_ref)
        Bc = torch.zeros_like(run.chunks[s])
        run.G.zero_()
        B.ag_gemm(c, run.A, run.chunks, tp, s, run.D, G=run.G, B_copy=Bc)
        torch.cuda.synchronize()
        assert np.array_equal(W.bits_u16(run.G.cpu()), G_ref)
        assert torch.equal(Bc.view(torch.int16), run.chunks[s].view(torch.int16))
        run.G.zero_()
        run.run(c, flags=B.RAG_COPY_ONLY)
        assert np.array_equal(W.bits_u16(run.G.cpu()), G_ref)
    c.check()


@pytest.mark.parametrize("engine", ["kernel", "assist"])
def test_ag_comm_cus_masked_side_stream(engine):
    """The side stream limited to 32 compute units (4 per XCD): exact results from a caller on a
    stream of its own (where the copies overlap the GEMM) and on the null stream (which the masked
    stream serialises with), back to back with fresh data, then the option switched off again."""
    c = ctx()
    set_engine(c, engine)
    c.set_option(B.RAG_OPT_COMM_CUS, 32)
    try:
        st = torch.cuda.Stream()
        for it, (tp, s) in enumerate(((4, 1), (8, 6), (4, 1))):
            inp = W.make_ag(W.ag_shape(tp, s, 256, 512, 512, dist="int3", seed=60 + it))
            _, ref = oracle_ag(inp)
            run = AGRun(inp)
            say(f"case comm_cus=32 engine={engine} tp={tp} s={s} (own stream)")
            with torch.cuda.stream(st):
                B.ag_gemm(c, run.A, run.chunks, tp, s, run.D, G=run.G)
            torch.cuda.synchronize()
            assert np.array_equal(run.D_bits(), O.f32_to_bf16(ref))
            say(f"case comm_cus=32 engine={engine} tp={tp} s={s} (null stream)")
            run.D.zero_()
            run.run(c)
            assert np.array_equal(run.D_bits(), O.f32_to_bf16(ref))
        c.check()
    finally:
        c.set_option(B.RAG_OPT_COMM_CUS, 0)


@pytest.mark.parametrize("engine", ENGINES)
def test_ag_internal_gather_buffer(engine):
    c = ctx()
    set_engine(c, engine)
    inp = W.make_ag(W.ag_shape(4, 3, 64, 128, 96, dist="int3", seed=3))
    run = AGRun(inp, with_G=False)
    say("case G=NULL")
    run.run(c)
    _, ref = oracle_ag(inp)
    assert np.array_equal(run.D_bits(), O.f32_to_bf16(ref))


@pytest.mark.parametrize("engine", ENGINES)
def test_ag_gating_delayed_arrivals_on_poisoned_slots(engine):
    """Every slot of G is NaN before the call and each arrival is held back 2 ms after its copy:
    a tile that read its chunk before the counter said so would produce NaN or a wrong value."""
    c = ctx()
    set_engine(c, engine)
    c.set_option(B.RAG_OPT_ARRIVAL_DELAY_US, 2000)
    inp = W.make_ag(W.ag_shape(4, 1, 256, 256, 256, dist="int3", seed=17))
    _, ref = oracle_ag(inp)
    want = O.f32_to_bf16(ref)
    run = AGRun(inp)
    for it in range(3):
        say(f"case gating it={it} engine={engine}")
        run.G.fill_(float("nan"))
        run.D.fill_(float("nan"))
        run.run(c)
        assert np.array_equal(run.D_bits(), want)


@pytest.mark.parametrize("engine", ENGINES)
def test_ag_withheld_chunk_times_out_and_context_recovers(engine):
    c = ctx()
    set_engine(c, engine)
    c.set_option(B.RAG_OPT_SPIN_LIMIT_US, 20000)
    c.set_option(B.RAG_OPT_WITHHOLD_MASK, 1 << 2)
    inp = W.make_ag(W.ag_shape(4, 0, 128, 128, 128, dist="int3", seed=23))
    run = AGRun(inp)
    say(f"case withheld chunk engine={engine}")
    run.run(c)
    with pytest.raises(B.RagError) as ei:
        c.check()
    assert ei.value.code == B.RAG_ETIMEOUT
    c.set_option(B.RAG_OPT_WITHHOLD_MASK, 0)
    c.set_option(B.RAG_OPT_SPIN_LIMIT_US, 2_000_000)
    run.run(c)
    c.check()
    _, ref = oracle_ag(inp)
    assert np.array_equal(run.D_bits(), O.f32_to_bf16(ref))


@pytest.mark.parametrize("engine", ENGINES)
def test_ag_epoch_stress_fresh_data_same_buffers(engine):
    """Back-to-back calls in the same buffers with new data each time: stale cache lines or a
    counter left over from the previous call would show up as a mismatch."""
    c = ctx()
    set_engine(c, engine)
    shape = W.ag_shape(4, 2, 256, 256, 256, dist="int3", seed=0)
    run = AGRun(W.make_ag(shape))
    for it in range(30):
        inp = W.make_ag(W.ag_shape(4, 2, 256, 256, 256, dist="int3", seed=1000 + it))
        run.A.copy_(inp.A)
        for d, h in zip(run.chunks, inp.chunks):
            d.copy_(h)
        run.run(c)
        _, ref = oracle_ag(inp)
        if not np.array_equal(run.D_bits(), O.f32_to_bf16(ref)):
            pytest.fail(f"iteration {it} differs from its oracle")
    say(f"case epoch stress done engine={engine}")


@pytest.mark.parametrize("engine", ENGINES)
def test_ag_fp8_small_parity_and_exact(engine):
    c = ctx()
    set_engine(c, engine)
    shape = W.ag_shape(4, 3, 160, 256, 224, dtype="fp8", dist="normal", seed=31)
    say(f"case {shape.name}")
    inp = W.make_ag(shape)
    run = AGRun(inp).run(c)
    G_ref, ref = oracle_ag(inp)
    assert np.array_equal(W.bits_u8(run.G.cpu()), G_ref)
    assert rel_err(run.D_bits(), ref) <= TOL_FP8
    for tile in TILE_NAMES:
        c.set_option(B.RAG_OPT_TILE, B.TILES[tile])
        inp = W.make_ag(W.ag_shape(2, 1, 100, 256, 90, dtype="fp8", dist="int3", seed=37))
        say(f"case fp8 exact tile={tile}")
        run = AGRun(inp).run(c)
        _, ref = oracle_ag(inp)
        assert np.array_equal(run.D_bits(), O.f32_to_bf16(ref))


FULL_CASES = [(name, engine, placement) for name in ("ag_4k", "ag_qkv", "ag_fc1_f8")
              for engine in ENGINES for placement in ("separate", "in-g")] + [
    # SDMA at full size: its counters are released by the runtime's write-value kernel, which the
    # GEMM must leave room for (with the fp8 256x256 8-wave kernel filling every SIMD, every wait
    # ran out its limit)
    ("ag_fc1_f8", "sdma", "in-g"), ("ag_qkv", "sdma", "separate"),
    # the late chunks by SDMA beside in-GEMM copies of the early ones
    ("ag_qkv", "in-gemm-sdma", "in-g"), ("ag_fc1_f8", "in-gemm-sdma", "separate")]


@pytest.mark.parametrize("name,engine,placement", FULL_CASES)
def test_ag_full_size_full_output(name, engine, placement):
    """The measured workloads at full size: every element of D against the full oracle, and G
    against the explicit concatenation, bit for bit.  placement "in-g" is the benchmark's: the own
    chunk sits in its slot of G, so only the peers' chunks are copied."""
    shape = W.WORKLOADS[name]
    set_engine(ctx(), engine)
    say(f"case {shape} engine={engine} placement={placement}")
    inp = W.make_ag(shape)
    run = AGRun(inp, own_in_g=(placement == "in-g"))
    for _ in range(3):   # back to back
        B.ag_gemm(ctx(), run.A, run.chunks, shape.tp, shape.self_rank, run.D, G=run.G,
                  scale_A=run.sA, scale_B=run.sB)
    torch.cuda.synchronize()
    ctx().check()
    G_ref, ref = cached(("ag", name), lambda: oracle_ag(inp))
    tol = TOL_FP8 if shape.dtype == "fp8" else TOL_BF16
    err = rel_err(run.D_bits(), ref)
    say(f"{name}: all {ref.shape[0]} x {ref.shape[1]} outputs, max rel err {err:.3e}")
    assert err <= tol
    G = run.G.cpu()
    Gb = W.bits_u8(G) if shape.dtype == "fp8" else W.bits_u16(G)
    assert np.array_equal(Gb, G_ref)


SLAB_TILES = ["256x256w8", "256x192w8"]
# (K-slab gating needs a grid of at least half as many workgroups as a group has pieces, so the
# narrow shapes have enough output columns to give it one)
SLAB_CASES = [   # tp, s, nc, K, M
    (2, 1, 16, 64, 80),       # one K stage: only group 0, one piece per chunk
    (2, 0, 300, 320, 1100),   # rows not a multiple of 16; 640-byte rows: a 128-byte last group
    (3, 2, 48, 576, 200),     # 9 stages: gates at stages 2 and 6, copy cycles in the K loop
    (4, 1, 256, 1024, 2048),  # 16 stages
    (8, 5, 100, 2048, 1100),  # ragged rows and columns, 7 peers
    (16, 9, 64, 512, 300),    # 15 peers
    (8, 3, 600, 320, 4000),   # more tiles than compute units: later rounds, copy slots carried over
]


@pytest.mark.parametrize("help_us", [20, 0])
@pytest.mark.parametrize("tile", SLAB_TILES)
@pytest.mark.parametrize("tp,s,nc,K,M", SLAB_CASES)
def test_ag_slab_gating_exact(tp, s, nc, K, M, tile, help_us):
    """K-slab gating (in-GEMM engine, bf16, 8-wave 2-stage tiles): exact integers, G and D bit for
    bit, on shapes that exercise ragged rows and groups, one and many rounds and up to 15 peers.
    help_us = 0: a tile copies a slab's missing pieces itself as soon as it finds one (the path
    that keeps the launch going when the owners of pieces are late)."""
    c = ctx()
    set_engine(c, "in-gemm-slab")
    c.set_option(B.RAG_OPT_TILE, B.TILES[tile])
    c.set_option(B.RAG_OPT_SLAB_HELP_US, help_us)
    assert "_slab_" in c.ag_kernel_name(nc, M, tp)
    inp = _int_case(tp, s, nc, K=K, M=M, seed=5000 + tp * 37 + nc + K)
    say(f"case slab tp={tp} s={s} nc={nc} K={K} M={M} tile={tile} help_us={help_us}")
    for own_in_g in (False, True):
        run = AGRun(inp, own_in_g=own_in_g)
        run.run(c)
        c.check()
        G_ref, ref = oracle_ag(inp)
        assert np.array_equal(W.bits_u16(run.G.cpu()), G_ref)
        assert np.array_equal(run.D_bits(), O.f32_to_bf16(ref))


def test_ag_slab_fresh_data_poisoned_g():
    """The full-size ag_4k shape under K-slab gating, 24 calls back to back on one G that is
    refilled with NaN before each call, alternating two input sets: a tile that read a slab before
    its pieces landed, or a stale line of the previous call, would put NaN or the other set's
    product into D."""
    c = ctx()
    set_engine(c, "in-gemm-slab")
    base = W.WORKLOADS["ag_4k"]
    assert "_slab_" in c.ag_kernel_name(base.nc, base.M, base.tp)
    sets = []
    for seed in (base.seed, base.seed + 1):
        shape = W.ag_shape(base.tp, base.self_rank, base.nc, base.K, base.M,
                           dist="normal_sqrtk", seed=seed)
        inp = W.make_ag(shape)
        _, ref = cached(("ag_4k_seed", seed), lambda: oracle_ag(inp))
        sets.append((AGRun(inp), ref))
    G = torch.empty_like(sets[0][0].G)
    for i in range(24):
        run, ref = sets[i % 2]
        say(f"case slab fresh data call {i}")
        G.fill_(float("nan"))
        run.D.fill_(float("nan"))
        s = run.inp.shape
        B.ag_gemm(c, run.A, run.chunks, s.tp, s.self_rank, run.D, G=G)
        torch.cuda.synchronize()
        err = rel_err(run.D_bits(), ref)
        assert err <= TOL_BF16, (i, err)
    c.check()


SPLIT_CASES = [(1, 0, 48), (2, 1, 256), (3, 2, 300), (4, 1, 256), (8, 5, 48)]


@pytest.mark.parametrize("engine", ["kernel", "sdma"])
@pytest.mark.parametrize("tp,s,nc", SPLIT_CASES)
def test_ag_split_form_exact(tp, s, nc, engine):
    """RAG_PER_CHUNK: one GEMM launch per chunk, gated by stream events; same result, bit for
    bit, as the oracle on integer data, and G complete."""
    c = ctx()
    set_engine(c, engine)
    inp = _int_case(tp, s, nc, K=192, M=144, seed=500 + tp * 10 + s)
    say(f"case split tp={tp} s={s} nc={nc} engine={engine}")
    run = AGRun(inp).run(c, flags=B.RAG_PER_CHUNK)
    c.check()
    G_ref, ref = oracle_ag(inp)
    assert np.array_equal(W.bits_u16(run.G.cpu()), G_ref)
    assert np.array_equal(run.D_bits(), O.f32_to_bf16(ref))


def test_ag_split_form_flags_and_gating():
    """Split form with staged output, copies only, G = NULL, and arrivals held back 2 ms on
    NaN-poisoned slots (a GEMM launched before its chunk's event would read NaN)."""
    c = ctx()
    set_engine(c, "kernel")
    inp = _int_case(4, 2, 256, K=256, M=256, seed=77)
    _, ref = oracle_ag(inp)
    want = O.f32_to_bf16(ref)
    G_ref = O.gather([W.bits_u16(x) for x in inp.chunks])
    run = AGRun(inp)
    say("case split staged")
    run.run(c, flags=B.RAG_PER_CHUNK | B.RAG_STAGED_OUT)
    assert np.array_equal(run.D_bits(), want)
    say("case split copy-only")
    run.D.fill_(7.0)
    run.G.zero_()
    run.run(c, flags=B.RAG_PER_CHUNK | B.RAG_COPY_ONLY)
    assert np.array_equal(W.bits_u16(run.G.cpu()), G_ref)
    assert bool((run.D.float() == 7.0).all())
    say("case split no-copy")
    run.D.zero_()
    run.run(c, flags=B.RAG_PER_CHUNK | B.RAG_NO_COPY)
    assert np.array_equal(run.D_bits(), want)
    say("case split G=NULL")
    run2 = AGRun(inp, with_G=False).run(c, flags=B.RAG_PER_CHUNK)
    assert np.array_equal(run2.D_bits(), want)
    c.set_option(B.RAG_OPT_ARRIVAL_DELAY_US, 2000)
    for it in range(2):
        say(f"case split gating it={it}")
        run.G.fill_(float("nan"))
        run.D.fill_(float("nan"))
        run.run(c, flags=B.RAG_PER_CHUNK)
        assert np.array_equal(run.D_bits(), want)
    c.check()


# --------------------------------------------------------- fp8 output (amax, scale) and B_copy

def _fp8_out_run(inp, c, scale_d, flags=0, with_copy=True):
    s = inp.shape
    run = AGRun(inp)
    D8 = torch.zeros((s.N, s.M), dtype=torch.float8_e4m3fn, device=DEV)
    sD = torch.tensor([scale_d], dtype=torch.float32, device=DEV)
    amax = torch.zeros(1, dtype=torch.float32, device=DEV)
    bc = torch.zeros_like(run.chunks[s.self_rank]) if with_copy else None
    B.ag_gemm(c, run.A, run.chunks, s.tp, s.self_rank, D8, G=run.G, scale_A=run.sA,
              scale_B=run.sB, flags=flags, scale_D=sD, amax_D=amax, B_copy=bc)
    torch.cuda.synchronize()
    c.check()
    return run, W.bits_u8(D8.cpu()), float(amax.cpu()[0]), bc


@pytest.mark.parametrize("engine", ENGINES + ["sdma"])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_ag_fp8_output_exact_integers(dtype, engine):
    """fp8 output: codes = E4M3(result * scale_D) bit for bit on integer data (the result is exact,
    so both sides round the same value), amax = max |result|, B_copy = this rank's chunk."""
    c = ctx()
    set_engine(c, engine)
    for tp, s, nc in ((4, 1, 256), (3, 2, 300), (1, 0, 48)):
        inp = W.make_ag(W.ag_shape(tp, s, nc, 256, 160, dtype=dtype, dist="int3",
                                   seed=1100 + tp * 10 + s))
        say(f"case fp8-out {dtype} tp={tp} s={s} nc={nc} engine={engine}")
        run, codes, amax, bc = _fp8_out_run(inp, c, 0.75)
        _, ref = oracle_ag(inp)
        want, want_amax = O.quantize_output_e4m3(ref, 0.75)
        assert np.array_equal(codes, want)
        assert amax == want_amax
        src = inp.chunks[s]
        bits = W.bits_u8 if dtype == "fp8" else W.bits_u16
        assert np.array_equal(bits(bc.cpu()), bits(src))


@pytest.mark.parametrize("tile", TILE_NAMES)
def test_ag_fp8_output_random_every_tile(tile):
    """Random data, ragged shape: the codes may differ from the oracle's only where the fp32
    result itself differs in its last bits (a different accumulation order), so each decoded value
    is within one E4M3 step of the oracle's; amax within fp32 rounding."""
    c = ctx()
    set_engine(c, "in-gemm")
    c.set_option(B.RAG_OPT_TILE, B.TILES[tile])
    inp = W.make_ag(W.ag_shape(3, 1, 300, 320, 333, dist="normal_sqrtk", seed=61))
    say(f"case fp8-out random tile={tile}")
    run, codes, amax, _ = _fp8_out_run(inp, c, 64.0, with_copy=False)
    _, ref = oracle_ag(inp)
    want, want_amax = O.quantize_output_e4m3(ref, 64.0)
    got_v, want_v = O.e4m3fn_to_f32(codes), O.e4m3fn_to_f32(want)
    step = np.maximum(np.abs(want_v) / 8.0, 2.0 ** -9)   # one E4M3 step at that magnitude
    assert np.all(np.abs(got_v - want_v) <= step + 1e-12)
    assert np.mean(codes == want) > 0.99
    assert abs(amax - want_amax) <= 1e-3 * want_amax


def test_ag_fp8_output_staged_and_split():
    c = ctx()
    set_engine(c, "kernel")
    inp = W.make_ag(W.ag_shape(4, 2, 128, 192, 96, dist="int3", seed=71))
    _, ref = oracle_ag(inp)
    want, want_amax = O.quantize_output_e4m3(ref, 2.0)
    for flags in (B.RAG_STAGED_OUT, B.RAG_PER_CHUNK, B.RAG_PER_CHUNK | B.RAG_STAGED_OUT):
        say(f"case fp8-out flags={flags}")
        run, codes, amax, bc = _fp8_out_run(inp, c, 2.0, flags=flags)
        assert np.array_equal(codes, want)
        assert amax == want_amax
        assert np.array_equal(W.bits_u16(bc.cpu()), W.bits_u16(inp.chunks[2]))


@pytest.mark.parametrize("tile", SLAB_TILES)
def test_ag_slab_fp8_output_and_b_copy(tile):
    """The E4M3-output K-slab kernels (rag_ag_bf16_o8_slab_*): codes and amax bit for bit on
    integer data, B_copy and the own chunk's copy into G after the slab copies."""
    c = ctx()
    set_engine(c, "in-gemm-slab")
    c.set_option(B.RAG_OPT_TILE, B.TILES[tile])
    tp, s, nc, K, M = 4, 1, 256, 576, 2048
    assert "_slab_" in c.ag_kernel_name(nc, M, tp)
    inp = W.make_ag(W.ag_shape(tp, s, nc, K, M, dist="int3", seed=1201))
    say(f"case slab fp8-out tile={tile}")
    run, codes, amax, bc = _fp8_out_run(inp, c, 0.5)
    G_ref, ref = oracle_ag(inp)
    want, want_amax = O.quantize_output_e4m3(ref, 0.5)
    assert np.array_equal(codes, want)
    assert amax == want_amax
    assert np.array_equal(W.bits_u16(bc.cpu()), W.bits_u16(inp.chunks[s]))
    assert np.array_equal(W.bits_u16(run.G.cpu()), G_ref)


def test_ag_b_copy_bf16_output_and_validation():
    """B_copy alone (bf16 output), and the argument checks of the extended call."""
    c = ctx()
    set_engine(c, "in-gemm")
    inp = W.make_ag(W.ag_shape(2, 1, 64, 128, 64, dist="int3", seed=81))
    run = AGRun(inp)
    bc = torch.zeros_like(run.chunks[1])
    B.ag_gemm(c, run.A, run.chunks, 2, 1, run.D, G=run.G, B_copy=bc)
    torch.cuda.synchronize()
    _, ref = oracle_ag(inp)
    assert np.array_equal(run.D_bits(), O.f32_to_bf16(ref))
    assert np.array_equal(W.bits_u16(bc.cpu()), W.bits_u16(inp.chunks[1]))
    D8 = torch.zeros(run.D.shape, dtype=torch.float8_e4m3fn, device=DEV)
    with pytest.raises(B.RagError):   # fp8 output without scale_D
        B.ag_gemm(c, run.A, run.chunks, 2, 1, D8, G=run.G, B_copy=bc)
    assert "scale_D" in B.last_error()
    sD = torch.ones(1, device=DEV)
    with pytest.raises(B.RagError):   # B_copy overlapping G
        B.ag_gemm(c, run.A, run.chunks, 2, 1, D8, G=run.G, scale_D=sD, B_copy=run.G[:64])
    assert "overlap" in B.last_error()
