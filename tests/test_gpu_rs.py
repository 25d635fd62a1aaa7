"""GPU parity of the GEMM+RS path (libringag.so through the C ABI) against the CPU oracle."""
import numpy as np
import pytest
import torch

from oracle import ringag_oracle as O
from ring_all_gather_amd import binding as B
from ring_all_gather_amd import workloads as W

from gpu_common import DEV, TOL_BF16, TOL_SEND, cached, ctx, rel_err, reset_options, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _fresh_options():
    reset_options(ctx())
    yield
    reset_options(ctx())


class RSRun:
    def __init__(self, inp: W.RSInputs, with_send=True):
        s = inp.shape
        self.inp = inp
        self.X = inp.X.to(DEV)
        self.W = inp.W.to(DEV)
        self.partials = [None if p is None else p.to(DEV) for p in inp.partials]
        self.D = torch.empty((s.nc, s.Mo), dtype=torch.bfloat16, device=DEV)
        self.send = torch.full((s.tp, s.nc, s.Mo), float("nan"), device=DEV) if with_send else None

    def run(self, c):
        s = self.inp.shape
        B.gemm_rs(c, self.X, self.W, self.partials, s.tp, s.self_rank, self.D, send=self.send)
        torch.cuda.synchronize()
        return self


def oracle_rs(inp: W.RSInputs):
    s = inp.shape
    peers = [None if p is None else p.numpy() for p in inp.partials]
    return O.gemm_rs(W.bits_u16(inp.X), W.bits_u16(inp.W), peers, s.tp, s.self_rank)


def _check_send(run, send_ref, exact=False):
    s = run.inp.shape
    got = run.send.cpu().numpy()
    for c in range(s.tp):
        if c == s.self_rank:
            assert np.isnan(got[c]).all(), "the own slot of send must stay untouched"
            continue
        if exact:
            assert np.array_equal(got[c], send_ref[c])
        else:
            scale = np.abs(send_ref[c]).max()
            assert np.abs(got[c] - send_ref[c]).max() <= TOL_SEND * scale


@pytest.mark.parametrize("tile", ["128x128", "256x128", "256x256", "256x256w8", "256x256w8s4",
                                  "256x192w8"])
def test_rs_ragged_random(tile):
    c = ctx()
    c.set_option(B.RAG_OPT_TILE, B.TILES[tile])
    shape = W.rs_shape(4, 1, 4 * 200, 192, 300, seed=3)
    say(f"case {shape.name} tile={tile}")
    inp = W.make_rs(shape)
    run = RSRun(inp).run(c)
    D_ref, send_ref, _ = oracle_rs(inp)
    assert rel_err(W.bits_u16(run.D.cpu()), D_ref) <= TOL_BF16
    _check_send(run, send_ref)


@pytest.mark.parametrize("tp,s", [(1, 0), (2, 0), (2, 1), (4, 3), (8, 5)])
def test_rs_exact_integers(tp, s):
    c = ctx()
    shape = W.rs_shape(tp, s, tp * 72, 128, 136, dist="int3", seed=tp * 10 + s)
    say(f"case {shape.name}")
    inp = W.make_rs(shape)
    run = RSRun(inp).run(c)
    D_ref, send_ref, _ = oracle_rs(inp)
    assert np.array_equal(W.bits_u16(run.D.cpu()), O.f32_to_bf16(D_ref))
    _check_send(run, send_ref, exact=True)


@pytest.mark.parametrize("kl", [64, 128, 192])
@pytest.mark.parametrize("tile", ["128x128", "256x128", "256x256", "256x256w8", "256x256w8s4",
                                  "256x192w8"])
def test_rs_short_k_every_tile(tile, kl):
    """Local K of one, two and three 128-byte k-steps (the K loop's first stage alone, one
    handover, the drained DMA past the last stage), exact integers, every tile."""
    c = ctx()
    c.set_option(B.RAG_OPT_TILE, B.TILES[tile])
    shape = W.rs_shape(4, 2, 4 * 72, kl, 136, dist="int3", seed=kl + 5)
    say(f"case {shape.name} tile={tile}")
    inp = W.make_rs(shape)
    run = RSRun(inp).run(c)
    D_ref, send_ref, _ = oracle_rs(inp)
    assert np.array_equal(W.bits_u16(run.D.cpu()), O.f32_to_bf16(D_ref))
    _check_send(run, send_ref, exact=True)


@pytest.mark.parametrize("tile", ["128x128", "256x128", "256x256", "256x256w8", "256x256w8s4",
                                  "256x192w8"])
def test_rs_padded_row_stride(tile):
    """Partials and incoming sums with a row stride past Mo (views of NaN-padded buffers): the
    padding must never reach D or send, in both the one-shot and the ring step forms, on ragged
    sizes (nc and Mo not multiples of the tile, Mo not a multiple of 32)."""
    c = ctx()
    c.set_option(B.RAG_OPT_TILE, B.TILES[tile])
    shape = W.rs_shape(4, 2, 4 * 136, 128, 212, dist="int3", seed=77)
    pad = 44
    say(f"case rs padded stride {shape.name} tile={tile}")

    def padded(t):
        buf = torch.full((t.shape[0], t.shape[1] + pad), float("nan"), device=DEV)
        buf[:, :t.shape[1]] = t.to(DEV)
        return buf[:, :t.shape[1]]

    inp = W.make_rs(shape)
    run = RSRun(inp)
    run.partials = [None if p is None else padded(p) for p in inp.partials]
    run.run(c)
    D_ref, send_ref, _ = oracle_rs(inp)
    assert np.array_equal(W.bits_u16(run.D.cpu()), O.f32_to_bf16(D_ref))
    _check_send(run, send_ref, exact=True)

    rin = W.make_rs_ring(shape)
    D = torch.empty((shape.nc, shape.Mo), dtype=torch.bfloat16, device=DEV)
    send = torch.full((shape.tp, shape.nc, shape.Mo), float("nan"), device=DEV)
    inc = [padded(t) for t in rin.incoming]
    B.gemm_rs_ring(c, rin.X.to(DEV), rin.W.to(DEV), inc, shape.tp, shape.self_rank, D, send=send)
    torch.cuda.synchronize()
    D_ref, send_ref, _ = oracle_ring(rin)
    assert np.array_equal(W.bits_u16(D.cpu()), O.f32_to_bf16(D_ref))
    got = send.cpu().numpy()
    for cix in range(shape.tp):
        if cix == shape.self_rank:
            assert np.isnan(got[cix]).all()
        else:
            assert np.array_equal(got[cix], send_ref[cix])


# Shapes with several persistent rounds: the one-shot form deals the own chunk's tiles over all
# rounds, in groups of eight workgroups (one per XCD) when the grid, the round and the round's
# share of the own chunk allow it, else over the whole grid.  (4, 2, 1100 rows, 3600 columns):
# 75 tiles per chunk at 256x256 (rounds of 256 and 44 tiles: grouped, then whole-grid), 261 at
# 128x128 (512, 512, 20).  (8, 3, 512 rows, 8192 columns): 64 tiles per chunk, two full rounds.
_MANY_ROUNDS = {}


def _many_rounds_case(tp, s, nc, mo):
    """Inputs and oracle results of one shape, computed once for all its tile / send cases."""
    key = (tp, s, nc, mo)
    if key not in _MANY_ROUNDS:
        inp = W.make_rs(W.rs_shape(tp, s, tp * nc, 128, mo, dist="int3", seed=tp * 100 + nc))
        _MANY_ROUNDS[key] = (inp, oracle_rs(inp))
    return _MANY_ROUNDS[key]


@pytest.mark.parametrize("with_send", [True, False])
@pytest.mark.parametrize("tile", ["256x256w8", "128x128"])
@pytest.mark.parametrize("tp,s,nc,mo", [(4, 2, 1100, 3600), (8, 3, 512, 8192)])
def test_rs_many_rounds_exact(tp, s, nc, mo, tile, with_send):
    c = ctx()
    c.set_option(B.RAG_OPT_TILE, B.TILES[tile])
    inp, (D_ref, send_ref, _) = _many_rounds_case(tp, s, nc, mo)
    say(f"case {inp.shape.name} tile {tile} send {with_send}")
    run = RSRun(inp, with_send=with_send).run(c)
    assert np.array_equal(W.bits_u16(run.D.cpu()), O.f32_to_bf16(D_ref))
    if with_send:
        _check_send(run, send_ref, exact=True)


def test_rs_special_cases_and_no_send():
    c = ctx()
    shape = W.rs_shape(4, 2, 4 * 64, 128, 192, dist="int3", seed=41)
    inp = W.make_rs(shape)
    # X = 0: pure reduction of the peers' chunk
    inp.X.zero_()
    say("case X=0")
    run = RSRun(inp, with_send=False).run(c)
    D_ref, _, _ = oracle_rs(inp)
    assert np.array_equal(W.bits_u16(run.D.cpu()), O.f32_to_bf16(D_ref))
    # zero partials: the GEMM's own chunk
    inp = W.make_rs(shape)
    for p in inp.partials:
        if p is not None:
            p.zero_()
    say("case zero partials")
    run = RSRun(inp).run(c)
    D_ref, send_ref, P = oracle_rs(inp)
    assert np.array_equal(W.bits_u16(run.D.cpu()), O.f32_to_bf16(P[2 * 64:3 * 64]))
    _check_send(run, send_ref, exact=True)


def _rs_8k_reference(inp):
    """Full oracle of the one-shot GEMM+RS at rs_8k, (D fp32, send [tp, nc, Mo]), computed once
    per session."""
    return cached(("rs_8k", "one-shot"), lambda: oracle_rs(inp)[:2])


def _check_full(D_dev, send_dev, D_ref, send_ref, self_rank, what):
    err = rel_err(W.bits_u16(D_dev.cpu()), D_ref)
    say(f"{what} D: all {D_ref.shape[0]} x {D_ref.shape[1]} outputs, max rel err {err:.3e}")
    assert err <= TOL_BF16
    if send_dev is None:
        return
    got = send_dev.cpu().numpy()
    for c in range(got.shape[0]):
        if c == self_rank:
            continue
        e = np.abs(got[c] - send_ref[c]).max() / np.abs(send_ref[c]).max()
        assert e <= TOL_SEND, (what, c, e)


def test_rs_full_size_full_output():
    """The measured GEMM+RS workload at full size (peer partial rows outside this rank's chunk are
    NaN, so reading them fails): every element of D and of every outgoing chunk against the full
    oracle."""
    shape = W.WORKLOADS["rs_8k"]
    say(f"case {shape}")
    inp = W.make_rs(shape)
    run = RSRun(inp).run(ctx())
    ctx().check()
    assert np.isnan(run.send[shape.self_rank].cpu().numpy()).all()
    D_ref, send_ref = _rs_8k_reference(inp)
    _check_full(run.D, run.send, D_ref, send_ref, shape.self_rank, "rs_8k")


# ------------------------------------------------- arrivals (counter-gated) and the ring step

COPY_ENGINES = ["kernel", "sdma", "in-gemm"]


def _engine(c, e):
    c.set_option(B.RAG_OPT_COPY_ENGINE, B.ENGINES[e])


@pytest.mark.parametrize("engine", COPY_ENGINES)
@pytest.mark.parametrize("tp,s", [(1, 0), (2, 1), (4, 3), (8, 5)])
def test_rs_arrive_exact_integers(tp, s, engine):
    """RAG_RS_ARRIVE: the peers' partials of the own chunk are copied in during the call and the
    own chunk's tiles wait for their counters; same result, bit for bit."""
    c = ctx()
    _engine(c, engine)
    shape = W.rs_shape(tp, s, tp * 72, 128, 136, dist="int3", seed=tp * 10 + s + 300)
    say(f"case rs arrive {shape.name} engine={engine}")
    inp = W.make_rs(shape)
    run = RSRun(inp)
    B.gemm_rs(c, run.X, run.W, run.partials, tp, s, run.D, send=run.send, flags=B.RAG_RS_ARRIVE)
    c.check()
    D_ref, send_ref, _ = oracle_rs(inp)
    assert np.array_equal(W.bits_u16(run.D.cpu()), O.f32_to_bf16(D_ref))
    _check_send(run, send_ref, exact=True)


@pytest.mark.parametrize("engine", ["kernel", "in-gemm"])
def test_rs_arrive_fresh_data_delayed(engine):
    """Back-to-back gated calls with new partials each time and every copy's counter held back
    1 ms: an epilogue that read the receive buffer before its counter would add the previous
    call's partials."""
    c = ctx()
    _engine(c, engine)
    c.set_option(B.RAG_OPT_ARRIVAL_DELAY_US, 1000)
    shape = W.rs_shape(4, 1, 4 * 64, 128, 128, dist="int3", seed=1)
    run = RSRun(W.make_rs(shape))
    for it in range(6):
        inp = W.make_rs(W.rs_shape(4, 1, 4 * 64, 128, 128, dist="int3", seed=600 + it))
        run.X.copy_(inp.X)
        run.W.copy_(inp.W)
        for d, h in zip(run.partials, inp.partials):
            if d is not None:
                d.copy_(h)
        say(f"case rs arrive fresh engine={engine} it={it}")
        B.gemm_rs(c, run.X, run.W, run.partials, 4, 1, run.D, send=run.send,
                  flags=B.RAG_RS_ARRIVE)
        torch.cuda.synchronize()
        D_ref, _, _ = oracle_rs(inp)
        assert np.array_equal(W.bits_u16(run.D.cpu()), O.f32_to_bf16(D_ref)), it
    c.check()


@pytest.mark.parametrize("engine", ["kernel", "in-gemm"])
def test_rs_arrive_withheld_times_out_and_recovers(engine):
    c = ctx()
    _engine(c, engine)
    c.set_option(B.RAG_OPT_SPIN_LIMIT_US, 20000)
    c.set_option(B.RAG_OPT_WITHHOLD_MASK, 1 << 2)
    shape = W.rs_shape(4, 0, 4 * 64, 128, 128, dist="int3", seed=5)
    inp = W.make_rs(shape)
    run = RSRun(inp)
    say("case rs arrive withheld")
    B.gemm_rs(c, run.X, run.W, run.partials, 4, 0, run.D, send=run.send, flags=B.RAG_RS_ARRIVE)
    with pytest.raises(B.RagError) as ei:
        c.check()
    assert ei.value.code == B.RAG_ETIMEOUT
    c.set_option(B.RAG_OPT_WITHHOLD_MASK, 0)
    c.set_option(B.RAG_OPT_SPIN_LIMIT_US, 2_000_000)
    B.gemm_rs(c, run.X, run.W, run.partials, 4, 0, run.D, send=run.send, flags=B.RAG_RS_ARRIVE)
    c.check()
    D_ref, _, _ = oracle_rs(inp)
    assert np.array_equal(W.bits_u16(run.D.cpu()), O.f32_to_bf16(D_ref))


class RSRingRun:
    def __init__(self, inp: W.RSRingInputs, with_send=True, poison_start=True):
        s = inp.shape
        self.inp = inp
        self.X = inp.X.to(DEV)
        self.W = inp.W.to(DEV)
        self.incoming = [t.to(DEV) for t in inp.incoming]
        self.start = O.rs_ring_order(s.self_rank, s.tp)[0]
        if poison_start:
            # the chain of this chunk starts here: its entry must not be read
            self.incoming[self.start] = torch.full_like(self.incoming[self.start], float("nan"))
        self.D = torch.empty((s.nc, s.Mo), dtype=torch.bfloat16, device=DEV)
        self.send = torch.full((s.tp, s.nc, s.Mo), float("nan"), device=DEV) if with_send else None

    def run(self, c, flags=0):
        s = self.inp.shape
        B.gemm_rs_ring(c, self.X, self.W, self.incoming, s.tp, s.self_rank, self.D,
                       send=self.send, flags=flags)
        torch.cuda.synchronize()
        return self


def oracle_ring(inp: W.RSRingInputs):
    s = inp.shape
    return O.gemm_rs_ring_step(W.bits_u16(inp.X), W.bits_u16(inp.W),
                               [t.numpy() for t in inp.incoming], s.tp, s.self_rank)


@pytest.mark.parametrize("mode", ["given", "kernel", "sdma", "in-gemm"])
@pytest.mark.parametrize("tp,s", [(1, 0), (2, 0), (3, 1), (4, 2), (8, 5)])
def test_rs_ring_step_exact_integers(tp, s, mode):
    """One ring step: send[c] = incoming[c] + P[c], D = incoming[s] + P[s], bit for bit on
    integer data; the chain-start entry is NaN and must not be read; the own slot of send stays
    untouched."""
    c = ctx()
    flags = 0
    if mode != "given":
        _engine(c, mode)
        flags = B.RAG_RS_ARRIVE
    shape = W.rs_shape(tp, s, tp * 72, 128, 136, dist="int3", seed=tp * 10 + s + 700)
    say(f"case rs ring {shape.name} mode={mode}")
    inp = W.make_rs_ring(shape)
    run = RSRingRun(inp).run(c, flags)
    c.check()
    D_ref, send_ref, _ = oracle_ring(inp)
    assert np.array_equal(W.bits_u16(run.D.cpu()), O.f32_to_bf16(D_ref))
    _check_send(run, send_ref, exact=True)


@pytest.mark.parametrize("tile", ["128x128", "256x128", "256x256w8"])
def test_rs_ring_ragged_random(tile):
    c = ctx()
    c.set_option(B.RAG_OPT_TILE, B.TILES[tile])
    _engine(c, "kernel")
    shape = W.rs_shape(4, 1, 4 * 200, 192, 300, seed=13)
    say(f"case rs ring ragged tile={tile}")
    inp = W.make_rs_ring(shape)
    run = RSRingRun(inp).run(c, B.RAG_RS_ARRIVE)
    c.check()
    D_ref, send_ref, _ = oracle_ring(inp)
    assert rel_err(W.bits_u16(run.D.cpu()), D_ref) <= TOL_BF16
    _check_send(run, send_ref)


@pytest.mark.parametrize("engine", ["kernel", "in-gemm"])
def test_rs_ring_no_send_and_delayed_arrivals(engine):
    """send = NULL (the passed-on sums are dropped, so only the own chunk waits on the device and
    the call joins the side stream, or the GEMM's workgroups copy what is left before they exit)
    with every copy held back 1 ms, then fresh data."""
    c = ctx()
    _engine(c, engine)
    c.set_option(B.RAG_OPT_ARRIVAL_DELAY_US, 1000)
    for it in range(3):
        shape = W.rs_shape(4, 3, 4 * 64, 128, 128, dist="int3", seed=800 + it)
        inp = W.make_rs_ring(shape)
        say(f"case rs ring no-send it={it}")
        run = RSRingRun(inp, with_send=False).run(c, B.RAG_RS_ARRIVE)
        D_ref, _, _ = oracle_ring(inp)
        assert np.array_equal(W.bits_u16(run.D.cpu()), O.f32_to_bf16(D_ref)), it
    c.check()


def _rs_8k_ring_reference(inp):
    """Full oracle of one ring-accumulate step at rs_8k, (D fp32, out [tp, nc, Mo]), computed
    once per session."""
    return cached(("rs_8k", "ring"), lambda: oracle_ring(inp)[:2])


@pytest.mark.parametrize("engine", ["kernel", "in-gemm"])
def test_rs_ring_full_size_full_output(engine):
    """The ring step at the measured GEMM+RS size with arrivals: every element of D and of every
    passed-on sum against the full oracle."""
    shape = W.WORKLOADS["rs_8k"]
    c = ctx()
    _engine(c, engine)
    say(f"case rs ring full {shape} engine={engine}")
    inp = W.make_rs_ring(shape)
    run = RSRingRun(inp).run(c, B.RAG_RS_ARRIVE)
    c.check()
    D_ref, out_ref = _rs_8k_ring_reference(inp)
    _check_full(run.D, run.send, D_ref, out_ref, shape.self_rank, "rs ring")


@pytest.mark.parametrize("engine", ["kernel", "in-gemm", "sdma"])
@pytest.mark.parametrize("ring", [False, True])
def test_rs_arrive_full_size_back_to_back(ring, engine):
    """Full-size gated calls back to back (no synchronisation between them).  With the copy kernel
    beside the GEMM, the GEMM's persistent grid must leave the copies room to run, or its waiting
    tiles would spin to the limit (RAG_ETIMEOUT); with the GEMM's own workgroups copying, every
    piece must be taken by some workgroup.  Then the last call's D and send are checked in full."""
    shape = W.WORKLOADS["rs_8k"]
    c = ctx()
    _engine(c, engine)
    c.set_option(B.RAG_OPT_COMM_WGS, 128)
    say(f"case rs arrive back-to-back ring={ring} engine={engine} {shape}")
    if ring:
        inp = W.make_rs_ring(shape)
        run = RSRingRun(inp, poison_start=False)
        for _ in range(4):
            B.gemm_rs_ring(c, run.X, run.W, run.incoming, shape.tp, shape.self_rank, run.D,
                           send=run.send, flags=B.RAG_RS_ARRIVE)
    else:
        inp = W.make_rs(shape)
        run = RSRun(inp)
        for _ in range(4):
            B.gemm_rs(c, run.X, run.W, run.partials, shape.tp, shape.self_rank, run.D,
                      send=run.send, flags=B.RAG_RS_ARRIVE)
    torch.cuda.synchronize()
    c.check()
    if ring:
        D_ref, send_ref = _rs_8k_ring_reference(inp)
    else:
        D_ref, send_ref = _rs_8k_reference(inp)
    _check_full(run.D, run.send, D_ref, send_ref, shape.self_rank, f"back-to-back ring={ring}")


# ------------------------------------------------------- row-parallel linear with all-reduce

@pytest.mark.parametrize("engine", COPY_ENGINES)
@pytest.mark.parametrize("tp,s", [(1, 0), (2, 1), (4, 2), (8, 7)])
def test_linear_allreduce_exact(tp, s, engine):
    """Y's own chunk is the reduce-scatter's sum (bit for bit on integers), every other chunk is
    the owner's reduced chunk as given, bit for bit; send as for gemm_rs."""
    c = ctx()
    _engine(c, engine)
    shape = W.rs_shape(tp, s, tp * 64, 128, 136, dist="int3", seed=900 + tp * 10 + s)
    say(f"case linear_allreduce {shape.name} engine={engine}")
    inp = W.make_rs(shape)
    red = W.make_reduced_chunks(shape)
    run = RSRun(inp)
    red_dev = [t.to(DEV) for t in red]
    Y = torch.full((shape.T, shape.Mo), float("nan"), dtype=torch.bfloat16, device=DEV)
    B.linear_allreduce(c, run.X, run.W, run.partials, red_dev, tp, s, Y, send=run.send)
    torch.cuda.synchronize()
    c.check()
    peers = [None if p is None else p.numpy() for p in inp.partials]
    Y_ref, send_ref = O.linear_allreduce_step(W.bits_u16(inp.X), W.bits_u16(inp.W), peers,
                                              [W.bits_u16(t) for t in red], tp, s)
    got = W.bits_u16(Y.cpu())
    nc = shape.nc
    for cix in range(tp):
        rows = slice(cix * nc, (cix + 1) * nc)
        if cix == s:
            assert np.array_equal(got[rows], O.f32_to_bf16(Y_ref[rows]))
        else:
            assert np.array_equal(got[rows], W.bits_u16(red[cix]))
    _check_send(run, send_ref, exact=True)


def _check_y(Y, D_ref, red, shape, what):
    """Y's own chunk against the reduce-scatter's oracle, every other chunk bit for bit against
    the owner's reduced chunk."""
    got = W.bits_u16(Y.cpu())
    nc, s = shape.nc, shape.self_rank
    for cix in range(shape.tp):
        rows = slice(cix * nc, (cix + 1) * nc)
        if cix == s:
            err = rel_err(got[rows], D_ref)
            say(f"{what}: own chunk max rel err {err:.3e}")
            assert err <= TOL_BF16
        else:
            assert np.array_equal(got[rows], W.bits_u16(red[cix])), (what, cix)


@pytest.mark.parametrize("engine", ["in-gemm", "kernel"])
def test_linear_allreduce_full_size(engine):
    """rs_8k shape: with the GEMM's own workgroups gathering the reduced chunks, each chunk is 16
    pieces and the launch runs several rounds, so the piece sizing, the per-tile quota and the
    final drain all run; every non-own chunk of Y is compared bit for bit, the own chunk and send
    with the full oracle."""
    shape = W.WORKLOADS["rs_8k"]
    c = ctx()
    _engine(c, engine)
    say(f"case linear_allreduce full {shape} engine={engine}")
    inp = W.make_rs(shape)
    red = W.make_reduced_chunks(shape)
    run = RSRun(inp)
    red_dev = [t.to(DEV) for t in red]
    Y = torch.full((shape.T, shape.Mo), float("nan"), dtype=torch.bfloat16, device=DEV)
    B.linear_allreduce(c, run.X, run.W, run.partials, red_dev, shape.tp, shape.self_rank, Y,
                       send=run.send)
    torch.cuda.synchronize()
    c.check()
    D_ref, send_ref = _rs_8k_reference(inp)
    _check_y(Y, D_ref, red, shape, f"linear_allreduce {engine}")
    _check_full(Y[shape.self_rank * shape.nc:(shape.self_rank + 1) * shape.nc], run.send, D_ref,
                send_ref, shape.self_rank, "linear_allreduce send")


def test_side_stream_arrivals_then_in_gemm_copies_back_to_back():
    """linear_allreduce with RAG_RS_ARRIVE runs its copies in a kernel on the side stream; the
    in-GEMM calls enqueued right after it on the caller's stream (no synchronisation) clear and
    reuse the piece counts that kernel used.  Two rounds of: gated linear_allreduce at rs_8k, an
    in-GEMM ag_gemm, an in-GEMM linear_allreduce; every output is then checked."""
    shape = W.WORKLOADS["rs_8k"]
    c = ctx()
    _engine(c, "in-gemm")
    c.set_option(B.RAG_OPT_COMM_WGS, 128)
    inp = W.make_rs(shape)
    red = W.make_reduced_chunks(shape)
    run = RSRun(inp)
    red_dev = [t.to(DEV) for t in red]
    ag_shape = W.ag_shape(4, 2, 512, 1024, 768, dist="int3", seed=4242)
    ag_inp = W.make_ag(ag_shape)
    outs = []
    say("case side-stream arrivals then in-GEMM copies, back to back")
    for _ in range(2):
        Y1 = torch.full((shape.T, shape.Mo), float("nan"), dtype=torch.bfloat16, device=DEV)
        B.linear_allreduce(c, run.X, run.W, run.partials, red_dev, shape.tp, shape.self_rank, Y1,
                           send=run.send, flags=B.RAG_RS_ARRIVE)
        ag = AGRunNoSync(ag_inp)
        ag.enqueue(c)
        Y2 = torch.full((shape.T, shape.Mo), float("nan"), dtype=torch.bfloat16, device=DEV)
        B.linear_allreduce(c, run.X, run.W, run.partials, red_dev, shape.tp, shape.self_rank, Y2,
                           send=run.send)
        outs.append((Y1, ag, Y2))
    torch.cuda.synchronize()
    c.check()
    D_ref, _ = _rs_8k_reference(inp)
    _, ag_ref = O.ag_gemm(W.bits_u16(ag_inp.A), [W.bits_u16(t) for t in ag_inp.chunks])
    for i, (Y1, ag, Y2) in enumerate(outs):
        _check_y(Y1, D_ref, red, shape, f"gated linear_allreduce #{i}")
        assert np.array_equal(W.bits_u16(ag.D.cpu()), O.f32_to_bf16(ag_ref)), i
        _check_y(Y2, D_ref, red, shape, f"in-GEMM linear_allreduce #{i}")


class AGRunNoSync:
    """An AG+GEMM call enqueued without a synchronisation after it."""

    def __init__(self, inp):
        s = inp.shape
        self.inp = inp
        self.A = inp.A.to(DEV)
        self.chunks = [t.to(DEV) for t in inp.chunks]
        self.G = torch.empty((s.N, s.K), dtype=torch.bfloat16, device=DEV)
        self.D = torch.full((s.N, s.M), float("nan"), dtype=torch.bfloat16, device=DEV)

    def enqueue(self, c):
        s = self.inp.shape
        B.ag_gemm(c, self.A, self.chunks, s.tp, s.self_rank, self.D, G=self.G)
