"""GPU parity of the GEMM+RS path (libringag.so through the C ABI) against the CPU oracle."""
import numpy as np
import pytest
import torch

from oracle import ringag_oracle as O
from ring_all_gather_amd import binding as B
from ring_all_gather_amd import workloads as W

from gpu_common import DEV, TOL_BF16, TOL_SEND, ctx, rel_err, reset_options, say

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


@pytest.mark.parametrize("tile", ["128x128", "256x128", "256x256", "256x256w8", "256x256w8s4"])
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


def test_rs_full_size_sampled_rows():
    """The measured GEMM+RS workload at full size (peer partial rows outside this rank's chunk are
    NaN, so reading them fails); sampled rows of D and of every outgoing chunk vs the oracle."""
    shape = W.WORKLOADS["rs_8k"]
    say(f"case {shape}")
    inp = W.make_rs(shape)
    run = RSRun(inp).run(ctx())
    g = np.random.default_rng(shape.seed)
    rows = np.unique(np.concatenate([[0, shape.nc - 1], g.choice(shape.nc, 62, replace=False)]))
    peers = [None if p is None else p.numpy() for p in inp.partials]
    Xb, Wb = W.bits_u16(inp.X), W.bits_u16(inp.W)
    D_rows = O.gemm_rs_rows(Xb, Wb, peers, shape.tp, shape.self_rank, rows)
    err = rel_err(W.bits_u16(run.D.cpu())[rows], D_rows)
    say(f"rs_8k D: {len(rows)} sampled rows, max rel err {err:.3e}")
    assert err <= TOL_BF16
    send = run.send.cpu().numpy()
    Xf, Wf = O.bf16_to_f32(Xb), O.bf16_to_f32(Wb)
    for cix in range(shape.tp):
        if cix == shape.self_rank:
            continue
        ref = O.gemm_tn_rows(Xf, Wf, cix * shape.nc + rows[:8])
        got = send[cix][rows[:8]]
        assert np.abs(got - ref).max() <= TOL_SEND * np.abs(ref).max()
