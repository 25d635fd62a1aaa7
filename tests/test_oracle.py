"""Pins of the CPU oracle against things other than itself (CPU only).

Each check below ties the oracle to an independent fact: exact integer products (numpy int64
matmul), float64 brute force within the fp32 error bound, hand-worked fixtures under
tests/golden/, torch's own number-format conversions, and the invariants the pages fix (chunked ==
unchunked, chunk r lands at offset r*n/tp, a reduce-scatter chunk is the sum of the ranks'
partials).  The last test plants plausible mistakes in copies of the oracle's functions and checks
that the pins catch every one.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import ringag_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16_bits(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def _exact_gemm(G_int, A_int):
    return (G_int.astype(np.int64) @ A_int.astype(np.int64).T)


def _fp32_bound(G, A):
    """|fl(sum) - sum| <= gamma_K * sum_k |g_k a_k|, gamma_K = K u / (1 - K u), u = 2^-24 (standard
    bound for recursive summation of exactly-formed products; products of fp32 operands are
    rounded once more, which the K+1 below accounts for)."""
    K = G.shape[1]
    u = 2.0 ** -24
    gamma = (K + 1) * u / (1 - (K + 1) * u)
    return gamma * (np.abs(G.astype(np.float64)) @ np.abs(A.astype(np.float64)).T)


# ------------------------------------------------------------------------------------ formats

def test_bf16_widen_closed_forms():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x0001, 0x7F7F, 0x3E80],
                    dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, np.inf, -np.inf, 2.0 ** -133, 3.3895313892515355e38, 0.25]
    got = O.bf16_to_f32(bits)
    for g, w in zip(got, want):
        assert g == np.float32(w)
    assert np.signbit(got[3])


def test_bf16_widen_matches_torch_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = O.bf16_to_f32(codes)
    ref = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_rne_ties_and_specials():
    one = np.float32(1.0)
    half_ulp = np.float32(2.0 ** -8)       # bf16 ulp at 1.0 is 2^-7
    vals = np.array([one + half_ulp,                     # tie -> even (1.0)
                     one + 3 * half_ulp,                 # tie -> even (1 + 2^-6)
                     one + half_ulp + np.float32(2.0 ** -20),  # above the tie -> up
                     np.float32(3.4e38),                 # above max bf16 + half ulp -> inf
                     np.float32(np.nan), np.float32(-np.inf), np.float32(-0.0)],
                    dtype=np.float32)
    got = O.f32_to_bf16(vals)
    assert got[0] == 0x3F80
    assert got[1] == 0x3F82
    assert got[2] == 0x3F81
    assert got[3] == 0x7F80
    assert (got[4] & 0x7F80) == 0x7F80 and (got[4] & 0x7F) != 0
    assert got[5] == 0xFF80
    assert got[6] == 0x8000


def test_bf16_rne_matches_torch_random():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 1e3,
        rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32).view(np.float32),
        # exact ties: low 16 bits = 0x8000
        ((rng.integers(0, 2 ** 16, 20000, dtype=np.uint32) << 16) | 0x8000).astype(
            np.uint32).view(np.float32),
    ])
    x = x[~np.isnan(x)]
    ours = O.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_e4m3_closed_forms():
    codes = np.array([0x00, 0x38, 0x7E, 0x01, 0x08, 0x40, 0xB8, 0x7F, 0xFF, 0x80], dtype=np.uint8)
    got = O.e4m3fn_to_f32(codes)
    assert got[0] == 0.0
    assert got[1] == 1.0                  # exponent field 7 = bias
    assert got[2] == 448.0                # largest finite value
    assert got[3] == 2.0 ** -9            # smallest subnormal: 1/8 * 2^-6
    assert got[4] == 2.0 ** -6            # smallest normal
    assert got[5] == 2.0                  # exponent 8, mantissa 0
    assert got[6] == -1.0
    assert np.isnan(got[7]) and np.isnan(got[8])
    assert got[9] == 0.0 and np.signbit(got[9])


def test_e4m3_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3fn_to_f32(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


# ------------------------------------------------------------------------------------ GEMM

@pytest.mark.parametrize("N,M,K", [(5, 7, 9), (1, 1, 1), (33, 17, 64), (64, 48, 300)])
def test_gemm_exact_integers(N, M, K):
    rng = np.random.default_rng(N * 1000 + M * 10 + K)
    G = rng.integers(-3, 4, (N, K))
    A = rng.integers(-3, 4, (M, K))
    got = O.gemm_tn(G.astype(np.float32), A.astype(np.float32))
    assert got.shape == (N, M)
    assert np.array_equal(got.astype(np.int64), _exact_gemm(G, A))


@pytest.mark.parametrize("N,M,K", [(16, 24, 1000), (3, 5, 4096)])
def test_gemm_within_fp32_bound_of_float64(N, M, K):
    rng = np.random.default_rng(K)
    G = rng.standard_normal((N, K)).astype(np.float32)
    A = rng.standard_normal((M, K)).astype(np.float32)
    exact = G.astype(np.float64) @ A.astype(np.float64).T
    err = np.abs(O.gemm_tn(G, A).astype(np.float64) - exact)
    assert np.all(err <= _fp32_bound(G, A))


def test_gemm_rows_matches_full():
    rng = np.random.default_rng(5)
    G = rng.standard_normal((40, 70)).astype(np.float32)
    A = rng.standard_normal((30, 70)).astype(np.float32)
    rows = [0, 39, 7, 7, 21]
    full = O.gemm_tn(G, A)
    assert np.array_equal(O.gemm_tn_rows(G, A, rows), full[rows])
    with pytest.raises(IndexError):
        O.gemm_tn_rows(G, A, [40])


def test_gemm_zero_k():
    out = O.gemm_tn(np.zeros((3, 0), np.float32), np.zeros((2, 0), np.float32))
    assert np.array_equal(out, np.zeros((3, 2), np.float32))


# ------------------------------------------------------------------------------------ ring / AG

def test_ring_orders_fixture():
    for case in _golden("ring_orders.json")["cases"]:
        assert O.ring_order(case["tp"], case["self_rank"]) == case["order"]


@pytest.mark.parametrize("tp", [1, 2, 3, 4, 5, 8])
def test_ring_exchange_delivers_every_chunk_once(tp):
    held = O.ring_exchange(tp)
    for r in range(tp):
        assert held[r][0] == r
        assert sorted(held[r]) == list(range(tp))


def test_ag_gemm_hand_fixture():
    fx = _golden("ag_tp3_hand.json")
    chunks = [_bf16_bits(c) for c in fx["chunks"]]
    G, D = O.ag_gemm(_bf16_bits(fx["A"]), chunks)
    assert np.array_equal(O.bf16_to_f32(G), np.array(sum(fx["chunks"], []), np.float32))
    assert np.array_equal(D, np.array(fx["D"], np.float32))


@pytest.mark.parametrize("tp", [1, 2, 3, 4, 8])
def test_chunked_ring_equals_unchunked_for_every_self_rank(tp):
    rng = np.random.default_rng(tp)
    nc, K, M = 3, 37, 11
    chunks = [rng.standard_normal((nc, K)).astype(np.float32) for _ in range(tp)]
    A = rng.standard_normal((M, K)).astype(np.float32)
    full = O.gemm_tn(O.gather(chunks), A)
    for s in range(tp):
        assert np.array_equal(O.ag_gemm_ring(A, chunks, s), full)


def test_chunk_lands_at_rank_offset():
    rng = np.random.default_rng(9)
    tp, nc, K, M = 4, 5, 16, 6
    chunks = [rng.integers(-3, 4, (nc, K)).astype(np.float32) for _ in range(tp)]
    A = rng.integers(-3, 4, (M, K)).astype(np.float32)
    base = O.gemm_tn(O.gather(chunks), A)
    for r in range(tp):
        pert = [c.copy() for c in chunks]
        pert[r] += 1.0
        G = O.gather(pert)
        assert np.array_equal(G[r * nc:(r + 1) * nc], pert[r])
        D = O.gemm_tn(G, A)
        changed = np.any(D != base, axis=1)
        assert not changed[:r * nc].any() and not changed[(r + 1) * nc:].any()
        assert changed[r * nc:(r + 1) * nc].any()


@pytest.mark.parametrize("tp", [2, 3, 4, 8])
def test_staged_output_readings(tp):
    """The listing's literal (tp+1)-chunk placement (slot 0 -> slot tp, D = slots 1..tp) yields
    rank order only when the chunks were consumed in the order [tp-1, 0, 1, ..., tp-2]; placing
    slot j at its origin rank's offset yields rank order for every self rank."""
    nc, M = 2, 3
    outs = {r: np.full((nc, M), float(r), np.float32) for r in range(tp)}
    rank_ordered = np.concatenate([outs[r] for r in range(tp)])
    for s in range(tp):
        order = O.ring_order(tp, s)
        slots = [outs[r] for r in order]
        assert np.array_equal(O.staged_output_by_rank(slots, order), rank_ordered)
        rot = O.staged_output_rotation(slots)
        assert np.array_equal(rot, rank_ordered) == (order == [tp - 1] + list(range(tp - 1)))
    # the ascending ring (send to rank-1) consumes [s, s+1, ...]; its last rank is the one case
    asc = [(tp - 1 + j) % tp for j in range(tp)]
    assert np.array_equal(O.staged_output_rotation([outs[r] for r in asc]), rank_ordered)


def test_fp8_gemm_exact_integers_and_scales():
    rng = np.random.default_rng(12)
    tp, nc, K, M = 2, 4, 32, 8
    ints_b = [rng.integers(-3, 4, (nc, K)) for _ in range(tp)]
    ints_a = rng.integers(-3, 4, (M, K))
    q = lambda x: torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()
    sa, sb = 0.5, 0.25
    G, D = O.ag_gemm_fp8(q(ints_a), sa, [q(b) for b in ints_b], sb)
    exact = _exact_gemm(np.concatenate(ints_b), ints_a) * (sa * sb)
    assert np.array_equal(D.astype(np.float64), exact)


def test_fp8_gemm_random_within_bound():
    rng = np.random.default_rng(13)
    x = torch.from_numpy(rng.standard_normal((64, 512)).astype(np.float32))
    codes = x.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    a_codes, b_codes = codes[:16], codes[16:]
    s_a, s_b = 0.03125, 0.0078125
    _, D = O.ag_gemm_fp8(a_codes, s_a, [b_codes[:24], b_codes[24:]], s_b)
    deq = lambda c, s: torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).double().numpy() * s
    Ga, Aa = deq(b_codes, s_b), deq(a_codes, s_a)
    exact = Ga @ Aa.T
    assert np.all(np.abs(D - exact) <= _fp32_bound(Ga.astype(np.float32), Aa.astype(np.float32)))


def _int_ag_inputs(rng, tp, nc, K, M):
    chunks = [rng.integers(-3, 4, (nc, K)) for _ in range(tp)]
    A = rng.integers(-3, 4, (M, K))
    return chunks, A


def _rows_pin_pass(rows_fn):
    """rows_fn(A_bits, chunk_bits, rows) against the exact int64 product of the explicitly
    concatenated chunks, on integer inputs (exact in bf16 and in fp32), at rows that span every
    chunk, repeat, and come out of order."""
    rng = np.random.default_rng(31)
    tp, nc, K, M = 3, 5, 48, 7
    chunks, A = _int_ag_inputs(rng, tp, nc, K, M)
    exact = _exact_gemm(np.concatenate(chunks), A)
    rows = [14, 0, 5, 4, 9, 10, 5, 13]
    try:
        got = rows_fn(_bf16_bits(A), [_bf16_bits(c) for c in chunks], rows)
        return got.shape == (len(rows), M) and np.array_equal(got.astype(np.int64), exact[rows])
    except Exception:
        return False


def test_ag_rows_exact_integers():
    assert _rows_pin_pass(O.ag_gemm_rows)


def test_ag_rows_match_full_random():
    """The sampled-row form used at full size is bit-identical to rows of the full AG+GEMM (same
    loop, same order), for random bf16 data and every chunk."""
    rng = np.random.default_rng(32)
    tp, nc, K, M = 4, 6, 96, 9
    chunks = [_bf16_bits(rng.standard_normal((nc, K))) for _ in range(tp)]
    A = _bf16_bits(rng.standard_normal((M, K)))
    rows = [23, 0, 6, 5, 11, 12, 17, 18, 1]
    _, full = O.ag_gemm(A, chunks)
    assert np.array_equal(O.ag_gemm_rows(A, chunks, rows), full[rows])
    with pytest.raises(IndexError):
        O.ag_gemm_rows(A, chunks, [tp * nc])


def test_ag_fp8_rows_exact_integers_and_match_full():
    rng = np.random.default_rng(33)
    tp, nc, K, M = 3, 4, 128, 6
    chunks, A = _int_ag_inputs(rng, tp, nc, K, M)
    q = lambda x: torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()
    sa, sb = 0.5, 0.125
    rows = [11, 0, 4, 3, 8, 4]
    got = O.ag_gemm_fp8_rows(q(A), sa, [q(c) for c in chunks], sb, rows)
    exact = _exact_gemm(np.concatenate(chunks), A)[rows] * (sa * sb)
    assert np.array_equal(got.astype(np.float64), exact)
    # random codes: bit-identical to rows of the full fp8 AG+GEMM
    x = torch.from_numpy(rng.standard_normal((M + tp * nc, K)).astype(np.float32))
    codes = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    a_codes, b = codes[:M], [codes[M + r * nc:M + (r + 1) * nc] for r in range(tp)]
    _, full = O.ag_gemm_fp8(a_codes, 0.03125, b, 0.0078125)
    assert np.array_equal(O.ag_gemm_fp8_rows(a_codes, 0.03125, b, 0.0078125, rows), full[rows])


def test_rows_pin_catches_planted_row_mistakes():
    """Plausible mistakes in a sampled-row helper, planted in copies on the CPU: a row index taken
    within its chunk instead of within the gathered N, off by one, or read from the chunks in
    arrival order instead of rank order."""
    nc = 5

    def within_chunk(A, ch, rows):
        return O.ag_gemm_rows(A, ch, [r % nc for r in rows])

    def off_by_one(A, ch, rows):
        return O.ag_gemm_rows(A, ch, [min(r + 1, 3 * nc - 1) for r in rows])

    def arrival_order(A, ch, rows):
        return O.ag_gemm_rows(A, [ch[r] for r in O.ring_order(len(ch), 1)], rows)

    for bad in (within_chunk, off_by_one, arrival_order):
        assert not _rows_pin_pass(bad), bad.__name__


# ------------------------------------------------------------------------------------ GEMM+RS

def test_rs_hand_fixture():
    fx = _golden("rs_tp2_hand.json")
    peer = np.array([[np.nan if v is None else v for v in row]
                     for row in fx["peer_partial_rank0"]], np.float32)
    D, send, P = O.gemm_rs(_bf16_bits(fx["X"]), _bf16_bits(fx["W"]), [peer, None], fx["tp"],
                           fx["self_rank"])
    assert np.array_equal(P, np.array(fx["P_local"], np.float32))
    assert np.array_equal(D, np.array(fx["D"], np.float32))
    assert np.array_equal(send[0], np.array(fx["send_chunk0"], np.float32))


@pytest.mark.parametrize("tp,s", [(1, 0), (2, 1), (4, 2), (8, 7)])
def test_rs_exact_integers(tp, s):
    rng = np.random.default_rng(tp * 10 + s)
    nc, Kl, Mo = 3, 20, 9
    T = tp * nc
    X = rng.integers(-3, 4, (T, Kl))
    W = rng.integers(-3, 4, (Mo, Kl))
    peers = [None if p == s else rng.integers(-50, 50, (T, Mo)).astype(np.float32)
             for p in range(tp)]
    D, send, P = O.gemm_rs(_bf16_bits(X), _bf16_bits(W), peers, tp, s)
    Pex = _exact_gemm(X, W)
    want = Pex[s * nc:(s + 1) * nc].copy()
    for p in range(tp):
        if p != s:
            want = want + peers[p][s * nc:(s + 1) * nc].astype(np.int64)
    assert np.array_equal(D.astype(np.int64), want)
    for c in range(tp):
        assert np.array_equal(send[c].astype(np.int64), Pex[c * nc:(c + 1) * nc])


def test_rs_special_cases():
    rng = np.random.default_rng(21)
    tp, s, nc, Kl, Mo = 4, 1, 4, 16, 8
    T = tp * nc
    peers = [None if p == s else rng.standard_normal((T, Mo)).astype(np.float32)
             for p in range(tp)]
    zeroX = np.zeros((T, Kl), np.float32)
    W = rng.standard_normal((Mo, Kl)).astype(np.float32)
    # X = 0: a pure reduction of the peers' chunk s, summed in increasing rank
    D, _, _ = O.gemm_rs(_bf16_bits(zeroX), _bf16_bits(W), peers, tp, s)
    want = np.zeros((nc, Mo), np.float32)
    for p in range(tp):
        if p != s:
            want = want + peers[p][s * nc:(s + 1) * nc]
    assert np.array_equal(D, want)
    # zero peers: the GEMM's own chunk
    X = rng.standard_normal((T, Kl)).astype(np.float32)
    zp = [None if p == s else np.zeros((T, Mo), np.float32) for p in range(tp)]
    D2, _, P = O.gemm_rs(_bf16_bits(X), _bf16_bits(W), zp, tp, s)
    assert np.array_equal(D2, P[s * nc:(s + 1) * nc])


def test_rs_rows_matches_full_and_ignores_poison():
    rng = np.random.default_rng(22)
    tp, s, nc, Kl, Mo = 4, 2, 6, 24, 10
    T = tp * nc
    X = _bf16_bits(rng.standard_normal((T, Kl)))
    W = _bf16_bits(rng.standard_normal((Mo, Kl)))
    peers = []
    for p in range(tp):
        if p == s:
            peers.append(None)
            continue
        part = np.full((T, Mo), np.nan, np.float32)
        part[s * nc:(s + 1) * nc] = rng.standard_normal((nc, Mo))
        peers.append(part)
    D, _, _ = O.gemm_rs(X, W, peers, tp, s)
    assert np.isfinite(D).all()
    rows = [0, 5, 3]
    assert np.array_equal(O.gemm_rs_rows(X, W, peers, tp, s, rows), D[rows])


def test_rs_ring_order_fixture():
    for case in _golden("rs_ring_orders.json")["cases"]:
        assert O.rs_ring_order(case["self_rank"], case["tp"]) == case["order"]


def _ring_incoming(P, tp, r, nc):
    """Running sums arriving at rank r in a ring reduce-scatter that sends to rank+1, from the
    plain definition: chunk c's sum at rank r is the sum of the partials of ranks c+1 .. r-1 (its
    chain so far), integers so that the order of the adds does not matter."""
    inc = []
    for c in range(tp):
        k = (r - c - 1) % tp
        if k == 0:
            inc.append(None)
            continue
        acc = np.zeros_like(P[0][:nc])
        for i in range(1, k + 1):
            q = (c + i) % tp
            acc = acc + P[q][c * nc:(c + 1) * nc]
        inc.append(acc.astype(np.float32))
    return inc


def _ring_pins_pass(step):
    rng = np.random.default_rng(91)
    for tp in (1, 2, 3, 4):
        nc, Kl, Mo = 2, 12, 5
        T = tp * nc
        Xs = [rng.integers(-3, 4, (T, Kl)) for _ in range(tp)]
        Ws = [rng.integers(-3, 4, (Mo, Kl)) for _ in range(tp)]
        P = [_exact_gemm(Xs[r], Ws[r]).astype(np.float32) for r in range(tp)]
        outs = []
        try:
            for r in range(tp):
                D, send, _ = step(_bf16_bits(Xs[r]), _bf16_bits(Ws[r]),
                                  _ring_incoming(P, tp, r, nc), tp, r)
                outs.append((D, send))
        except Exception:
            return False
        for r in range(tp):
            D, send = outs[r]
            want = sum(P[q][r * nc:(r + 1) * nc].astype(np.int64) for q in range(tp))
            if not np.array_equal(D.astype(np.int64), want):
                return False
            nxt = _ring_incoming(P, tp, (r + 1) % tp, nc)
            for c in range(tp):
                if c != r and not np.array_equal(send[c], nxt[c]):
                    return False
    return True


def test_rs_ring_simulation_equals_reduce_scatter():
    """Every rank runs one ring step on the running sums its predecessor would hand it: each
    owner's result is the sum of all ranks' partials of its chunk, and what a rank sends on is
    exactly what its successor receives."""
    assert _ring_pins_pass(O.gemm_rs_ring_step)

    def wrong_start(X, W, inc, tp, s):
        inc = list(inc)
        inc[(s - 1) % tp], inc[(s + 1) % tp] = inc[(s + 1) % tp], inc[(s - 1) % tp]
        return O.gemm_rs_ring_step(X, W, inc, tp, s)

    def dropped_incoming(X, W, inc, tp, s):
        return O.gemm_rs_ring_step(X, W, [None if i is None else 0 * i for i in inc], tp, s)

    def wrong_rows(X, W, inc, tp, s):
        D, send, P = O.gemm_rs_ring_step(X, W, inc, tp, s)
        return D, np.roll(send, 1, axis=0), P

    assert not _ring_pins_pass(wrong_start)
    assert not _ring_pins_pass(dropped_incoming)
    assert not _ring_pins_pass(wrong_rows)


def test_rs_ring_rows_matches_full():
    rng = np.random.default_rng(93)
    tp, s, nc, Kl, Mo = 4, 1, 5, 16, 7
    T = tp * nc
    X = _bf16_bits(rng.standard_normal((T, Kl)))
    W = _bf16_bits(rng.standard_normal((Mo, Kl)))
    inc = [None if c == (s - 1) % tp else rng.standard_normal((nc, Mo)).astype(np.float32)
           for c in range(tp)]
    D, send, _ = O.gemm_rs_ring_step(X, W, inc, tp, s)
    rows = [0, 4, 2]
    for c in range(tp):
        assert np.array_equal(O.gemm_rs_ring_step_rows(X, W, inc, tp, s, c, rows), send[c][rows])
    assert np.array_equal(send[s], D)


def test_linear_allreduce_equals_unsharded_linear():
    """With every rank's partial and every owner's reduced chunk consistent (integers, so exact),
    one rank's step gives the whole row-parallel linear: sum over ranks of X_r W_r^T, i.e. the
    linear on the unsharded input and weight, for every self rank."""
    rng = np.random.default_rng(97)
    for tp in (1, 2, 4):
        nc, Kl, Mo = 3, 8, 6
        T = tp * nc
        # entries in {-1, 0, 1}: every sum stays within +-32, exact in bf16 as well
        Xs = [rng.integers(-1, 2, (T, Kl)) for _ in range(tp)]
        Ws = [rng.integers(-1, 2, (Mo, Kl)) for _ in range(tp)]
        P = [_exact_gemm(Xs[r], Ws[r]) for r in range(tp)]
        # the unsharded linear: the input is [X_0 | X_1 | ...] along k, the weight likewise
        full = _exact_gemm(np.concatenate(Xs, axis=1), np.concatenate(Ws, axis=1))
        assert np.array_equal(full, sum(P))
        reduced = [_bf16_bits(full[c * nc:(c + 1) * nc]) for c in range(tp)]
        for s in range(tp):
            peers = [None if p == s else P[p].astype(np.float32) for p in range(tp)]
            Y, send = O.linear_allreduce_step(_bf16_bits(Xs[s]), _bf16_bits(Ws[s]), peers,
                                              reduced, tp, s)
            assert np.array_equal(Y.astype(np.int64), full)
            for c in range(tp):
                if c != s:
                    assert np.array_equal(send[c].astype(np.int64), P[s][c * nc:(c + 1) * nc])


def _torch_e4m3_codes(x):
    t = torch.tensor(np.clip(np.asarray(x, np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch():
    """The encoder against torch's own fp32 -> float8_e4m3fn cast (after the same clamp), over
    normal, subnormal and saturating values."""
    rng = np.random.default_rng(101)
    x = np.concatenate([rng.uniform(-500, 500, 20000), rng.standard_normal(20000) * 0.01,
                        rng.uniform(-2 ** -6, 2 ** -6, 20000),
                        np.array([0.0, -0.0, 448.0, -448.0, 460.0, 1e30, -1e30])]).astype(np.float32)
    assert np.array_equal(O.f32_to_e4m3fn_sat(x), _torch_e4m3_codes(x))


def test_e4m3_round_trip_and_ties_to_even():
    codes = np.array([c for c in range(256) if c not in (0x7f, 0xff)], np.uint8)
    vals = O.e4m3fn_to_f32(codes)
    assert np.array_equal(O.f32_to_e4m3fn_sat(vals), codes)
    # midpoints between neighbouring positive codes go to the even mantissa
    pos = np.arange(0, 0x7e, dtype=np.uint8)
    lo, hi = O.e4m3fn_to_f32(pos), O.e4m3fn_to_f32(pos + 1)
    mid = ((lo.astype(np.float64) + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo.astype(np.float64) + hi) / 2)  # exact
    got = O.f32_to_e4m3fn_sat(mid)
    want = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint8)
    assert np.array_equal(got, want)
    # saturation and NaN
    sat = O.f32_to_e4m3fn_sat(np.array([449.0, 1e6, -1e6, np.nan, -np.nan], np.float32))
    assert list(sat[:3]) == [0x7e, 0x7e, 0xfe] and sat[3] & 0x7f == 0x7f


def test_quantize_output_exact_on_integers():
    D = np.array([[3.0, -5.0], [0.0, 96.0], [100.0, -300.0]], np.float32)
    codes, amax = O.quantize_output_e4m3(D, 2.0)
    assert amax == 300.0
    # 200 lies halfway between 192 and 208 (mantissas 4 and 5): ties go to 192; -600 saturates
    want = np.array([[6.0, -10.0], [0.0, 192.0], [192.0, -448.0]], np.float32)
    assert np.array_equal(O.e4m3fn_to_f32(codes), want)


# ------------------------------------------------------------------------------------ mutants

def _pins_pass(gemm, gather, order_fn):
    """Run a compact version of the pins above against candidate functions."""
    rng = np.random.default_rng(77)
    tp, nc, K, M = 3, 2, 7, 5
    ch = [rng.integers(-3, 4, (nc, K)).astype(np.float32) for _ in range(tp)]
    A = rng.integers(-3, 4, (M, K)).astype(np.float32)
    try:
        D = gemm(gather(ch), A)
        if D.shape != (tp * nc, M):
            return False
        if not np.array_equal(D.astype(np.int64), _exact_gemm(np.concatenate(ch), A)):
            return False
        for case in _golden("ring_orders.json")["cases"]:
            if order_fn(case["tp"], case["self_rank"]) != case["order"]:
                return False
    except Exception:
        return False
    return True


def test_pins_catch_planted_mistakes():
    assert _pins_pass(O.gemm_tn, O.gather, O.ring_order)

    def dropped_last_k(G, A):
        return O.gemm_tn(G[:, :-1], A[:, :-1])

    def transposed(G, A):
        # weight read as [K, M] row-major (NN layout) instead of [M, K] (TN)
        m, k = A.shape
        return O.gemm_tn(G, np.ascontiguousarray(A.reshape(k, m).T))

    def wrong_sign(G, A):
        return O.gemm_tn(G, -A)

    def off_by_one_chunk(chunks):
        return O.gather(chunks[1:] + chunks[:1])

    def reversed_ring(tp, s):
        return [(s + j) % tp for j in range(tp)]

    assert not _pins_pass(dropped_last_k, O.gather, O.ring_order)
    assert not _pins_pass(transposed, O.gather, O.ring_order)
    assert not _pins_pass(wrong_sign, O.gather, O.ring_order)
    assert not _pins_pass(O.gemm_tn, off_by_one_chunk, O.ring_order)
    assert not _pins_pass(O.gemm_tn, O.gather, reversed_ring)
