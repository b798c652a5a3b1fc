"""Pins of the reference oracle against things other than itself.

Each test checks the oracle against a fact fixed by the block format or by
mathematics: hand-built blocks whose values were worked out by hand
(tests/golden), exhaustive or randomized comparison with numpy's own IEEE
binary16 conversions, an independently written numpy decoder that uses
index tables instead of bit formulas, closed forms, brute force over all
6-bit scale/min pairs, numpy float64 matrix products, and invariants
(linearity, permutation, splitting along K).  They are chosen so that a
plausible slip in the oracle (a swapped nibble, a wrong scale bit, a dropped
or sign-flipped min term, a transposed operand) fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

from quantized_unpack_q4_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# An independent numpy decoder built from index tables (not bit formulas).
# ---------------------------------------------------------------------------

def _scale_min_bit_table():
    """For each sub-block j and each of the 6 bits (LSB first) of its scale
    and of its min, the (byte, bit) position inside the 12-byte field."""
    sc_pos, m_pos = [], []
    for j in range(8):
        if j < 4:
            sc_pos.append([(j, b) for b in range(6)])
            m_pos.append([(j + 4, b) for b in range(6)])
        else:
            sc_pos.append([(j + 4, b) for b in range(4)] + [(j - 4, 6), (j - 4, 7)])
            m_pos.append([(j + 4, 4 + b) for b in range(4)] + [(j, 6), (j, 7)])
    return sc_pos, m_pos


_SC_POS, _M_POS = _scale_min_bit_table()


def np_decode_q4k(blocks: np.ndarray):
    """blocks: uint8 [n][144] -> (d, dmin, sc[n][8], m[n][8], q[n][256])."""
    blocks = blocks.reshape(-1, 144)
    n = blocks.shape[0]
    d = blocks[:, 0:2].copy().view("<f2").astype(np.float64).reshape(n)
    dmin = blocks[:, 2:4].copy().view("<f2").astype(np.float64).reshape(n)
    bits = np.unpackbits(blocks[:, 4:16], axis=1, bitorder="little").reshape(n, 12, 8)
    sc = np.zeros((n, 8), np.int64)
    m = np.zeros((n, 8), np.int64)
    for j in range(8):
        for i, (byte, bit) in enumerate(_SC_POS[j]):
            sc[:, j] += bits[:, byte, bit].astype(np.int64) << i
        for i, (byte, bit) in enumerate(_M_POS[j]):
            m[:, j] += bits[:, byte, bit].astype(np.int64) << i
    qs = blocks[:, 16:].reshape(n, 4, 32)
    q = np.concatenate([qs & 0x0F, qs >> 4], axis=2).reshape(n, 256).astype(np.int64)
    return d, dmin, sc, m, q


def np_weights_q4k(blocks: np.ndarray) -> np.ndarray:
    """binary32 weights [n][256] via the independent decoder (exact in float64)."""
    d, dmin, sc, m, q = np_decode_q4k(blocks)
    scj = np.repeat(sc, 32, axis=1)
    mj = np.repeat(m, 32, axis=1)
    w = d[:, None] * scj * q - dmin[:, None] * mj
    return w.astype(np.float32)


def np_pack_scale_min(sc, m) -> np.ndarray:
    """Write eight scales and mins into 12 bytes through the same position tables."""
    sc = np.asarray(sc, np.int64)
    m = np.asarray(m, np.int64)
    bits = np.zeros((12, 8), np.uint8)
    for j in range(8):
        for i, (byte, bit) in enumerate(_SC_POS[j]):
            bits[byte, bit] = (sc[j] >> i) & 1
        for i, (byte, bit) in enumerate(_M_POS[j]):
            bits[byte, bit] = (m[j] >> i) & 1
    return np.packbits(bits.reshape(-1), bitorder="little")


def make_q4k_block(d, dmin, sc, m, q) -> np.ndarray:
    blk = np.zeros(144, np.uint8)
    blk[0:2] = np.array([d], "<f2").view(np.uint8)
    blk[2:4] = np.array([dmin], "<f2").view(np.uint8)
    blk[4:16] = np_pack_scale_min(sc, m)
    q = np.asarray(q, np.uint8).reshape(4, 64)
    blk[16:] = (q[:, :32] | (q[:, 32:] << 4)).reshape(-1)
    return blk


def make_q8_0_block(d_bits: int, q) -> np.ndarray:
    blk = np.zeros(34, np.uint8)
    blk[0] = d_bits & 0xFF
    blk[1] = d_bits >> 8
    blk[2:] = np.asarray(q, np.int8).view(np.uint8)
    return blk


# ---------------------------------------------------------------------------
# binary16
# ---------------------------------------------------------------------------

def test_half_decode_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint16)
    ours = orc.half_to_double(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros decode with their sign
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_half_encode_matches_numpy_rne(orc):
    g = np.random.default_rng(123)
    # binary32 values spread over every binary16 exponent, subnormals included
    v = (g.standard_normal(200000) * np.exp2(g.uniform(-27, 17, 200000))).astype(np.float32)
    # exact ties: midpoints between neighbouring binary16 values
    h = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    ties = ((lo + hi) / 2).astype(np.float32)
    extra = np.array([65504, 65519.996, 65520, 65536, 1e6, 2.0 ** -24, 2.0 ** -25,
                      2.0 ** -25 * 1.0000001, 2.0 ** -14, 2.0 ** -14 * (1 - 2 ** -12),
                      0.0, -0.0, 1.0, -1.0], np.float32)
    allv = np.concatenate([v, ties, -ties, extra])
    ours = orc.double_to_half(allv.astype(np.float64))
    with np.errstate(over="ignore"):
        ref = allv.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------------------
# Hand-built blocks (tests/golden)
# ---------------------------------------------------------------------------

def test_q4k_handbuilt_golden(orc):
    gd = json.load(open(os.path.join(GOLDEN, "q4k_handbuilt.json")))
    f = gd["fields"]
    q = np.arange(256) % 16
    blk = make_q4k_block(f["d"], f["dmin"], f["sc"], f["m"], q)
    # the packed header must be the bytes derived by hand
    assert blk[:16].tobytes().hex() == gd["header_hex"]
    assert np.all(blk[16:].reshape(4, 32) == (0x11 * (np.arange(32) % 16)).astype(np.uint8))
    d, dmin, sc, m, qo = orc.q4k_fields(blk)
    assert d == 1.0 and dmin == 0.5
    assert list(sc) == f["sc"] and list(m) == f["m"]
    assert np.array_equal(qo, q)
    w32, w16 = orc.dequant(orc.Q4_K, blk, 1, 256)
    for k, val in gd["weights"].items():
        assert w32[0, int(k)] == val, k
    assert float(w32.astype(np.float64).sum()) == gd["row_sum"]
    y, S = orc.gemv(orc.Q4_K, blk, np.ones((1, 256), np.float32), 1, 256)
    assert y[0, 0] == gd["row_sum"]


def test_q8_0_handbuilt_golden(orc):
    gd = json.load(open(os.path.join(GOLDEN, "q8_0_handbuilt.json")))
    b0, b1 = gd["blocks"]
    blk0 = make_q8_0_block(int(b0["d_bits"], 16), np.arange(32) - 16)
    q1 = np.zeros(32, np.int64)
    q1[0], q1[1] = -128, 127
    blk1 = make_q8_0_block(int(b1["d_bits"], 16), q1)
    for blk, gdb in ((blk0, b0), (blk1, b1)):
        w32, _ = orc.dequant(orc.Q8_0, blk, 1, 32)
        for k, val in gdb["weights"].items():
            assert w32[0, int(k)] == val
        y, _ = orc.gemv(orc.Q8_0, blk, np.ones((1, 32), np.float32), 1, 32)
        assert y[0, 0] == gdb["row_sum"]


# ---------------------------------------------------------------------------
# Independent decoder, brute force, special cases
# ---------------------------------------------------------------------------

def test_scale_min_all_pairs_roundtrip(orc):
    """Every (scale, min) pair at every sub-block position survives pack->unpack."""
    vals = np.arange(64)
    for j in range(8):
        for s in vals:
            sc = np.full(8, 17)
            m = np.full(8, 42)
            # sweep all 64 mins for this scale in 64 blocks at once
            blocks = []
            for mm in vals:
                sc[j] = s
                m[j] = mm
                blocks.append(make_q4k_block(0.0, 0.0, sc, m, np.zeros(256)))
            blocks = np.stack(blocks)
            for i in range(64):
                _, _, so, mo, _ = orc.q4k_fields(blocks[i])
                assert so[j] == s and mo[j] == i
                others = [t for t in range(8) if t != j]
                assert np.all(so[others] == 17) and np.all(mo[others] == 42)


def test_independent_decoder_agrees_on_random_blocks(orc):
    blocks = synth.q4k_blocks(99, 0, 40, 256 * 250).reshape(-1, 144)  # 10^4 blocks
    assert blocks.shape[0] == 10000
    d, dmin, sc, m, q = np_decode_q4k(blocks)
    for i in range(0, 10000, 97):
        od, odm, osc, om, oq = orc.q4k_fields(blocks[i])
        assert od == d[i] and odm == dmin[i]
        assert np.array_equal(osc, sc[i]) and np.array_equal(om, m[i])
        assert np.array_equal(oq, q[i])
    w32, w16 = orc.dequant(orc.Q4_K, blocks.reshape(-1), 10000, 256)
    ref = np_weights_q4k(blocks)
    assert np.array_equal(w32.view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(w16, ref.astype(np.float16).view(np.uint16))


def test_nibble_positions_one_hot(orc):
    """A block with one non-zero quant gives exactly one non-zero weight, at
    the position the layout assigns to that byte and nibble."""
    sc = np.full(8, 1)
    m = np.zeros(8)
    for byte in range(128):
        for hi in (0, 1):
            blk = make_q4k_block(1.0, 0.0, sc, m, np.zeros(256))
            blk[16 + byte] = (7 << 4) if hi else 7
            w32, _ = orc.dequant(orc.Q4_K, blk, 1, 256)
            nz = np.flatnonzero(w32[0])
            g, i = divmod(byte, 32)
            assert list(nz) == [64 * g + 32 * hi + i]
            assert w32[0, nz[0]] == 7.0


def test_q4k_special_cases(orc):
    g = np.random.default_rng(5)
    q = g.integers(0, 16, 256)
    sc = g.integers(0, 64, 8)
    m = g.integers(0, 64, 8)
    d, dmin = np.float16(0.0123), np.float16(0.0457)
    dd, dm = float(d), float(dmin)
    # all-zero quants: w = -dmin * m
    w, _ = orc.dequant(orc.Q4_K, make_q4k_block(d, dmin, sc, m, np.zeros(256)), 1, 256)
    assert np.array_equal(w[0], np.float32(-dm * np.repeat(m, 32)))
    # all-max: q = 15, sc = m = 63 -> 945 d - 63 dmin
    w, _ = orc.dequant(orc.Q4_K, make_q4k_block(d, dmin, np.full(8, 63), np.full(8, 63),
                                                np.full(256, 15)), 1, 256)
    assert np.all(w[0] == np.float32(945 * dd - 63 * dm))
    # d = 0: w = -dmin * m whatever the quants
    w, _ = orc.dequant(orc.Q4_K, make_q4k_block(0.0, dmin, sc, m, q), 1, 256)
    assert np.array_equal(w[0], np.float32(-dm * np.repeat(m, 32)))
    # d = dmin = 0: every output is exactly zero
    blk = make_q4k_block(0.0, 0.0, sc, m, q)
    y, S = orc.gemv(orc.Q4_K, blk, g.standard_normal((3, 256)).astype(np.float32), 1, 256)
    assert np.all(y == 0) and np.all(S == 0)
    # negative and subnormal d / dmin
    for dv, dmv in ((-0.25, 0.5), (2.0 ** -24 * 3, 2.0 ** -20), (-(2.0 ** -15), -(2.0 ** -23))):
        w, w16 = orc.dequant(orc.Q4_K, make_q4k_block(dv, dmv, sc, m, q), 1, 256)
        exact = dv * np.repeat(sc, 32) * q - dmv * np.repeat(m, 32)
        assert np.array_equal(w[0], exact.astype(np.float32))
        assert np.array_equal(w16[0], exact.astype(np.float32).astype(np.float16).view(np.uint16))


def test_single_nonzero_weight_row_is_exact(orc):
    """A row whose only non-zero weight sits at column j gives y = w * x_j exactly."""
    K = 512
    sc = np.zeros(8)
    sc[3] = 5
    blk0 = make_q4k_block(0.75, 0.0, sc, np.zeros(8), np.where(np.arange(256) == 100, 9, 0))
    blk1 = make_q4k_block(0.0, 0.0, np.zeros(8), np.zeros(8), np.zeros(256))
    row = np.concatenate([blk0, blk1])
    x = np.random.default_rng(1).standard_normal((2, K)).astype(np.float32)
    y, S = orc.gemv(orc.Q4_K, row, x, 1, K)
    w = 0.75 * 5 * 9
    assert np.array_equal(y[:, 0], w * x[:, 100].astype(np.float64))
    assert np.array_equal(S[:, 0], np.abs(y[:, 0]))


def test_q8_0_random_against_numpy(orc):
    M, K = 7, 96
    w = synth.q8_0_blocks(3, 0, M, K)
    blocks = w.reshape(-1, 34)
    d = blocks[:, 0:2].copy().view("<f2").astype(np.float64)
    q = blocks[:, 2:].view(np.int8).astype(np.float64)
    ref = (d * q).astype(np.float32).reshape(M, K)
    w32, w16 = orc.dequant(orc.Q8_0, w, M, K)
    assert np.array_equal(w32, ref)
    assert np.array_equal(w16, ref.astype(np.float16).view(np.uint16))


# ---------------------------------------------------------------------------
# Products: closed forms, library routine, invariants
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def q4k_small():
    M, K = 37, 1024
    w = synth.q4k_blocks(11, 0, M, K)
    x = synth.activations_f32(11, 0, 3, K)
    return M, K, w, x


def test_one_hot_reads_a_column(orc, q4k_small):
    M, K, w, _ = q4k_small
    w32, _ = orc.dequant(orc.Q4_K, w, M, K)
    for k in (0, 31, 32, 255, 256, 700, K - 1):
        e = np.zeros((1, K), np.float32)
        e[0, k] = 1.0
        y, _ = orc.gemv(orc.Q4_K, w, e, M, K)
        assert np.array_equal(y[0], w32[:, k].astype(np.float64))


def test_ones_gives_closed_form_row_sums(orc, q4k_small):
    M, K, w, _ = q4k_small
    d, dmin, sc, m, q = np_decode_q4k(w.reshape(-1, 144))
    qsum = q.reshape(-1, 8, 32).sum(axis=2)
    # per super-block: sum_j (d sc_j sum(q) - dmin m_j 32), every term exact in float64
    per_sb = (d[:, None] * sc * qsum - dmin[:, None] * m * 32).sum(axis=1)
    # the oracle rounds each weight to binary32 first; the generator's values keep
    # every weight exact in binary32 only sometimes, so compare with a tight bound
    closed = per_sb.reshape(M, -1).sum(axis=1)
    y, S = orc.gemv(orc.Q4_K, w, np.ones((1, K), np.float32), M, K)
    assert np.all(np.abs(y[0] - closed) <= 1e-6 * S[0])


def test_matches_numpy_float64_matmul(orc, q4k_small):
    M, K, w, x = q4k_small
    ref = np_weights_q4k(w.reshape(-1, 144)).reshape(M, K).astype(np.float64)
    y, S = orc.gemv(orc.Q4_K, w, x, M, K)
    yref = x.astype(np.float64) @ ref.T
    assert np.all(np.abs(y - yref) <= 1e-12 * S)
    assert np.allclose(S, np.abs(x.astype(np.float64)) @ np.abs(ref).T, rtol=1e-12)


def test_fused_equals_separate(orc, q4k_small):
    M, K, w, x = q4k_small
    y, _ = orc.gemv(orc.Q4_K, w, x, M, K)
    y2 = orc.gemv_separate(orc.Q4_K, w, x, M, K)
    assert np.array_equal(y, y2)
    wq = synth.q8_0_blocks(12, 0, 9, 256)
    xq = synth.activations_f32(12, 0, 2, 256)
    assert np.array_equal(orc.gemv(orc.Q8_0, wq, xq, 9, 256)[0],
                          orc.gemv_separate(orc.Q8_0, wq, xq, 9, 256))


def test_linearity_and_permutation(orc, q4k_small):
    M, K, w, x = q4k_small
    y, S = orc.gemv(orc.Q4_K, w, x, M, K)
    # linearity: scaling by a power of two is exact, sums within rounding
    y2, _ = orc.gemv(orc.Q4_K, w, (4 * x).astype(np.float32), M, K)
    assert np.array_equal(y2, 4 * y)
    ysum, _ = orc.gemv(orc.Q4_K, w, (x[0:1] + x[1:2]).astype(np.float32), M, K)
    Ssum = S[0] + S[1]
    assert np.all(np.abs(ysum[0] - (y[0] + y[1])) <= 1e-6 * Ssum)
    # row permutation: permuting the packed rows permutes the outputs
    perm = np.random.default_rng(2).permutation(M)
    rb = K // 256 * 144
    wp = w.reshape(M, rb)[perm].reshape(-1)
    yp, _ = orc.gemv(orc.Q4_K, wp, x, M, K)
    assert np.array_equal(yp, y[:, perm])
    # row subset selection matches full computation
    ys, _ = orc.gemv(orc.Q4_K, w, x, M, K, rows=perm[:5])
    assert np.array_equal(ys, y[:, perm[:5]])


def test_split_along_k_adds_up(orc, q4k_small):
    M, K, w, x = q4k_small
    rb = K // 256 * 144
    rows = w.reshape(M, rb)
    split = 3 * 144  # after three super-blocks
    k1 = 3 * 256
    w1 = np.ascontiguousarray(rows[:, :split]).reshape(-1)
    w2 = np.ascontiguousarray(rows[:, split:]).reshape(-1)
    y, S = orc.gemv(orc.Q4_K, w, x, M, K)
    y1, _ = orc.gemv(orc.Q4_K, w1, np.ascontiguousarray(x[:, :k1]), M, k1)
    y2, _ = orc.gemv(orc.Q4_K, w2, np.ascontiguousarray(x[:, k1:]), M, K - k1)
    assert np.all(np.abs(y - (y1 + y2)) <= 1e-13 * S)


def test_gemm_single_token_equals_gemv(orc, q4k_small):
    M, K, w, _ = q4k_small
    x16 = synth.activations_f16(11, 5, 4, K)
    y, S = orc.gemm(orc.Q4_K, w, x16, M, K)
    yv, Sv = orc.gemv(orc.Q4_K, w, x16.astype(np.float32), M, K)
    assert np.array_equal(y, yv) and np.array_equal(S, Sv)
    ys, _ = orc.gemm(orc.Q4_K, w, x16, M, K, rows=[3, 1], toks=[2])
    assert np.array_equal(ys, y[[2]][:, [3, 1]])


def test_gemm_matches_numpy(orc):
    M, K, N = 20, 512, 6
    w = synth.q4k_blocks(21, 0, M, K)
    x16 = synth.activations_f16(21, 0, N, K)
    ref = np_weights_q4k(w.reshape(-1, 144)).reshape(M, K).astype(np.float64)
    y, S = orc.gemm(orc.Q4_K, w, x16, M, K)
    assert np.all(np.abs(y - x16.astype(np.float64) @ ref.T) <= 1e-12 * S)


# ---------------------------------------------------------------------------
# Mixture of experts
# ---------------------------------------------------------------------------

def test_moe_route_brute_force(orc):
    T, E, k = 300, 64, 8
    logits = synth.router_logits(4, 0, T, E)
    # exact ties: duplicate some logits so the lower index must win
    logits[0, 10] = logits[0, 3]
    logits[1, :] = 0.5
    ids, wts = orc.moe_route(logits, k)
    l64 = logits.astype(np.float64)
    p = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-p[t, e], e))[:k]
        assert list(ids[t]) == order
        assert np.allclose(wts[t], p[t, order], rtol=1e-14, atol=0)
    assert list(ids[1]) == list(range(8))
    assert np.all(np.diff(wts, axis=1) <= 0)


def test_moe_route_renormalized(orc):
    """Renormalised top-k: the same experts, weights divided by their sum
    (brute force in numpy; they sum to one and keep their ratios)."""
    T, E, k = 200, 60, 6
    logits = synth.router_logits(5, 0, T, E)
    logits[2, :] = -1.25  # all tied: experts 0..k-1, equal weights 1/k
    ids, wts = orc.moe_route(logits, k)
    ids_r, wts_r = orc.moe_route(logits, k, renormalize=True)
    assert np.array_equal(ids, ids_r)
    l64 = logits.astype(np.float64)
    p = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-p[t, e], e))[:k]
        q = p[t, order]
        assert np.allclose(wts_r[t], q / q.sum(), rtol=1e-14, atol=0)
    assert np.allclose(wts_r.sum(axis=1), 1.0, rtol=0, atol=1e-15 * k)
    assert np.allclose(wts_r / wts_r[:, :1], wts / wts[:, :1], rtol=1e-14, atol=0)
    assert list(ids_r[2]) == list(range(k)) and np.allclose(wts_r[2], 1.0 / k, rtol=1e-15)


def test_swiglu_closed_forms(orc):
    """h = silu(g) * u: silu(0) = 0, silu(1) = 1/(1+e^-1) (the logistic function
    at 1, 0.7310585786300049), silu(-1) = -1/(1+e) (0.2689414213699951 negated),
    silu(2) = 2/(1+e^-2) (1.7615941559557646), silu(z) - silu(-z) = z, silu
    of a large positive z is z and of a large negative z is (-)0; linear in u."""
    g = np.array([0.0, 1.0, -1.0, 2.0, 40.0, -800.0, 0.5, -0.5, 3.25, -3.25])
    u = np.array([5.0, 1.0, 1.0, 1.0, 0.25, 7.0, 1.0, 1.0, -2.0, -2.0])
    h = orc.swiglu(g, u)
    assert h[0] == 0.0
    assert abs(h[1] - 0.7310585786300049) <= 2e-16
    assert abs(h[2] + 0.2689414213699951) <= 2e-16
    assert abs(h[3] - 1.7615941559557646) <= 4e-16
    assert h[4] == 10.0 and h[5] == 0.0 and np.isfinite(h).all()
    assert abs((h[6] - h[7]) - 0.5) <= 1e-15 and abs((h[8] - h[9]) / -2.0 - 3.25) <= 1e-15
    h3 = orc.swiglu(g, 3.0 * u)
    assert np.allclose(h3, 3.0 * h, rtol=1e-15, atol=0)


def test_moe_input_weighted(orc):
    """Slot weight on the expert's input: with weight 2 (an exact scaling of
    binary16 activations) it equals the output-weighted layer run on 2x with
    weight 1, bit for bit; with weight 1 both forms agree; and the output is
    the unweighted sum of the slots' d."""
    T, H, I, E, k = 3, 512, 256, 4, 2
    wg = synth.q4k_blocks(33, 0, E * I, H)
    wu = synth.q4k_blocks(33, 1, E * I, H)
    wd = synth.q4k_blocks(33, 2, E * H, I)
    x16 = synth.activations_f16(33, 0, T, H)
    ids = np.array([[0, 3], [2, 1], [1, 0]], np.int32)
    two = np.full((T, k), 2.0, np.float32)
    one = np.ones((T, k), np.float32)
    r_in = orc.moe_ffn(wg, wu, wd, x16, ids, two, H, I, E, weight_input=True)
    x2 = (x16.astype(np.float32) * 2).astype(np.float16)
    assert np.array_equal(x2.astype(np.float64), 2 * x16.astype(np.float64))
    r_out = orc.moe_ffn(wg, wu, wd, x2, ids, one, H, I, E)
    for key in ("g", "u", "h", "d", "out"):
        assert np.array_equal(r_in[key], r_out[key]), key
    w = np.array([[0.7, 0.3], [0.5, 0.25], [1.0, 0.125]], np.float32)
    r_in = orc.moe_ffn(wg, wu, wd, x16, ids, w, H, I, E, weight_input=True)
    assert np.allclose(r_in["out"], r_in["d"].reshape(T, k, H).sum(axis=1), rtol=1e-15, atol=1e-300)
    r_1 = orc.moe_ffn(wg, wu, wd, x16, ids, one, H, I, E, weight_input=True)
    r_1o = orc.moe_ffn(wg, wu, wd, x16, ids, one, H, I, E)
    assert np.array_equal(r_1["out"], r_1o["out"])


def _silu(z):
    return z / (1.0 + np.exp(-z))


def test_moe_single_expert_is_dense_swiglu(orc):
    T, H, I, E = 5, 512, 256, 1
    wg = synth.q4k_blocks(31, 0, I, H)
    wu = synth.q4k_blocks(31, 1, I, H)
    wd = synth.q4k_blocks(31, 2, H, I)
    x16 = synth.activations_f16(31, 0, T, H)
    ids = np.zeros((T, 1), np.int32)
    wts = np.ones((T, 1), np.float32)
    r = orc.moe_ffn(wg, wu, wd, x16, ids, wts, H, I, E)
    g, _ = orc.gemm(orc.Q4_K, wg, x16, I, H)
    u, _ = orc.gemm(orc.Q4_K, wu, x16, I, H)
    h = _silu(g) * u
    Wd = np_weights_q4k(wd.reshape(-1, 144)).reshape(H, I).astype(np.float64)
    d = h @ Wd.T
    assert np.array_equal(r["g"], g) and np.array_equal(r["u"], u)
    assert np.allclose(r["h"], h, rtol=1e-15, atol=0)
    assert np.all(np.abs(r["d"] - d) <= 1e-12 * r["Sd"])
    assert np.array_equal(r["out"], r["d"])


def test_moe_combines_experts_with_weights(orc):
    T, H, I, E, k = 4, 256, 256, 6, 3
    wg = synth.q4k_blocks(32, 0, E * I, H)
    wu = synth.q4k_blocks(32, 1, E * I, H)
    wd = synth.q4k_blocks(32, 2, E * H, I)
    x16 = synth.activations_f16(32, 0, T, H)
    ids, wts = orc.moe_route(synth.router_logits(32, 0, T, E), k)
    r = orc.moe_ffn(wg, wu, wd, x16, ids, wts, H, I, E)
    gu = I * (H // 256) * 144
    dn = H * (I // 256) * 144
    for t in range(T):
        acc = np.zeros(H)
        for s in range(k):
            e = ids[t, s]
            g, _ = orc.gemm(orc.Q4_K, wg[e * gu:(e + 1) * gu], x16[t:t + 1], I, H)
            u, _ = orc.gemm(orc.Q4_K, wu[e * gu:(e + 1) * gu], x16[t:t + 1], I, H)
            h = _silu(g[0]) * u[0]
            Wd = np_weights_q4k(wd[e * dn:(e + 1) * dn].reshape(-1, 144)).reshape(H, I)
            d = Wd.astype(np.float64) @ h
            a = t * k + s
            assert np.all(np.abs(r["d"][a] - d) <= 1e-12 * r["Sd"][a])
            acc += np.float32(wts[t, s]).astype(np.float64) * d
        assert np.allclose(r["out"][t], acc, rtol=1e-12, atol=1e-300)


def _np_weights_q8_0(w, R, C):
    blocks = np.ascontiguousarray(w).reshape(-1, 34)
    d = blocks[:, 0:2].copy().view("<f2").astype(np.float64)
    q = blocks[:, 2:].view(np.int8).astype(np.float64)
    return (d * q).astype(np.float32).reshape(R, C).astype(np.float64)


@pytest.mark.parametrize("weight_input", [False, True])
def test_moe_q8_0_against_numpy(orc, weight_input):
    """Q8_0 expert stacks: every slot's g, u, d against numpy products of the
    numpy-decoded weights (d * q per 32-weight block, rounded to binary32),
    and the combine as the weighted (or, input-weighted, unweighted) sum."""
    T, H, I, E, k = 3, 256, 128, 3, 2
    wg = synth.q8_0_blocks(34, 0, E * I, H)
    wu = synth.q8_0_blocks(34, 1, E * I, H)
    wd = synth.q8_0_blocks(34, 2, E * H, I)
    x16 = synth.activations_f16(34, 0, T, H)
    ids = np.array([[0, 2], [1, 0], [2, 1]], np.int32)
    wts = np.array([[0.6, 0.4], [0.75, 0.25], [0.5, 0.5]], np.float32)
    r = orc.moe_ffn(wg, wu, wd, x16, ids, wts, H, I, E, weight_input=weight_input, fmt=orc.Q8_0)
    Wg = _np_weights_q8_0(wg, E * I, H).reshape(E, I, H)
    Wu = _np_weights_q8_0(wu, E * I, H).reshape(E, I, H)
    Wd = _np_weights_q8_0(wd, E * H, I).reshape(E, H, I)
    x = x16.astype(np.float64)
    for t in range(T):
        acc = np.zeros(H)
        for s in range(k):
            e, a, p = ids[t, s], t * k + s, np.float64(wts[t, s])
            xin = p * x[t] if weight_input else x[t]
            g, u = Wg[e] @ xin, Wu[e] @ xin
            assert np.all(np.abs(r["g"][a] - g) <= 1e-12 * r["Sg"][a])
            assert np.all(np.abs(r["u"][a] - u) <= 1e-12 * r["Su"][a])
            d = Wd[e] @ r["h"][a]
            assert np.all(np.abs(r["d"][a] - d) <= 1e-12 * r["Sd"][a])
            acc += (1.0 if weight_input else p) * r["d"][a]
        assert np.allclose(r["out"][t], acc, rtol=1e-12, atol=1e-300)
    assert np.allclose(r["h"], _silu(r["g"]) * r["u"], rtol=1e-15, atol=0)


# ---------------------------------------------------------------------------
# Activations as 8-bit blocks and the integer-dot product
# ---------------------------------------------------------------------------

def test_quantize_q8k_closed_forms(orc):
    """A block of integers in [-127, 127] that holds 127 has scale 127/127 = 1
    and keeps its values as codes (ties 2.5 -> 2, 3.5 -> 4, -2.5 -> -2 go to
    even); a constant block codes to 127 with scale c/127; a zero block has
    scale 0 and zero codes; sub-block sums are the sums of the 32 codes."""
    K = 768
    x = np.zeros((1, K), np.float32)
    blk = np.arange(-128, 128, dtype=np.float32)
    blk[0] = 127.0
    blk[1:5] = [2.5, 3.5, -2.5, -0.5]
    x[0, :256] = blk
    x[0, 256:512] = np.float32(0.3)
    q, d, bs = orc.quantize_q8k(x, K)
    assert d[0, 0] == 1.0 and d[0, 2] == 0.0
    expect = blk.copy()
    expect[1:5] = [2, 4, -2, 0]
    assert np.array_equal(q[0, :256].astype(np.float32), expect)
    assert np.all(q[0, 256:512] == 127)
    assert d[0, 1] == np.float32(0.3) / np.float32(127)
    assert np.all(q[0, 512:] == 0)
    assert np.array_equal(bs[0], q[0].reshape(-1, 32).astype(np.int64).sum(axis=1))
    assert bs[0, 8] == 127 * 32


def test_quantize_q8k_bounds_and_scaling(orc):
    """Random blocks: codes in [-127, 127] with 127 reached in magnitude, the
    rounding error |x - d q| within half a step (plus the binary32 rounding
    of the scale), and power-of-two scaling of x leaves the codes unchanged
    and scales d exactly."""
    B, K = 3, 1024
    x = synth.activations_f32(40, 0, B, K)
    x[1, 256:512] *= np.float32(1e-30)
    x[2, 512:768] *= np.float32(1e30)
    q, d, bs = orc.quantize_q8k(x, K)
    qb = q.reshape(B, -1, 256).astype(np.int64)
    assert np.all(np.abs(qb).max(axis=2) == 127)
    step = np.repeat(d.astype(np.float64), 256, axis=1)
    err = np.abs(x.astype(np.float64) - step * q)
    assert np.all(err <= step * (0.5 + 2.0 ** -16))
    q2, d2, _ = orc.quantize_q8k(x * np.float32(2.0 ** 20), K)
    assert np.array_equal(q2, q) and np.array_equal(d2, d * np.float32(2.0 ** 20))


def test_gemv_q4k_q8k_against_numpy(orc):
    """The integer-dot product against numpy: exact fp64 weights from the
    independent table decoder times the decoded activations d * q."""
    M, K, B = 9, 768, 3
    w = synth.q4k_blocks(41, 0, M, K)
    x = synth.activations_f32(41, 0, B, K)
    q, d, _ = orc.quantize_q8k(x, K)
    dd, dmin, sc, m, qq = np_decode_q4k(w.reshape(-1, 144))
    W = (dd[:, None] * np.repeat(sc, 32, axis=1) * qq
         - dmin[:, None] * np.repeat(m, 32, axis=1)).reshape(M, K)
    xh = np.repeat(d.astype(np.float64), 256, axis=1) * q
    ref = xh @ W.T
    y, S = orc.gemv_q4k_q8k(w, q, d, M, K)
    assert np.all(np.abs(y - ref) <= 1e-12 * S)
    rows = np.array([8, 0, 4])
    yr, Sr = orc.gemv_q4k_q8k(w, q, d, M, K, rows=rows)
    assert np.array_equal(yr, y[:, rows]) and np.array_equal(Sr, S[:, rows])


def test_gemv_q4k_q8k_deviation_from_binary32_path(orc):
    """The documented cost of quantizing activations: against the binary32
    product, |y_q8 - y| <= sum_k |w_k| |x_k - d q_k| (plus the binary32
    rounding of the weights in y), and it vanishes when x is already a block
    of integers with 127 in it."""
    M, K, B = 16, 1024, 2
    w = synth.q4k_blocks(42, 0, M, K)
    x = synth.activations_f32(42, 0, B, K)
    q, d, _ = orc.quantize_q8k(x, K)
    y8, _ = orc.gemv_q4k_q8k(w, q, d, M, K)
    y, S = orc.gemv(orc.Q4_K, w, x, M, K)
    W = np.abs(np_weights_q4k(w.reshape(-1, 144)).reshape(M, K).astype(np.float64))
    dx = np.abs(x.astype(np.float64) - np.repeat(d.astype(np.float64), 256, axis=1) * q)
    bound = dx @ W.T + 2.0 ** -23 * S
    assert np.all(np.abs(y8 - y) <= bound)
    xi = np.clip(np.round(x * 40), -127, 127).astype(np.float32)
    xi[:, ::256] = 127.0
    qi, di, _ = orc.quantize_q8k(xi, K)
    assert np.all(di == 1.0) and np.array_equal(qi.astype(np.float32), xi)
    y8i, S8 = orc.gemv_q4k_q8k(w, qi, di, M, K)
    yi, Si = orc.gemv(orc.Q4_K, w, xi, M, K)
    assert np.all(np.abs(y8i - yi) <= 2.0 ** -23 * Si + 1e-12 * S8)


def test_gemm_matmul_equals_gemm(orc):
    """The matrix-product form of the oracle's GEMM (used for large parity
    samples) agrees with the plain loop: same decoded weights, binary64 sums,
    only the summation order differs; rows and tokens subsets index alike."""
    from quantized_unpack_q4_amd import synth
    for fmt, M, K, N in ((orc.Q4_K, 37, 512, 11), (orc.Q8_0, 29, 320, 7)):
        blocks = synth.q4k_blocks if fmt == orc.Q4_K else synth.q8_0_blocks
        w = blocks(61, 0, M, K)
        x16 = synth.activations_f16(61, 1, N, K)
        y, S = orc.gemm(fmt, w, x16, M, K)
        y2, S2 = orc.gemm_matmul(fmt, w, x16, M, K)
        assert np.all(np.abs(y - y2) <= 1e-13 * S)
        assert np.allclose(S, S2, rtol=1e-13, atol=0)
        rows, toks = np.array([0, 5, M - 1]), np.array([N - 1, 2])
        y3, S3 = orc.gemm_matmul(fmt, w, x16, M, K, rows=rows, toks=toks)
        assert np.all(np.abs(y3 - y[np.ix_(toks, rows)]) <= 1e-13 * S[np.ix_(toks, rows)])


def test_q4k_terms_against_independent_decoder(orc):
    """The two exact weight terms from the C decoder equal those of the
    independent numpy table decoder, and a - c rounded once to binary32 is the
    oracle's binary32 weight."""
    M, K = 7, 512
    w = synth.q4k_blocks(43, 0, M, K)
    dd, dmin, sc, m, qq = np_decode_q4k(w.reshape(-1, 144))
    A = (dd[:, None] * np.repeat(sc, 32, axis=1) * qq).reshape(M, K)
    C = (dmin[:, None] * np.repeat(m, 32, axis=1)).reshape(M, K)
    a, c = orc.q4k_terms(w, M, K)
    assert np.array_equal(a, A) and np.array_equal(c, C)
    w32, _ = orc.dequant(orc.Q4_K, w, M, K)
    assert np.array_equal((a - c).astype(np.float32).view(np.uint32), w32.view(np.uint32))
    a2, c2 = orc.q4k_terms(w, M, K, rows=[6, 1])
    assert np.array_equal(a2, a[[6, 1]]) and np.array_equal(c2, c[[6, 1]])


def test_gemm_q4k_q8k_forms_agree(orc):
    """The integer-dot product over many tokens: the plain loop with tokens as
    its batch rows, the matrix-product form, and numpy on the independently
    decoded weights all agree; a token subset indexes alike."""
    M, K, N = 11, 512, 9
    w = synth.q4k_blocks(44, 0, M, K)
    x = synth.activations_f32(44, 1, N, K)
    q, d, _ = orc.quantize_q8k(x, K)
    y, S = orc.gemm_q4k_q8k(w, q, d, M, K)
    y2, S2 = orc.gemm_q4k_q8k_matmul(w, q, d, M, K)
    assert y.shape == (N, M)
    assert np.all(np.abs(y - y2) <= 1e-13 * S) and np.allclose(S, S2, rtol=1e-13, atol=0)
    dd, dmin, sc, m, qq = np_decode_q4k(w.reshape(-1, 144))
    W = (dd[:, None] * np.repeat(sc, 32, axis=1) * qq
         - dmin[:, None] * np.repeat(m, 32, axis=1)).reshape(M, K)
    ref = (np.repeat(d.astype(np.float64), 256, axis=1) * q) @ W.T
    assert np.all(np.abs(y - ref) <= 1e-12 * S)
    toks, rows = np.array([8, 2]), np.array([0, 10, 5])
    y3, _ = orc.gemm_q4k_q8k_matmul(w, q, d, M, K, rows=rows, toks=toks)
    assert np.all(np.abs(y3 - y[np.ix_(toks, rows)]) <= 1e-13 * S[np.ix_(toks, rows)])
