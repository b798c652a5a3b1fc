"""Parity of the fused dequant matrix product (prefill) with the binary64 oracle.

Bound: |Y_gpu - Y_ref| <= 2e-3 * S with S = sum_k |w_k x_k|: binary16
weights and output, binary32 accumulation, oracle in binary64 on the binary32
weights.  One-hot activation rows must read out the binary16 weights exactly.
"""
import numpy as np
import pytest

import oracle
from quantized_unpack_q4_amd import gq, synth
from tests._gpu import dev, half_bits, say, torch_cuda, within

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _gemm(w_d, x16, M, K, tile_rows=None):
    torch = torch_cuda()
    N = x16.shape[0]
    y = torch.empty((N, M), dtype=torch.float16, device="cuda")
    if tile_rows is None:
        gq.gq_gemm_q4k(w_d, dev(x16), y, M, K, N)
    else:
        gq.gq_gemm_q4k_tiles(w_d, dev(x16), y, M, K, N, tile_rows)
    return half_bits(y).view(np.float16).astype(np.float64)


@pytest.mark.parametrize("M,K,N", [(128, 256, 1), (130, 512, 37), (256, 1024, 128),
                                   (200, 2048, 300), (64, 768, 8), (1, 256, 5)])
def test_gemm_parity_small(M, K, N):
    say("gemm", M, K, N)
    w = synth.q4k_blocks(90, M, M, K)
    x16 = synth.activations_f16(90, N, N, K)
    y = _gemm(dev(w), x16, M, K)
    yr, S = oracle.gemm(oracle.Q4_K, w, x16, M, K)
    r = within(y, yr, S, TOL, "gemm %dx%dx%d" % (M, K, N))
    say("  max err/S", r)


def _with_fixed(g, fixed, size, n):
    """The fixed indices plus random others, n in all (sorted, distinct)."""
    fixed = np.unique(np.asarray(fixed, dtype=np.int64))
    others = np.setdiff1d(np.arange(size), fixed)
    extra = g.choice(others, max(0, n - fixed.size), replace=False)
    return np.sort(np.concatenate([fixed, extra]))


def sample_rows(g, M, n=512):
    """n rows: the first and last rows and both sides of the first 256-row
    tile boundaries, the rest at random."""
    edges = [r for t in range(256, M, 256)[:16] for r in (t - 1, t)]
    return _with_fixed(g, [0, M - 1] + edges, M, n)


def sample_tokens(g, N, n=16):
    """n tokens: the first and last and both sides of the first three
    256-token tile boundaries, the rest at random."""
    edges = [t for b in range(256, N, 256)[:3] for t in (b - 1, b)]
    return _with_fixed(g, [0, N - 1] + edges, N, n)


def check_prefill_sample(y, w, x16, M, K, N, g, fmt=oracle.Q4_K):
    """512 rows over all tokens and all rows over 16 tokens against the
    oracle (its matrix-product form)."""
    rows = sample_rows(g, M)
    yr, S = oracle.gemm_matmul(fmt, w, x16, M, K, rows=rows)
    r1 = within(y[:, rows], yr, S, TOL, "%d rows x all %d tokens" % (rows.size, N))
    toks = sample_tokens(g, N)
    yr2, S2 = oracle.gemm_matmul(fmt, w, x16, M, K, toks=toks)
    r2 = within(y[toks], yr2, S2, TOL, "all rows x %d tokens" % toks.size)
    return r1, r2


@pytest.mark.parametrize("M,K,N", [(14336, 4096, 512), (4096, 14336, 512),
                                   (14336, 4096, 4096), (4096, 14336, 4096)])
def test_gemm_parity_prefill_sampled(M, K, N):
    """Prefill shapes at full size: 512 rows over all tokens, and all rows
    over 16 tokens (tile edges included)."""
    say("gemm full", M, K, N)
    g = np.random.default_rng(91)
    w = synth.q4k_blocks(3, M, M, K)
    x16 = synth.activations_f16(3, N, N, K)
    y = _gemm(dev(w), x16, M, K)
    r1, r2 = check_prefill_sample(y, w, x16, M, K, N, g)
    say("  max err/S", r1, r2)


def test_gemm_parity_ragged_large_tiles():
    """The automatic dispatch on a shape with 17 x 16 = 272 tiles of 256 x 256
    (more than one round of the chip), ragged in weight rows (the last tile
    holds 156) and in tokens (4000 = 15 x 256 + 160): all rows over sampled
    tokens and all tokens over sampled rows, across tile boundaries."""
    M, K, N = 4252, 256, 4000
    say("gemm ragged large", M, K, N)
    g = np.random.default_rng(93)
    w = synth.q4k_blocks(95, M, M, K)
    x16 = synth.activations_f16(95, N, N, K)
    y = _gemm(dev(w), x16, M, K)
    toks = np.unique(np.concatenate([[0, 3839, 3840, N - 1], g.choice(N, 60, replace=False)]))
    yr, S = oracle.gemm(oracle.Q4_K, w, x16, M, K, toks=toks)
    r1 = within(y[toks], yr, S, TOL, "token sample")
    rows = np.unique(np.concatenate([[0, 4095, 4096, M - 1], g.choice(M, 60, replace=False)]))
    yr2, S2 = oracle.gemm(oracle.Q4_K, w, x16, M, K, rows=rows)
    r2 = within(y[:, rows], yr2, S2, TOL, "row sample")
    say("  max err/S", r1, r2)


def test_gemm_parity_pinned_small_tiles_128():
    """The LDS-tile kernel pinned at a shape with 576 tiles of 128 x 128, so
    that it runs its 128 x 128 instance, ragged in both dimensions (3000 is
    not a multiple of 128): all rows over sampled tokens and all tokens over
    sampled rows, across tile boundaries."""
    M, K, N = 3000, 256, 3000
    say("gemm pinned 64 / 128x128", M, K, N)
    g = np.random.default_rng(95)
    w = synth.q4k_blocks(94, M, M, K)
    x16 = synth.activations_f16(94, N, N, K)
    y = _gemm(dev(w), x16, M, K, 64)
    edges = np.array([0, 127, 128, 2943, 2944, 2999])
    toks = np.unique(np.concatenate([edges, g.choice(N, 40, replace=False)]))
    yr, S = oracle.gemm(oracle.Q4_K, w, x16, M, K, toks=toks)
    r1 = within(y[toks], yr, S, TOL, "128x128 token sample")
    rows = np.unique(np.concatenate([edges, g.choice(M, 40, replace=False)]))
    yr2, S2 = oracle.gemm(oracle.Q4_K, w, x16, M, K, rows=rows)
    r2 = within(y[:, rows], yr2, S2, TOL, "128x128 row sample")
    say("  max err/S", r1, r2)


@pytest.mark.parametrize("tile_rows", [256, 128, 64])
@pytest.mark.parametrize("M,K,N", [(256, 256, 256), (600, 1024, 520), (512, 2048, 300),
                                   (1000, 512, 1030), (130, 768, 37)])
def test_gemm_parity_pinned_tiles(M, K, N, tile_rows):
    """Each kernel family pinned through gq_gemm_q4k_tiles, at sizes the oracle
    computes in full: several tiles, ragged M and N (also fewer rows than one
    tile), the smallest K."""
    say("gemm tiles", tile_rows, M, K, N)
    w = synth.q4k_blocks(94, M, M, K)
    x16 = synth.activations_f16(94, N, N, K)
    y = _gemm(dev(w), x16, M, K, tile_rows)
    yr, S = oracle.gemm(oracle.Q4_K, w, x16, M, K)
    r = within(y, yr, S, TOL, "gemm %d-row tiles %dx%dx%d" % (tile_rows, M, K, N))
    say("  max err/S", r)


@pytest.mark.parametrize("tile_rows", [256, 128])
def test_gemm_one_hot_exact_large_tiles(tile_rows):
    """One-hot activation rows read out the binary16 weights exactly on the
    large-tile kernel, in every row of a ragged multi-tile output; the k of row
    i walks every position of a 64-weight step, so each lane and sub-step of
    the k permutation is checked."""
    M, K, N = 300, 1024, 270
    w = synth.q4k_blocks(95, 0, M, K)
    _, w16 = oracle.dequant(oracle.Q4_K, w, M, K)
    ks = (np.arange(N) * 37 + 5) % K
    x16 = np.zeros((N, K), np.float16)
    x16[np.arange(N), ks] = 1.0
    torch = torch_cuda()
    y = torch.empty((N, M), dtype=torch.float16, device="cuda")
    gq.gq_gemm_q4k_tiles(dev(w), dev(x16), y, M, K, N, tile_rows)
    yb = half_bits(y)
    for i, k in enumerate(ks):
        assert np.array_equal(yb[i].view(np.float16), w16[:, k].view(np.float16)), (i, k)


def test_gemm_one_hot_exact():
    M, K = 256, 1024
    w = synth.q4k_blocks(92, 0, M, K)
    _, w16 = oracle.dequant(oracle.Q4_K, w, M, K)
    ks = np.array([0, 1, 31, 32, 63, 64, 255, 256, 300, 511, 512, 700, 1023])
    x16 = np.zeros((ks.size, K), np.float16)
    x16[np.arange(ks.size), ks] = 1.0
    torch = torch_cuda()
    y = torch.empty((ks.size, M), dtype=torch.float16, device="cuda")
    gq.gq_gemm_q4k(dev(w), dev(x16), y, M, K, ks.size)
    yb = half_bits(y)
    for i, k in enumerate(ks):
        a = yb[i].view(np.float16)
        b = w16[:, k].view(np.float16)
        assert np.array_equal(a, b), k  # equal values (+0 and -0 compare equal)


@pytest.mark.parametrize("N", [200, 300])
def test_gemm_deterministic(N):
    M, K = 384, 2048
    w = dev(synth.q4k_blocks(93, 0, M, K))
    x16 = synth.activations_f16(93, 0, N, K)
    a = _gemm(w, x16, M, K)
    b = _gemm(w, x16, M, K)
    assert np.array_equal(a, b)


def _gemm_kg(w_d, x16, M, K, groups):
    torch = torch_cuda()
    N = x16.shape[0]
    y = torch.empty((N, M), dtype=torch.float16, device="cuda")
    y.fill_(float("nan"))
    gq.gq_gemm_q4k_kgroups(w_d, dev(x16), y, M, K, N, groups)
    return half_bits(y).view(np.float16).astype(np.float64)


@pytest.mark.parametrize("groups", [2, 4])
@pytest.mark.parametrize("M,K,N", [(200, 1024, 300), (1000, 2048, 260), (1, 1024, 5),
                                   (130, 4096, 37), (640, 1024, 1030)])
def test_gemm_kgroups_parity(M, K, N, groups):
    """K split across groups of waves inside each workgroup, at sizes the
    oracle computes in full: ragged weight rows (tiles of 64 or 128) and
    activation rows (tiles of 128), a single weight row, runs of K of one
    super-block per group (K = 1024 with four groups).  The output starts as
    NaN, so every element must be written."""
    say("gemm kgroups", groups, M, K, N)
    w = synth.q4k_blocks(99, M, M, K)
    x16 = synth.activations_f16(99, N, N, K)
    y = _gemm_kg(dev(w), x16, M, K, groups)
    yr, S = oracle.gemm(oracle.Q4_K, w, x16, M, K)
    r = within(y, yr, S, TOL, "gemm kgroups %d %dx%dx%d" % (groups, M, K, N))
    say("  max err/S", r)


@pytest.mark.parametrize("M,K,N,groups", [(4096, 14336, 512, 4), (4096, 14336, 1024, 2),
                                          (6144, 4096, 512, 2), (4096, 4096, 512, 4)])
def test_gemm_kgroups_prefill_sampled(M, K, N, groups):
    """Few-token prefill shapes at full size, where the automatic dispatch
    takes the K groups: gq_gemm_q4k equals the pinned group count bit for bit
    (the same kernel), and 512 rows over all tokens and all rows over 16
    tokens match the oracle."""
    say("gemm kgroups full", groups, M, K, N)
    g = np.random.default_rng(100)
    w = synth.q4k_blocks(3, M, M, K)
    x16 = synth.activations_f16(3, N, N, K)
    wd = dev(w)
    y = _gemm_kg(wd, x16, M, K, groups)
    assert np.array_equal(_gemm(wd, x16, M, K), y)
    r1, r2 = check_prefill_sample(y, w, x16, M, K, N, g)
    say("  max err/S", r1, r2)


@pytest.mark.parametrize("groups", [2, 4])
def test_gemm_kgroups_one_hot_exact(groups):
    """One-hot activation rows read out the binary16 weights exactly with K
    split in groups: the group whose run holds the one-hot k sums the weight
    exactly and the others add exact zeros.  The k of row i walks every
    position of a 64-weight step and every group's run."""
    M, K, N = 300, 1024, 270
    w = synth.q4k_blocks(101, 0, M, K)
    _, w16 = oracle.dequant(oracle.Q4_K, w, M, K)
    ks = (np.arange(N) * 37 + 5) % K
    x16 = np.zeros((N, K), np.float16)
    x16[np.arange(N), ks] = 1.0
    y = _gemm_kg(dev(w), x16, M, K, groups)
    for i, k in enumerate(ks):
        assert np.array_equal(y[i].astype(np.float16).view(np.uint16), w16[:, k]), (i, k)


@pytest.mark.parametrize("groups", [2, 4])
def test_gemm_kgroups_deterministic(groups):
    M, K, N = 384, 2048, 300
    w = dev(synth.q4k_blocks(102, 0, M, K))
    x16 = synth.activations_f16(102, 0, N, K)
    assert np.array_equal(_gemm_kg(w, x16, M, K, groups), _gemm_kg(w, x16, M, K, groups))


def _gemm_splitk(w_d, x16, M, K, splits):
    torch = torch_cuda()
    N = x16.shape[0]
    y = torch.empty((N, M), dtype=torch.float16, device="cuda")
    need = gq.gq_gemm_q4k_splitk_workspace_bytes(M, K, N, splits)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    gq.gq_gemm_q4k_splitk(w_d, dev(x16), y, M, K, N, splits, ws)
    return half_bits(y).view(np.float16).astype(np.float64)


@pytest.mark.parametrize("splits", [1, 2, 4])
@pytest.mark.parametrize("M,K,N", [(600, 1024, 300), (256, 1024, 256), (130, 2048, 37)])
def test_gemm_splitk_parity(M, K, N, splits):
    """Split-K product at sizes the oracle computes in full: ragged M and N,
    1, 2 and 4 runs of K."""
    say("gemm splitk", M, K, N, splits)
    w = synth.q4k_blocks(96, M, M, K)
    x16 = synth.activations_f16(96, N, N, K)
    y = _gemm_splitk(dev(w), x16, M, K, splits)
    yr, S = oracle.gemm(oracle.Q4_K, w, x16, M, K)
    r = within(y, yr, S, TOL, "gemm splitk %d %dx%dx%d" % (splits, M, K, N))
    say("  max err/S", r)


@pytest.mark.parametrize("M,K", [(4096, 14336), (14336, 4096)])
def test_gemm_splitk_prefill_sampled(M, K):
    """The 512-token prefill shapes at full size with the automatic split
    count: 512 rows over all tokens, all rows over 16 tokens."""
    N = 512
    say("gemm splitk full", M, K, N)
    g = np.random.default_rng(97)
    w = synth.q4k_blocks(3, M, M, K)
    x16 = synth.activations_f16(3, N, N, K)
    y = _gemm_splitk(dev(w), x16, M, K, 0)
    r1, r2 = check_prefill_sample(y, w, x16, M, K, N, g)
    say("  max err/S", r1, r2)


def test_gemm_splitk_one_hot_exact():
    """One-hot activation rows read out the binary16 weights exactly through
    the split form too: only one run holds the non-zero product, the others
    add exact zeros."""
    M, K = 256, 1024
    w = synth.q4k_blocks(98, 0, M, K)
    cols = [0, 255, 256, 700, 1023]
    x16 = np.zeros((len(cols), K), np.float16)
    for i, c in enumerate(cols):
        x16[i, c] = 1.0
    y = _gemm_splitk(dev(w), x16, M, K, 4)
    _, w16 = oracle.dequant(oracle.Q4_K, w, M, K)
    for i, c in enumerate(cols):
        assert np.array_equal(y[i].astype(np.float16).view(np.uint16), w16[:, c]), c


def _gemm_q8(w_d, x16, M, K):
    torch = torch_cuda()
    N = x16.shape[0]
    y = torch.empty((N, M), dtype=torch.float16, device="cuda")
    gq.gq_gemm_q8_0(w_d, dev(x16), y, M, K, N)
    return half_bits(y)


@pytest.mark.parametrize("M,K,N", [(128, 64, 1), (130, 192, 37), (300, 1088, 270),
                                   (1000, 1024, 520), (1700, 64, 2048), (3000, 64, 3000),
                                   (256, 1024, 128), (300, 2048, 200)])
def test_gemm_q8_0_parity(M, K, N):
    """Q8_0 product at sizes the oracle computes in full, across the tile
    families (N <= 64, 64 x 64, 64 x 128, 128 x 128), ragged M and N, the
    smallest K; the last two take K split across groups of waves (the
    automatic choice for few tiles and K % 256 == 0)."""
    say("gemm q8_0", M, K, N)
    w = synth.q8_0_blocks(97, M, M, K)
    x16 = synth.activations_f16(97, N, N, K)
    y = _gemm_q8(dev(w), x16, M, K).view(np.float16).astype(np.float64)
    yr, S = oracle.gemm(oracle.Q8_0, w, x16, M, K)
    r = within(y, yr, S, TOL, "gemm q8_0 %dx%dx%d" % (M, K, N))
    say("  max err/S", r)


def _gemm_q8_tiles(w_d, x16, M, K, tile_rows):
    torch = torch_cuda()
    N = x16.shape[0]
    y = torch.empty((N, M), dtype=torch.float16, device="cuda")
    gq.gq_gemm_q8_0_tiles(w_d, dev(x16), y, M, K, N, tile_rows)
    return half_bits(y)


@pytest.mark.parametrize("M,K,N,tile_rows", [(300, 512, 270, 256), (520, 256, 600, 128),
                                             (1000, 1024, 300, 256), (130, 768, 257, 128)])
def test_gemm_q8_0_large_tiles_parity(M, K, N, tile_rows):
    """Q8_0 on the large-tile kernel (pinned), at sizes the oracle computes in
    full: several tiles, ragged M and N, K of one to four runs of 256."""
    say("gemm q8_0 large tiles", M, K, N, tile_rows)
    w = synth.q8_0_blocks(96, M, M, K)
    x16 = synth.activations_f16(96, N, N, K)
    y = _gemm_q8_tiles(dev(w), x16, M, K, tile_rows).view(np.float16).astype(np.float64)
    yr, S = oracle.gemm(oracle.Q8_0, w, x16, M, K)
    r = within(y, yr, S, TOL, "gemm q8_0 tiles %d %dx%dx%d" % (tile_rows, M, K, N))
    say("  max err/S", r)


def test_gemm_q8_0_one_hot_exact_and_special_blocks():
    """One-hot activation rows read out the binary16 weights binary16(d*q)
    exactly, on random blocks and on hand-set ones: q = -128, a negative
    scale, a binary16 subnormal scale, d = 0.  Compared as values: d = 0 with
    a negative quant is the weight -0, which a sum that starts from +0 reads
    out as +0 (every other binary16 value compares equal only bit for bit)."""
    M, K, N = 130, 256, 70
    w = synth.q8_0_blocks(98, 0, M, K).reshape(M, K // 32, 34)
    w[0, 0, 0:2] = np.array([1.0], "<f2").view(np.uint8)
    w[0, 0, 2:] = np.uint8(0x80)                                    # q = -128, d = 1
    w[1, 3, 0:2] = np.array([-0.5], "<f2").view(np.uint8)           # negative d
    w[2, 5, 0:2] = np.array([2.0 ** -20], "<f2").view(np.uint8)     # subnormal d
    w[3, 7, 0:2] = 0                                                # d = 0
    w = w.reshape(-1)
    _, w16 = oracle.dequant(oracle.Q8_0, w, M, K)
    ks = (np.arange(N) * 37 + 3) % K
    ks[:4] = [0, 3 * 32 + 5, 5 * 32 + 31, 7 * 32]
    x16 = np.zeros((N, K), np.float16)
    x16[np.arange(N), ks] = 1.0
    for tile_rows in (64, 128, 256):
        yb = _gemm_q8_tiles(dev(w), x16, M, K, tile_rows)
        for i, k in enumerate(ks):
            assert np.array_equal(yb[i].view(np.float16), w16[:, k].view(np.float16)), \
                (tile_rows, i, k)
        assert yb[0].view(np.float16)[0] == -128.0


def test_gemm_q8_0_prefill_sampled():
    """Q8_0 at a prefill shape, 14336 x 4096 weights and 512 tokens: 512 rows
    over all tokens and all rows over 16 tokens."""
    M, K, N = 14336, 4096, 512
    say("gemm q8_0 full", M, K, N)
    g = np.random.default_rng(99)
    w = synth.q8_0_blocks(3, M, M, K)
    x16 = synth.activations_f16(3, N, N, K)
    y = _gemm_q8(dev(w), x16, M, K).view(np.float16).astype(np.float64)
    r1, r2 = check_prefill_sample(y, w, x16, M, K, N, g, fmt=oracle.Q8_0)
    say("  max err/S", r1, r2)
