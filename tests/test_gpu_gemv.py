"""Parity of the fused dequant matrix-vector products with the binary64 oracle.

Bound: |y_gpu - y_ref| <= 1e-5 * S with S = sum_k |w_k x_k| (binary32
accumulation; the oracle sums in binary64).  One-hot activations must read
out the binary32 weights exactly.
"""
import numpy as np
import pytest

import oracle
from quantized_unpack_q4_amd import gq, synth
from tests._gpu import dev, host, say, torch_cuda, within

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _gemv(fmt, w_d, x, M, K):
    torch = torch_cuda()
    xd = dev(x)
    y = torch.empty((x.shape[0], M), dtype=torch.float32, device="cuda")
    if fmt == "q4k":
        gq.gq_gemv_q4k(w_d, xd, y, M, K, x.shape[0])
    else:
        gq.gq_gemv_q8_0(w_d, xd, y, M, K, x.shape[0])
    return host(y)


# -- Q8_0 ------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,B", [(256, 1024, 1), (1, 32, 1), (7, 96, 3), (33, 160, 16),
                                   (130, 2048, 2), (8195, 96, 1), (8195, 128, 1), (77, 14336, 1),
                                   (8200, 256, 1), (3, 16384, 1)])
def test_q8_0_parity(M, K, B):
    say("q8_0 gemv", M, K, B)
    w = synth.q8_0_blocks(80, M, M, K)
    x = synth.activations_f32(80, M, B, K)
    y = _gemv("q8_0", dev(w), x, M, K)
    yr, S = oracle.gemv(oracle.Q8_0, w, x, M, K)
    r = within(y, yr, S, TOL, "q8_0 %dx%d B=%d" % (M, K, B))
    say("  max err/S", r)


def test_q8_0_one_hot_exact():
    M, K = 19, 320
    w = synth.q8_0_blocks(81, 0, M, K)
    w32, _ = oracle.dequant(oracle.Q8_0, w, M, K)
    ks = [0, 1, 31, 32, 33, 100, 255, K - 1]
    x = np.zeros((len(ks), K), np.float32)
    for b, k in enumerate(ks):
        x[b, k] = 1.0
    y = _gemv("q8_0", dev(w), x, M, K)
    for b, k in enumerate(ks):
        assert np.array_equal(y[b], w32[:, k]), k


@pytest.mark.parametrize("M,K,B", [(1, 64, 2), (17, 128, 5), (100, 4096, 16), (61, 14336, 3),
                                   (333, 1024, 8), (12300, 256, 7), (8200, 192, 3),
                                   (4100, 1088, 4), (8200, 320, 12), (12300, 320, 4),
                                   (12400, 128, 3)])
def test_q8_0_matrix_core_ragged(M, K, B):
    """Batch 2..16 with K % 64 == 0 (the matrix-core kernel): rows that leave a
    partial 16-row group (12300 rows: a partial 32-row group of the two-tile
    form; 8200 and 4100 rows: the one-tile form with eight waves), K from one
    pair of blocks to the maximum and pair counts that leave the last chunk of
    staged weights partial (3, 5 and 17 pairs), batch sizes on the 16x16x4
    product and on both 4x4x1 layouts (batch 2 and 3 on two-tile launches:
    groups; batch 4, and 3 on one-tile launches: slices), and activation rows
    scaled from 1e-30 to 1e30 plus an all-zero row."""
    say("q8_0 mfma gemv", M, K, B)
    w = synth.q8_0_blocks(83, M, M, K)
    x = synth.activations_f32(83, M + B, B, K)
    scales = np.array([1e-30, 1e-8, 1.0, 3e4, 1e12, 1e30, 0.0, 7.0] * 2, np.float32)[:B]
    x = (x * scales[:, None]).astype(np.float32)
    y = _gemv("q8_0", dev(w), x, M, K)
    yr, S = oracle.gemv(oracle.Q8_0, w, x, M, K)
    r = within(y, yr, S, TOL, "q8_0 mfma %dx%d B=%d" % (M, K, B))
    if B > 6:
        assert np.all(y[6] == 0)
    say("  max err/S", r)


@pytest.mark.parametrize("M,K,B", [(14336, 4096, 16), (4096, 14336, 4), (11008, 4096, 2),
                                   (14336, 4096, 4)])
def test_q8_0_matrix_core_full_size_sampled(M, K, B):
    """Decode shapes at batch 2, 4 and 16 (every launch form of the kernel), 64
    sampled rows, and the same bits on a second call."""
    torch = torch_cuda()
    say("q8_0 mfma gemv full", M, K, B)
    w = synth.q8_0_blocks(84, M, M, K)
    x = synth.activations_f32(84, M, B, K)
    wd, xd = dev(w), dev(x)
    y = torch.empty((B, M), dtype=torch.float32, device="cuda")
    gq.gq_gemv_q8_0(wd, xd, y, M, K, B)
    y1 = host(y).copy()
    gq.gq_gemv_q8_0(wd, xd, y, M, K, B)
    assert np.array_equal(y1.view(np.uint32), host(y).view(np.uint32))
    g = np.random.default_rng(84)
    rows = np.sort(g.choice(M, 64, replace=False))
    rows[0], rows[-1] = 0, M - 1
    yr, S = oracle.gemv(oracle.Q8_0, w, x, M, K, rows=rows)
    say("  max err/S", within(y1[:, rows], yr, S, TOL, "q8_0 mfma full %dx%d" % (M, K)))


def test_q8_0_batch1_one_hot_exact():
    """Batch 1: a one-hot activation reads out the binary32 weight d * q
    exactly, on a tall matrix (four rows per wave) and short ones (two)."""
    torch = torch_cuda()
    for M, K in ((9000, 128), (19, 320), (40, 512), (17, 4096)):
        w = synth.q8_0_blocks(85, M, M, K)
        w32, _ = oracle.dequant(oracle.Q8_0, w, M, K)
        wd = dev(w)
        y = torch.empty((1, M), dtype=torch.float32, device="cuda")
        for k in (0, 1, 31, 32, 33, 63, 64, K - 1):
            x = np.zeros((1, K), np.float32)
            x[0, k] = 1.0
            gq.gq_gemv_q8_0(wd, dev(x), y, M, K, 1)
            assert np.array_equal(host(y)[0], w32[:, k]), (M, K, k)


# -- Q4_K ------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,B", [(1, 256, 1), (37, 1024, 1), (5, 512, 2), (131, 2048, 3),
                                   (64, 4096, 4), (29, 14336, 1), (100, 768, 7), (48, 4096, 16),
                                   (17, 256, 16)])
def test_q4k_parity_small(M, K, B):
    say("q4k gemv", M, K, B)
    w = synth.q4k_blocks(82, M, M, K)
    x = synth.activations_f32(82, M + B, B, K)
    y = _gemv("q4k", dev(w), x, M, K)
    yr, S = oracle.gemv(oracle.Q4_K, w, x, M, K)
    r = within(y, yr, S, TOL, "q4k %dx%d B=%d" % (M, K, B))
    say("  max err/S", r)


@pytest.mark.parametrize("M,K", [(4096, 4096), (14336, 4096)])
def test_q4k_parity_full_single_matrix(M, K):
    """Batch-1 matrix-vector product at the decode shapes, every row checked."""
    say("q4k gemv full", M, K)
    w = synth.q4k_blocks(1, M, M, K)
    x = synth.activations_f32(1, M, 1, K)
    y = _gemv("q4k", dev(w), x, M, K)
    yr, S = oracle.gemv(oracle.Q4_K, w, x, M, K)
    r = within(y, yr, S, TOL, "q4k full %dx%d" % (M, K))
    say("  max err/S", r)


@pytest.mark.parametrize("M,K,B", [(12300, 768, 2), (8200, 1280, 2), (4100, 256, 3),
                                   (1000, 4352, 12), (300, 8448, 3), (8000, 512, 4),
                                   (9000, 512, 4), (12200, 768, 3)])
def test_q4k_batched_single_ragged(M, K, B):
    """Single products at batch 2..16 on the binary32 matrix-core form (batch
    2, batch 3-4 below 12288 rows, or at most 32 rows per CU): each launch
    form (two 16-row tiles of eight
    waves at 12300 rows, one tile of eight waves at 8200 and 4100, one of
    sixteen at 1000 and 300; the 16x16x4 product and both 4x4x1 layouts: by
    4-row groups, and by 4-weight slices at batch 4 and at batch 3 with K of
    8192 or more) with a partial last 32- or 16-row group and a partial last
    chunk of staged super-blocks (12, 20, 4, 68, 132 and 8 units of 64
    weights), activation rows scaled from 1e-30 to 1e30 plus an all-zero
    row."""
    say("q4k batched single", M, K, B)
    w = synth.q4k_blocks(86, M, M, K)
    x = synth.activations_f32(86, M + B, B, K)
    scales = np.array([1e-30, 1e-8, 1.0, 3e4, 1e12, 1e30, 0.0, 7.0] * 2, np.float32)[:B]
    x = (x * scales[:, None]).astype(np.float32)
    y = _gemv("q4k", dev(w), x, M, K)
    yr, S = oracle.gemv(oracle.Q4_K, w, x, M, K)
    say("  max err/S", within(y, yr, S, TOL, "q4k batched %dx%d B=%d" % (M, K, B)))
    if B > 6:
        assert np.all(y[6] == 0)


@pytest.mark.parametrize("M,K,B", [(14336, 4096, 2), (4096, 14336, 4), (11008, 4096, 2),
                                   (4096, 4096, 16), (14336, 4096, 16), (11008, 4096, 4)])
def test_q4k_batched_single_full_size_sampled(M, K, B):
    """Decode shapes at batch 2..16 as single products (the binary32 form at
    batch 2 and up to 32 rows per CU, the split-activation kernel for 14336
    rows at batch 16), 64 sampled rows, and the same bits on a second call."""
    torch = torch_cuda()
    say("q4k batched single full", M, K, B)
    w = synth.q4k_blocks(87, M, M, K)
    x = synth.activations_f32(87, M, B, K)
    wd, xd = dev(w), dev(x)
    y = torch.empty((B, M), dtype=torch.float32, device="cuda")
    gq.gq_gemv_q4k(wd, xd, y, M, K, B)
    y1 = host(y).copy()
    gq.gq_gemv_q4k(wd, xd, y, M, K, B)
    assert np.array_equal(y1.view(np.uint32), host(y).view(np.uint32))
    g = np.random.default_rng(87)
    rows = np.sort(g.choice(M, 64, replace=False))
    rows[0], rows[-1] = 0, M - 1
    yr, S = oracle.gemv(oracle.Q4_K, w, x, M, K, rows=rows)
    say("  max err/S", within(y1[:, rows], yr, S, TOL, "q4k batched full %dx%d" % (M, K)))


def test_q4k_one_hot_exact():
    M, K = 45, 1024
    w = synth.q4k_blocks(83, 0, M, K)
    w32, _ = oracle.dequant(oracle.Q4_K, w, M, K)
    ks = [0, 15, 31, 32, 63, 64, 100, 255, 256, 511, 600, 777, 900, 1000, 1022, 1023]
    x = np.zeros((len(ks), K), np.float32)
    for b, k in enumerate(ks):
        x[b, k] = 1.0
    for B in (1, 4, 16):
        y = _gemv("q4k", dev(w), np.ascontiguousarray(x[:B]), M, K)
        for b in range(B):
            assert np.array_equal(y[b], w32[:, ks[b]]), (B, ks[b])


def test_q4k_deterministic_and_zero_weights():
    M, K, B = 300, 4096, 4
    w = synth.q4k_blocks(84, 0, M, K)
    x = synth.activations_f32(84, 0, B, K)
    wd = dev(w)
    y1 = _gemv("q4k", wd, x, M, K)
    y2 = _gemv("q4k", wd, x, M, K)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    # d = dmin = 0 everywhere: outputs are exactly zero
    wz = w.reshape(-1, 144).copy()
    wz[:, 0:4] = 0
    yz = _gemv("q4k", dev(wz.reshape(-1)), x, M, K)
    assert np.all(yz == 0)


def test_q4k_decode_stack_layer_sampled():
    """One layer of the Llama-3-8B-shaped decode stack at full size, batch 1, 4
    and 16, the same launches the benchmark times; sampled rows vs the oracle."""
    torch = torch_cuda()
    shapes = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
              ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336)]
    g = np.random.default_rng(85)
    for t, (name, M, K) in enumerate(shapes):
        w = synth.q4k_blocks(2, t, M, K)
        wd = dev(w)
        rows = np.sort(g.choice(M, 48, replace=False))
        rows[0], rows[-1] = 0, M - 1
        for B in (1, 4, 16):
            say("stack layer", name, M, K, "B", B)
            x = synth.activations_f32(2, 100 * t + B, B, K)
            y = _gemv("q4k", wd, x, M, K)
            yr, S = oracle.gemv(oracle.Q4_K, w, x, M, K, rows=rows)
            within(y[:, rows], yr, S, TOL, "%s B=%d" % (name, B))
        del wd
        torch.cuda.empty_cache()
