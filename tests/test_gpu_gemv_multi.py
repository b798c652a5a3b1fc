"""Parity of the one-launch batch-1 multi-product (and of the single-matrix
batch-1 product, which runs the same streaming kernel) with the oracle.

Bound: |y - y_ref| <= 1e-5 * S per output.  Activations are split into two
binary16 halves after a power-of-two scaling, so inputs of very different
magnitudes are part of the check.
"""
import numpy as np
import pytest

import oracle
from quantized_unpack_q4_amd import gq, synth
from tests._gpu import dev, host, say, torch_cuda, within

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _table(shapes, workload, xscale=None):
    torch = torch_cuda()
    items, host_in = [], []
    for i, (M, K) in enumerate(shapes):
        w = synth.q4k_blocks(workload, i, M, K)
        x = synth.activations_f32(workload, i, 1, K)
        if xscale is not None:
            x = (x * np.float32(xscale[i])).astype(np.float32)
        y = torch.full((1, M), float("nan"), dtype=torch.float32, device="cuda")
        items.append((dev(w), dev(x), y, M, K))
        host_in.append((w, x))
    return gq.GemvTable(items), host_in


def _check(table, host_in, shapes, rows_cap=None, what=""):
    worst = 0.0
    g = np.random.default_rng(5)
    for (w, x), (_, _, y, M, K), (M2, K2) in zip(host_in, table.items, shapes):
        yg = host(y)
        # outputs start as NaN: every row must be written by exactly the
        # workgroup whose byte range holds its first byte
        assert np.isfinite(yg).all(), "%s %dx%d: rows %s not written" % (
            what, M, K, np.argwhere(~np.isfinite(yg))[:5, -1].tolist())
        rows = None
        if rows_cap is not None and M > rows_cap:
            rows = np.sort(g.choice(M, rows_cap, replace=False))
            rows[0], rows[-1] = 0, M - 1
        yr, S = oracle.gemv(oracle.Q4_K, w, x, M, K, rows=rows)
        got = yg if rows is None else yg[:, rows]
        worst = max(worst, within(got, yr, S, TOL, "%s %dx%d" % (what, M, K)))
    return worst


def test_multi_mixed_shapes():
    """Ragged rows, every K from one super-block up to the maximum, tables whose
    byte ranges split inside matrices and across them."""
    shapes = [(1, 256), (37, 1024), (24, 4096), (25, 4096), (100, 768), (5, 16384),
              (300, 2048), (49, 14336), (7, 256), (1024, 4096)]
    t, h = _table(shapes, 20)
    t.run()
    r = _check(t, h, shapes, what="mixed")
    say("multi mixed max err/S", r)


def test_multi_activation_magnitudes():
    """Per-matrix activation scales from 1e-30 to 1e30, and zero vectors."""
    shapes = [(64, 1024)] * 6
    scales = [1e-30, 1e-8, 1.0, 3e4, 1e12, 1e30]
    t, h = _table(shapes, 21, xscale=scales)
    t.run()
    r = _check(t, h, shapes, what="scaled")
    say("multi scaled max err/S", r)
    z, hz = _table([(40, 512)], 22, xscale=[0.0])
    z.run()
    assert np.all(host(z.items[0][2]) == 0)


def test_multi_one_hot_exact_and_deterministic():
    torch = torch_cuda()
    M, K = 77, 4096
    w = synth.q4k_blocks(23, 0, M, K)
    w32, _ = oracle.dequant(oracle.Q4_K, w, M, K)
    wd = dev(w)
    ks = [0, 31, 32, 63, 100, 255, 256, 1000, 2047, 4095]
    items = []
    for k in ks:
        x = np.zeros((1, K), np.float32)
        x[0, k] = 1.0
        items.append((wd, dev(x), torch.empty((1, M), dtype=torch.float32, device="cuda"), M, K))
    t = gq.GemvTable(items)
    t.run()
    for k, it in zip(ks, items):
        assert np.array_equal(host(it[2])[0], w32[:, k]), k
    first = [host(it[2]).copy() for it in items]
    t.run()
    for a, it in zip(first, items):
        assert np.array_equal(a.view(np.uint32), host(it[2]).view(np.uint32))


def test_multi_decode_layer_full_size():
    """One Llama-3-8B-shaped layer (q, k, v, o, gate, up, down) at full size in
    one launch, with the generator streams the benchmark uses; sampled rows."""
    shapes = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096), (14336, 4096),
              (14336, 4096), (4096, 14336)]
    torch = torch_cuda()
    items, host_in = [], []
    for t, (M, K) in enumerate(shapes):
        w = synth.q4k_blocks(2, t, M, K)
        x = synth.activations_f32(2, 100 * t + 1, 1, K)
        items.append((dev(w), dev(x), torch.empty((1, M), dtype=torch.float32, device="cuda"),
                      M, K))
        host_in.append((w, x))
    tab = gq.GemvTable(items)
    tab.run()
    r = _check(tab, host_in, shapes, rows_cap=64, what="layer")
    say("multi layer max err/S", r)


def test_multi_tensor_parallel_share():
    """Two layers of one GPU's 8-way tensor-parallel share (q/k/v/gate/up by
    rows, o and down by K): thousands of 288-byte rows (K = 512) among long
    ones, where the work split counts a row as at least a fixed cost; every
    row written once, sampled rows against the oracle."""
    shapes = [(512, 4096), (128, 4096), (128, 4096), (4096, 512), (1792, 4096), (1792, 4096),
              (4096, 1792)] * 2
    t, h = _table(shapes, 25)
    t.run()
    r = _check(t, h, shapes, rows_cap=64, what="tp share")
    say("multi tp share max err/S", r)


def test_single_matrix_batch1_large_k_and_ragged():
    """The single-matrix entry point at batch 1 (same streaming kernel)."""
    torch = torch_cuda()
    for M, K in ((1, 16384), (333, 256), (61, 14336)):
        w = synth.q4k_blocks(24, M, M, K)
        x = synth.activations_f32(24, M, 1, K)
        y = torch.empty((1, M), dtype=torch.float32, device="cuda")
        gq.gq_gemv_q4k(dev(w), dev(x), y, M, K, 1)
        yr, S = oracle.gemv(oracle.Q4_K, w, x, M, K)
        within(host(y), yr, S, TOL, "single %dx%d" % (M, K))


# -- batches 2..16 (matrix cores) ---------------------------------------------------

def _table_b(shapes, workload, B, xrow_scale=None):
    torch = torch_cuda()
    items, host_in = [], []
    for i, (M, K) in enumerate(shapes):
        w = synth.q4k_blocks(workload, i, M, K)
        x = synth.activations_f32(workload, 1000 + i, B, K)
        if xrow_scale is not None:
            x = (x * np.asarray(xrow_scale[i], np.float32)[:, None]).astype(np.float32)
        y = torch.full((B, M), float("nan"), dtype=torch.float32, device="cuda")
        items.append((dev(w), dev(x), y, M, K))
        host_in.append((w, x))
    return gq.GemvTable(items, batch=B), host_in


@pytest.mark.parametrize("B", [2, 5, 16])
def test_multi_batched_mixed_shapes(B):
    """Ragged row counts (partial 16-row tiles and 128-row blocks), K from one
    super-block to the maximum, block ranges that split across matrices."""
    shapes = [(1, 256), (37, 1024), (130, 4096), (100, 768), (5, 16384), (300, 2048),
              (49, 14336), (7, 256), (1024, 4096)]
    t, h = _table_b(shapes, 30, B)
    t.run()
    say("multi batched B", B)
    r = _check(t, h, shapes, what="batched B=%d" % B)
    say("  max err/S", r)


def test_multi_batched_activation_magnitudes():
    """Activation rows of one batch at very different magnitudes (each row and
    super-block gets its own power-of-two scale), and an all-zero row."""
    shapes = [(64, 1024), (40, 2048)]
    scales = [[1e-30, 1e-8, 1.0, 3e4, 1e12, 1e30], [0.0, 1.0, 1e-20, 1e20, 7.0, 0.5]]
    t, h = _table_b(shapes, 31, 6, xrow_scale=scales)
    t.run()
    r = _check(t, h, shapes, what="batched scaled")
    assert np.all(host(t.items[1][2])[0] == 0)
    say("multi batched scaled max err/S", r)


def test_multi_batched_one_hot_exact_and_deterministic():
    """One-hot activation rows read out the binary32 weights exactly."""
    torch = torch_cuda()
    M, K, B = 150, 2048, 16
    w = synth.q4k_blocks(32, 0, M, K)
    w32, _ = oracle.dequant(oracle.Q4_K, w, M, K)
    wd = dev(w)
    items, kss = [], []
    for rep in range(3):
        ks = [(37 * b + 101 * rep + 5) % K for b in range(B)]
        x = np.zeros((B, K), np.float32)
        x[np.arange(B), ks] = 1.0
        items.append((wd, dev(x), torch.empty((B, M), dtype=torch.float32, device="cuda"), M, K))
        kss.append(ks)
    t = gq.GemvTable(items, batch=B)
    t.run()
    for ks, it in zip(kss, items):
        y = host(it[2])
        for b, k in enumerate(ks):
            assert np.array_equal(y[b], w32[:, k]), (b, k)
    first = [host(it[2]).copy() for it in items]
    t.run()
    for a, it in zip(first, items):
        assert np.array_equal(a.view(np.uint32), host(it[2]).view(np.uint32))


@pytest.mark.parametrize("B", [4, 16])
def test_multi_batched_decode_layer_full_size(B):
    """One Llama-3-8B-shaped layer at full size in one launch, batch 4 and 16,
    with the generator streams the benchmark uses; sampled rows."""
    shapes = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096), (14336, 4096),
              (14336, 4096), (4096, 14336)]
    torch = torch_cuda()
    items, host_in = [], []
    for t, (M, K) in enumerate(shapes):
        w = synth.q4k_blocks(2, t, M, K)
        x = synth.activations_f32(2, 100 * t + B, B, K)
        items.append((dev(w), dev(x), torch.empty((B, M), dtype=torch.float32, device="cuda"),
                      M, K))
        host_in.append((w, x))
    tab = gq.GemvTable(items, batch=B)
    tab.run()
    r = _check(tab, host_in, shapes, rows_cap=48, what="layer B=%d" % B)
    say("multi batched layer B=%d max err/S" % B, r)


@pytest.mark.parametrize("M,K", [(1, 256), (300, 1024), (1000, 768), (37, 14336), (14336, 4096)])
def test_gemv_swiglu(M, K):
    """Gate and up products with the SwiGLU epilogue in one launch: every
    output against h = silu(g) * u from the oracle's binary64 products.
    Bound: the 1e-5 * S bounds of g and u carried through silu(g) * u
    (|silu'| <= 1.1), plus the binary32 epilogue: the exponential's argument
    rounds once (|g| * 2^-24 relative in e^-g) and exp, the division and the
    product add a few ulp, (4 + |g|) * 2^-23 relative in all."""
    torch = torch_cuda()
    say("swiglu", M, K)
    wg = synth.q4k_blocks(52, 2 * M, M, K)
    wu = synth.q4k_blocks(52, 2 * M + 1, M, K)
    x = synth.activations_f32(52, M, 1, K)
    h = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    gq.gq_gemv_q4k_swiglu(dev(wg), dev(wu), dev(x), h, M, K)
    hg = host(h).astype(np.float64)
    g, Sg = oracle.gemv(oracle.Q4_K, wg, x, M, K)
    u, Su = oracle.gemv(oracle.Q4_K, wu, x, M, K)
    g, Sg, u, Su = g[0], Sg[0], u[0], Su[0]
    hr = oracle.swiglu(g, u)
    sg = oracle.swiglu(g, np.ones_like(g))
    bound = TOL * (1.1 * Sg * np.abs(u) + np.abs(sg) * Su) + (4 + np.abs(g)) * 2.0 ** -23 * np.abs(hr)
    err = np.abs(hg - hr)
    assert np.isfinite(hg).all()
    assert np.all(err <= bound), "swiglu %dx%d: worst %.3g of bound" % (M, K, (err / bound).max())
    say("  worst err/bound", (err / bound).max())


@pytest.mark.parametrize("B", [2, 5, 16])
@pytest.mark.parametrize("M,K", [(1, 256), (300, 1024), (37, 14336), (14336, 4096)])
def test_gemv_swiglu_batched(M, K, B):
    """Gate and up products with the SwiGLU epilogue at batch 2-16 in one
    launch on the matrix cores (blocks of 64 output rows, each pairing 64 gate
    rows with the same up rows; ragged M, a single row): every output of
    every activation row against the oracle, with the bound of the batch-1
    test.  The output starts as NaN, so every element must be written."""
    torch = torch_cuda()
    say("swiglu batched", M, K, B)
    wg = synth.q4k_blocks(53, 2 * M, M, K)
    wu = synth.q4k_blocks(53, 2 * M + 1, M, K)
    x = synth.activations_f32(53, M, B, K)
    h = torch.full((B, M), float("nan"), dtype=torch.float32, device="cuda")
    gq.gq_gemv_q4k_swiglu_batched(dev(wg), dev(wu), dev(x), h, M, K, B)
    hg = host(h).astype(np.float64)
    g, Sg = oracle.gemv(oracle.Q4_K, wg, x, M, K)
    u, Su = oracle.gemv(oracle.Q4_K, wu, x, M, K)
    hr = oracle.swiglu(g, u)
    sg = oracle.swiglu(g, np.ones_like(g))
    bound = TOL * (1.1 * Sg * np.abs(u) + np.abs(sg) * Su) + (4 + np.abs(g)) * 2.0 ** -23 * np.abs(hr)
    err = np.abs(hg - hr)
    assert np.isfinite(hg).all()
    assert np.all(err <= bound), "swiglu B=%d %dx%d: worst %.3g of bound" % (
        B, M, K, (err / bound).max())
    say("  worst err/bound", (err / bound).max())


@pytest.mark.parametrize("B", [2, 3, 8, 16])
def test_multi_batched_prestaged(B):
    """Batch 2-16 tables with the activations staged once per product into a
    workspace (gq_gemv_q4k_multi_batched_ws), on ragged shapes (a single row,
    one super-block, 14336-long rows, 2000 rows): bit-identical to the
    per-block staging and within 1e-5 * S of the oracle on sampled rows; the
    workspace starts as all-ones bytes and the outputs as NaN."""
    torch = torch_cuda()
    shapes = [(1, 256), (130, 1024), (2000, 4096), (64, 14336), (777, 768), (4096, 512)]
    g = np.random.default_rng(500 + B)
    it1, it2, host_in = [], [], []
    for i, (M, K) in enumerate(shapes):
        w = synth.q4k_blocks(56, 10 * i + B, M, K)
        x = synth.activations_f32(56, 10 * i + B, B, K)
        wd, xd = dev(w), dev(x)
        it1.append((wd, xd, torch.full((B, M), float("nan"), dtype=torch.float32, device="cuda"), M, K))
        it2.append((wd, xd, torch.full((B, M), float("nan"), dtype=torch.float32, device="cuda"), M, K))
        host_in.append((w, x))
    t1 = gq.GemvTable(it1, batch=B)
    t2 = gq.GemvTable(it2, batch=B, prestaged=True)
    t2.ws.fill_(255)
    t1.run()
    t2.run()
    worst = 0.0
    for (M, K), a, b, (w, x) in zip(shapes, it1, it2, host_in):
        ya, yb = host(a[2]), host(b[2])
        assert np.isfinite(yb).all(), (M, K, B)
        assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32)), (M, K, B)
        rows = np.unique(np.concatenate([[0, M - 1], g.choice(M, min(M, 6), replace=False)]))
        rb = K // 256 * 144
        yr, S = oracle.gemv(oracle.Q4_K, w.reshape(M, rb)[rows].reshape(-1), x, rows.size, K)
        worst = max(worst, within(yb[:, rows], yr, S, TOL, "prestaged %dx%d B=%d" % (M, K, B)))
    say("prestaged B=%d max err/S" % B, worst)
