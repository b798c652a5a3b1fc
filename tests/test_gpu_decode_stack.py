"""The decode step exactly as the benchmark times it: the 224 products of a
Llama-3-8B-shaped stack (32 layers x q, k, v, o 4096-row; k, v 1024-row;
gate, up 14336 x 4096; down 4096 x 14336; 3,925,868,544 bytes of Q4_K
weights) planned as one table and run by one launch, with the benchmark's
generator streams, at batch 1 (the streaming kernel on its grid of two
workgroups per CU, each walking several matrices) and at batch 4 and 16 (the
matrix-core kernel on its full grid, workgroups crossing matrix boundaries).

Every output starts as NaN and must be written; eight rows of every product
(its first and last and six at random) are checked against the oracle with
|y - y_ref| <= 1e-5 * S.
"""
import numpy as np
import pytest

import oracle
from quantized_unpack_q4_amd import gq, synth
from tests._gpu import host, say, torch_cuda, within

pytestmark = pytest.mark.gpu

TOL = 1e-5
LAYER = (("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
         ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336))
N_LAYERS = 32
WORKLOAD = 2  # the benchmark's generator streams for the decode stack


@pytest.fixture(scope="module")
def stack():
    torch = torch_cuda()
    g = np.random.default_rng(11)
    mats = []
    total = 0
    for layer in range(N_LAYERS):
        for i, (name, M, K) in enumerate(LAYER):
            t = layer * len(LAYER) + i
            w = synth.q4k_blocks(WORKLOAD, t, M, K)
            rb = K // 256 * 144
            rows = np.array(sorted({0, M - 1} | set(g.choice(M, 6, replace=False).tolist())))
            wrows = w.reshape(M, rb)[rows].copy()
            mats.append((name, M, K, t, torch.from_numpy(w).cuda(), rows, wrows))
            total += w.size
            del w
    say("decode stack: %d products, %d weight bytes" % (len(mats), total))
    assert total == 3925868544
    yield mats
    del mats
    torch.cuda.empty_cache()


def _table_header(tab):
    h = np.frombuffer(bytes(tab.host)[:40], dtype=np.int64)
    return {"n": int(h[1]), "bytes": int(h[2]), "tiles": int(h[3]), "work": int(h[4])}


@pytest.mark.parametrize("B", [1, 4, 16])
def test_decode_stack_as_timed(stack, B):
    torch = torch_cuda()
    say("decode stack batch", B)
    items, xs = [], []
    for name, M, K, t, wd, rows, wrows in stack:
        x = synth.activations_f32(WORKLOAD, 100 * t + B, B, K)
        y = torch.full((B, M), float("nan"), dtype=torch.float32, device="cuda")
        items.append((wd, torch.from_numpy(x).cuda(), y, M, K))
        xs.append(x)
    tab = gq.GemvTable(items, batch=B)
    hd = _table_header(tab)
    assert hd["n"] == 224 and hd["bytes"] == 3925868544
    # the launch shapes the benchmark times: batch 1 takes two workgroups
    # per CU from 2^28 bytes of work up; the matrix-core kernel's 128-row
    # blocks (3,008 of them) exceed its 2 x CU grid
    if B == 1:
        assert hd["work"] >= 1 << 28
    tab.run()
    worst = 0.0
    for (name, M, K, t, wd, rows, wrows), x, it in zip(stack, xs, items):
        yg = host(it[2])
        bad = ~np.isfinite(yg)
        assert not bad.any(), "product %d (%s) B=%d: %d outputs not written, first at %s" % (
            t, name, B, int(bad.sum()), np.argwhere(bad)[0].tolist())
        yr, S = oracle.gemv(oracle.Q4_K, wrows, x, rows.size, K)
        worst = max(worst, within(yg[:, rows], yr, S, TOL, "product %d (%s) B=%d" % (t, name, B)))
    say("  max err/S", worst)
    del items


@pytest.mark.parametrize("B", [4, 16])
def test_decode_stack_prestaged(stack, B):
    """The same stack with the activations staged once per product into a
    workspace (gq_gemv_q4k_multi_batched_ws): every output bit-identical to
    the per-block staging, which the test above checks against the oracle;
    the workspace starts as all-ones bytes (NaN as binary32)."""
    torch = torch_cuda()
    say("decode stack prestaged batch", B)
    items, items2 = [], []
    for name, M, K, t, wd, rows, wrows in stack:
        x = torch.from_numpy(synth.activations_f32(WORKLOAD, 100 * t + B, B, K)).cuda()
        items.append((wd, x, torch.full((B, M), float("nan"), dtype=torch.float32, device="cuda"), M, K))
        items2.append((wd, x, torch.full((B, M), float("nan"), dtype=torch.float32, device="cuda"), M, K))
    tab = gq.GemvTable(items, batch=B)
    tab2 = gq.GemvTable(items2, batch=B, prestaged=True)
    tab2.ws.fill_(255)
    tab.run()
    tab2.run()
    for (name, M, K, t, wd, rows, wrows), a, b in zip(stack, items, items2):
        ya, yb = host(a[2]), host(b[2])
        assert np.isfinite(yb).all(), "product %d (%s) B=%d: outputs not written" % (t, name, B)
        assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32)), (t, name, B)
    del items, items2, tab, tab2
