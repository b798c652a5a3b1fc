"""Binary32-activation products against the oracle on activations with a wide
dynamic range inside one vector, and on weight rows built to expose it
(inputs from tests/_adversarial.py, whose docstring lists them).

Every kernel that takes binary32 activations is covered: batch 1 (single
matrix, multi-product table, gate/up with SwiGLU, the general kernel for
K > 16384), batches 2-16 on the matrix cores (single matrix and table) and
Q8_0 at batch 1 and 2-16.

Bound: |y - y_ref| <= 1e-5 * S + floor, S = sum |w x| in binary64; floor is
0 except for vectors whose results fall in the binary32 subnormal range
(_adversarial.floor_for).
"""
import numpy as np
import pytest

import oracle
from quantized_unpack_q4_amd import gq
from tests._adversarial import (PATTERNS, _cols, activations, adversarial_q4k, adversarial_q8_0,
                                floor_for)
from tests._gpu import dev, host, say, torch_cuda

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _compare(y, w, xs, M, K, fmt, kernel, what):
    worst = 0.0
    for b, (pat, x) in enumerate(xs):
        yr, S = oracle.gemv(fmt, w, x[None, :], M, K)
        fl = floor_for(pat, K, kernel)
        err = np.abs(np.asarray(y[b], np.float64) - yr[0])
        bad = ~(err <= TOL * S[0] + fl)
        if np.any(bad):
            i = int(np.argmax(np.where(bad, err - TOL * S[0], -np.inf)))
            raise AssertionError("%s %s: %d rows out of bound; row %d (kind %d) gpu %.9g ref %.9g S %.4g"
                                 % (what, pat, int(bad.sum()), i, i % 8, y[b][i], yr[0, i], S[0, i]))
        pos = S[0] > 0
        worst = max(worst, float((err[pos] / S[0][pos]).max()) if np.any(pos) else 0.0)
    return worst


@pytest.mark.parametrize("M,K", [(520, 4096), (264, 14336), (100, 1024)])
def test_q4k_batch1_single(M, K):
    torch = torch_cuda()
    w, kinds = adversarial_q4k(91, K, M, K)
    wd = dev(w)
    worst = 0.0
    for i, pat in enumerate(PATTERNS):
        x = activations(pat, K, i)
        say("batch1 single", M, K, pat)
        y = torch.full((1, M), float("nan"), dtype=torch.float32, device="cuda")
        gq.gq_gemv_q4k(wd, dev(x[None, :]), y, M, K, 1)
        worst = max(worst, _compare(host(y), w, [(pat, x)], M, K, oracle.Q4_K, "stream",
                                    "b1 %dx%d" % (M, K)))
    say("  worst err/S", worst)


def test_q4k_batch1_general_kernel():
    """K = 16640 is past the streaming kernel's limit: the general kernel."""
    torch = torch_cuda()
    M, K = 136, 16640
    w, kinds = adversarial_q4k(92, K, M, K)
    wd = dev(w)
    for i, pat in enumerate(PATTERNS):
        x = activations(pat, K, 100 + i)
        say("batch1 general", M, K, pat)
        y = torch.full((1, M), float("nan"), dtype=torch.float32, device="cuda")
        gq.gq_gemv_q4k(wd, dev(x[None, :]), y, M, K, 1)
        _compare(host(y), w, [(pat, x)], M, K, oracle.Q4_K, "general", "general")


def test_q4k_batch1_table():
    """One multi-product table, a different activation pattern per product."""
    torch = torch_cuda()
    shapes = [(200, 4096), (72, 14336), (48, 256), (130, 2048)] * 2
    items, host_in = [], []
    for i, (M, K) in enumerate(shapes):
        w, _ = adversarial_q4k(93, i, M, K)
        pat = PATTERNS[i % len(PATTERNS)]
        x = activations(pat, K, 200 + i)
        y = torch.full((1, M), float("nan"), dtype=torch.float32, device="cuda")
        items.append((dev(w), dev(x[None, :]), y, M, K))
        host_in.append((w, x, pat))
    t = gq.GemvTable(items)
    t.run()
    for (w, x, pat), (_, _, y, M, K) in zip(host_in, items):
        say("table", M, K, pat)
        _compare(host(y), w, [(pat, x)], M, K, oracle.Q4_K, "stream", "table %dx%d" % (M, K))


@pytest.mark.parametrize("B", [2, 4, 16])
def test_q4k_batched(B):
    """Batch rows with different patterns in one call: a single matrix (the
    binary32 matrix-core form) and a table (the binary16-split matrix-core
    kernel)."""
    torch = torch_cuda()
    M, K = 392, 4096
    w, _ = adversarial_q4k(94, B, M, K)
    pats = [PATTERNS[(b + B) % len(PATTERNS)] for b in range(B)]
    xs = [(p, activations(p, K, 300 + 17 * B + b)) for b, p in enumerate(pats)]
    x = np.stack([v for _, v in xs])
    say("batched single", B, pats)
    y = torch.full((B, M), float("nan"), dtype=torch.float32, device="cuda")
    gq.gq_gemv_q4k(dev(w), dev(x), y, M, K, B)
    w1 = _compare(host(y), w, xs, M, K, oracle.Q4_K, "f32mma", "batched B=%d" % B)
    # the same rows as one entry of a two-entry table (the second a shorter K)
    M2, K2 = 130, 1024
    w2, _ = adversarial_q4k(95, B, M2, K2)
    xs2 = [(p, activations(p, K2, 400 + 17 * B + b)) for b, p in enumerate(pats)]
    x2 = np.stack([v for _, v in xs2])
    y1 = torch.full((B, M), float("nan"), dtype=torch.float32, device="cuda")
    y2 = torch.full((B, M2), float("nan"), dtype=torch.float32, device="cuda")
    t = gq.GemvTable([(dev(w), dev(x), y1, M, K), (dev(w2), dev(x2), y2, M2, K2)], batch=B)
    t.run()
    _compare(host(y1), w, xs, M, K, oracle.Q4_K, "mfma", "batched table B=%d" % B)
    _compare(host(y2), w2, xs2, M2, K2, oracle.Q4_K, "mfma", "batched table B=%d K=%d" % (B, K2))
    # the same table with the activations pre-staged into a workspace (the
    # exact path then reads the binary32 activations from global memory)
    z1 = torch.full((B, M), float("nan"), dtype=torch.float32, device="cuda")
    z2 = torch.full((B, M2), float("nan"), dtype=torch.float32, device="cuda")
    tp = gq.GemvTable([(dev(w), dev(x), z1, M, K), (dev(w2), dev(x2), z2, M2, K2)], batch=B,
                      prestaged=True)
    tp.run()
    assert np.array_equal(host(z1).view(np.uint32), host(y1).view(np.uint32))
    assert np.array_equal(host(z2).view(np.uint32), host(y2).view(np.uint32))
    say("  worst err/S", w1)


def test_q4k_swiglu_spikes():
    """Gate/up with the SwiGLU epilogue on spiked and wide-range vectors."""
    torch = torch_cuda()
    M, K = 264, 4096
    wg, _ = adversarial_q4k(96, 0, M, K)
    wu, _ = adversarial_q4k(96, 1, M, K)
    for i, pat in enumerate(["spike", "spike_alone", "lograng", "unit_on_tiny"]):
        x = activations(pat, K, 500 + i)
        # keep silu(g) * u finite in binary32: bring the vector to ~1e3 at most
        x = (x * np.float32(1e3 / np.abs(x).max())).astype(np.float32)
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
        assert np.all(err <= bound), "swiglu %s: worst %.3g of bound" % (pat, np.nanmax(err / bound))


def test_q4k_swiglu_batched_spikes():
    """Gate/up with the SwiGLU epilogue at batch 4 on the matrix cores, one
    spiked or wide-range pattern per activation row."""
    torch = torch_cuda()
    M, K = 264, 4096
    wg, _ = adversarial_q4k(97, 0, M, K)
    wu, _ = adversarial_q4k(97, 1, M, K)
    pats = ["spike", "spike_alone", "lograng", "unit_on_tiny"]
    x = np.stack([activations(p, K, 600 + i) for i, p in enumerate(pats)])
    x = (x * (np.float32(1e3) / np.abs(x).max(axis=1, keepdims=True))).astype(np.float32)
    B = x.shape[0]
    h = torch.full((B, M), float("nan"), dtype=torch.float32, device="cuda")
    gq.gq_gemv_q4k_swiglu_batched(dev(wg), dev(wu), dev(x), h, M, K, B)
    hg = host(h).astype(np.float64)
    g, Sg = oracle.gemv(oracle.Q4_K, wg, x, M, K)
    u, Su = oracle.gemv(oracle.Q4_K, wu, x, M, K)
    hr = oracle.swiglu(g, u)
    sg = oracle.swiglu(g, np.ones_like(g))
    bound = TOL * (1.1 * Sg * np.abs(u) + np.abs(sg) * Su) + (4 + np.abs(g)) * 2.0 ** -23 * np.abs(hr)
    err = np.abs(hg - hr)
    assert np.all(err <= bound), "swiglu batched: worst %.3g of bound" % np.nanmax(err / bound)


@pytest.mark.parametrize("B", [1, 4, 16])
def test_q8_0_patterns(B):
    torch = torch_cuda()
    M, K = 520, 4096
    w = adversarial_q8_0(97, M, K)
    w32, _ = oracle.dequant(oracle.Q8_0, w, M, K)
    c, c2 = _cols(K)
    assert np.all(w32[1::8, c] == 0) and np.all(w32[4::8, c2] == 5)
    pats = [PATTERNS[(b + 3 * B) % len(PATTERNS)] for b in range(max(B, len(PATTERNS)))]
    for start in range(0, len(pats), B):
        sel = pats[start:start + B]
        xs = [(p, activations(p, K, 600 + 31 * B + start + i)) for i, p in enumerate(sel)]
        x = np.stack([v for _, v in xs])
        say("q8_0", B, sel)
        y = torch.full((len(sel), M), float("nan"), dtype=torch.float32, device="cuda")
        gq.gq_gemv_q8_0(dev(w), dev(x), y, M, K, len(sel))
        _compare(host(y), w, xs, M, K, oracle.Q8_0, "q8", "q8_0 B=%d" % len(sel))
