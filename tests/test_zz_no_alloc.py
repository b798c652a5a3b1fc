"""The no-allocation split-K entry point (gq_gemm_q4k_splitk_static) against
the workspace form (gq_gemm_q4k_splitk) through the C ABI: bit-identical
outputs on two calls in a row, the second with a smaller input (the static
scratch keeps the first call's partials), both within the oracle's bound."""
import ctypes

import numpy as np
import pytest

import oracle
from quantized_unpack_q4_amd import gq, synth
from tests._gpu import dev, half_bits, say, torch_cuda, within

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _call_pair(w, x16, M, K, splits):
    torch = torch_cuda()
    N = x16.shape[0]
    wd, xd = dev(w), dev(x16)
    ys = torch.full((N, M), float("nan"), dtype=torch.float16, device="cuda")
    yw = torch.full((N, M), float("nan"), dtype=torch.float16, device="cuda")
    L = gq.lib()
    st = L.gq_gemm_q4k_splitk_static(ctypes.c_void_p(wd.data_ptr()),
                                     ctypes.c_void_p(xd.data_ptr()),
                                     ctypes.c_void_p(ys.data_ptr()), M, K, N, splits, None)
    assert st == 0, gq.last_error()
    nbytes = gq.gq_gemm_q4k_splitk_workspace_bytes(M, K, N, splits)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    gq.gq_gemm_q4k_splitk(wd, xd, yw, M, K, N, splits, ws)
    return half_bits(ys), half_bits(yw)


def test_static_splitk_matches_workspace_form_twice():
    cases = [(4096, 14336, 512, 0), (600, 1024, 300, 4)]  # full size, then smaller
    for i, (M, K, N, splits) in enumerate(cases):
        say("static split-K call", i, M, K, N, splits)
        w = synth.q4k_blocks(3 if i == 0 else 96, M, M, K)
        x16 = synth.activations_f16(3 if i == 0 else 96, N, N, K)
        ys, yw = _call_pair(w, x16, M, K, splits)
        assert np.array_equal(ys, yw), "static and workspace forms differ (call %d)" % i
        g = np.random.default_rng(5)
        rows = np.unique(np.concatenate([[0, M - 1], g.choice(M, 64, replace=False)]))
        yr, S = oracle.gemm_matmul(oracle.Q4_K, w, x16, M, K, rows=rows)
        r = within(ys.view(np.float16).astype(np.float64)[:, rows], yr, S, TOL, "static call %d" % i)
        say("  max err/S", r)


def test_static_splitk_refuses_beyond_scratch():
    torch = torch_cuda()
    M, K, N = 4096, 14336, 4096  # 8 runs of 4096 x 4096 binary32 partials: 512 MiB
    cap = gq.gq_gemm_q4k_splitk_static_max_bytes()
    assert cap == 64 << 20
    w = torch.zeros(M * K // 256 * 144, dtype=torch.uint8, device="cuda")
    x = torch.zeros((N, K), dtype=torch.float16, device="cuda")
    y = torch.zeros((N, M), dtype=torch.float16, device="cuda")
    L = gq.lib()
    st = L.gq_gemm_q4k_splitk_static(ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(x.data_ptr()),
                                     ctypes.c_void_p(y.data_ptr()), M, K, N, 8, None)
    assert st == 4 and "static scratch" in gq.last_error()  # GQ_EWORKSPACE, nothing launched
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(y)) == 0
