"""Dequantized weights must equal the oracle's bit for bit (binary32 and binary16)."""
import numpy as np
import pytest

import oracle
from quantized_unpack_q4_amd import gq, synth
from tests._gpu import dev, half_bits, host, say

pytestmark = pytest.mark.gpu


def _special_q4k_blocks():
    """Blocks with subnormal, negative, zero and extreme scales, all-max quants."""
    g = np.random.default_rng(77)
    blocks = synth.q4k_blocks(70, 0, 8, 256 * 8).reshape(-1, 144).copy()
    vals = np.array([0.0, -0.0, 2.0 ** -24, 3 * 2.0 ** -24, 2.0 ** -14, -0.125, 65504.0,
                     -1.5e-5, 1e-3, 0.5], np.float16)
    for i in range(blocks.shape[0]):
        blocks[i, 0:2] = np.array([vals[i % vals.size]], "<f2").view(np.uint8)
        blocks[i, 2:4] = np.array([vals[(3 * i + 1) % vals.size]], "<f2").view(np.uint8)
        if i % 5 == 0:
            blocks[i, 16:] = 0xFF  # every quant 15
        if i % 7 == 0:
            blocks[i, 4:16] = 0xFF  # every scale and min 63
    return blocks.reshape(-1), g


@pytest.mark.parametrize("M,K", [(1, 256), (37, 1024), (64, 4096)])
def test_dequant_q4k_bit_exact(M, K):
    say("dequant q4k", M, K)
    w = synth.q4k_blocks(71, M, M, K)
    r32, r16 = oracle.dequant(oracle.Q4_K, w, M, K)
    o32, o16 = gq.dequant("q4k", dev(w), M, K)
    assert np.array_equal(host(o32).view(np.uint32), r32.view(np.uint32))
    assert np.array_equal(half_bits(o16), r16)


def test_dequant_q4k_special_blocks():
    w, _ = _special_q4k_blocks()
    M, K = 8, 256 * 8
    r32, r16 = oracle.dequant(oracle.Q4_K, w, M, K)
    o32, o16 = gq.dequant("q4k", dev(w), M, K)
    assert np.array_equal(host(o32).view(np.uint32), r32.view(np.uint32))
    assert np.array_equal(half_bits(o16), r16)
    # only one output requested
    o32b, none16 = gq.dequant("q4k", dev(w), M, K, want16=False)
    assert none16 is None and np.array_equal(host(o32b).view(np.uint32), r32.view(np.uint32))


@pytest.mark.parametrize("M,K", [(1, 32), (7, 96), (256, 1024)])
def test_dequant_q8_0_bit_exact(M, K):
    say("dequant q8_0", M, K)
    w = synth.q8_0_blocks(72, M, M, K)
    blocks = w.reshape(-1, 34)
    blocks[0, 2] = 0x80  # quant -128, allowed by the format
    blocks[-1, 0:2] = np.array([2.0 ** -24], "<f2").view(np.uint8)
    r32, r16 = oracle.dequant(oracle.Q8_0, w, M, K)
    o32, o16 = gq.dequant("q8_0", dev(w), M, K)
    assert np.array_equal(host(o32).view(np.uint32), r32.view(np.uint32))
    assert np.array_equal(half_bits(o16), r16)
