"""Adversarial inputs for the binary32-activation products: activation
vectors with a wide dynamic range inside one vector, and Q4_K / Q8_0 weight
rows built so that the weight at a spike's column is zero, cancels exactly or
nearly, or is the row's only non-zero weight.  Inputs only: the expected
values come from the oracle.

Activation patterns (standard-normal vectors with):
  spike        one element at 1e12 and, in another super-block, one at 3e-12
               among its standard-normal neighbours;
  spike_alone  one element at -4e11 whose sub-block is otherwise zero;
  lograng      every element scaled by 10^U(-12, 12);
  unit_on_tiny x[c] = 1 and every other element 1.37 * 2^-26;
  onehot_big   a one-hot vector scaled by 1e12;
  tiny, subnormal, huge   the whole vector scaled by 1e-36, 1e-40, 1e30.

Weight rows (every 8th row of each kind, the rest natural): kind 1, the
weight at the spike's column exactly zero (q = 0, m = 0); kind 2, exactly zero
by cancellation (dmin = d, sc = m, q = 1); kind 3, nearly cancelling (dmin
one binary16 step from d); kind 4, a row whose only non-zero weight sits at
the tiny element's column; kind 5, zero from large cancelling terms
(d = 2^-10, q = 15, sc = m = 63, dmin = 15 * 2^-10).  check_kinds confirms
each edit with the oracle's own decoder.
"""
import numpy as np

import oracle
from quantized_unpack_q4_amd import synth
from tests import _q4k_edit as qe

PATTERNS = ["spike", "spike_alone", "lograng", "unit_on_tiny", "onehot_big", "tiny", "subnormal",
            "huge"]


def _cols(K):
    # spike column in super-block 3 (sub-block 7 when K >= 1024), tiny column
    # in super-block 1 + K/512
    c = min(1000, K - 24)
    c2 = 256 * (1 + K // 512) + 40 if K >= 1024 else 40
    if c2 // 32 == c // 32:
        c2 = (c2 + 64) % K
    return c, c2


def activations(pattern, K, seed):
    g = np.random.default_rng([77, seed, K])
    x = g.standard_normal(K).astype(np.float64)
    c, c2 = _cols(K)
    if pattern == "spike":
        x[c] = 1e12
        x[c2] = 3e-12
    elif pattern == "spike_alone":
        s0 = 32 * (c // 32)
        x[s0:s0 + 32] = 0.0
        x[c] = -4e11
    elif pattern == "lograng":
        x *= 10.0 ** g.uniform(-12, 12, K)
    elif pattern == "unit_on_tiny":
        x[:] = 1.37 * 2.0 ** -26
        x[c] = 1.0
    elif pattern == "onehot_big":
        x[:] = 0.0
        x[c] = 1e12
    elif pattern == "tiny":
        x *= 1e-36
    elif pattern == "subnormal":
        x *= 1e-40
    elif pattern == "huge":
        x *= 1e30
    else:
        raise ValueError(pattern)
    return x.astype(np.float32)


def floor_for(pattern, K, kernel):
    """Absolute floor of the bound: results in the binary32 subnormal range are
    rounded to multiples of 2^-149 at each conversion to the output scale:
    once per output (batch-1 streaming kernel), up to 16 times per
    super-block (matrix-core kernel), once per block (Q8_0) or once per
    product (general kernel).  The binary32 matrix-core form of single Q4_K
    products at batch 2-16 ("f32mma") rounds each product w*x once, by at most
    2^-150 (its sums of multiples of 2^-149 are exact), so K/2 units."""
    if pattern != "subnormal":
        return 0.0
    n = {"stream": 1.0, "mfma": K / 16.0, "q8": K / 32.0, "general": float(K),
         "f32mma": K / 2.0}[kernel]
    return n * 2.0 ** -149


def adversarial_q4k(workload, tensor, M, K):
    """Synthetic Q4_K rows with edited rows of five kinds (see the module
    docstring); returns the packed bytes and the kinds."""
    w = synth.q4k_blocks(workload, tensor, M, K)
    c, c2 = _cols(K)
    kinds = np.zeros(M, np.int32)
    for r in range(M):
        kind = r % 8
        if kind not in (1, 2, 3, 4, 5):
            continue
        kinds[r] = kind
        b = qe.block(w, K, r, c)
        j = (c % 256) // 32
        if kind == 1:  # zero weight at c: q = 0, m = 0
            qe.set_quant(b, c % 256, 0)
            qe.set_scale_min(b, j, 17, 0)
        elif kind in (2, 3):  # d*sc*q - dmin*m with sc = m, q = 1, dmin = d (+1 step)
            d, _ = qe.get_d_dmin(b)
            d = max(d, 2.0 ** -14)
            dmin = d if kind == 2 else float(np.nextafter(np.float16(d), np.float16(1)))
            qe.set_d_dmin(b, d, dmin)
            qe.set_quant(b, c % 256, 1)
            qe.set_scale_min(b, j, 37, 37)
        elif kind == 5:  # large cancelling terms: 2^-10 * 63 * 15 - (15 * 2^-10) * 63
            qe.set_d_dmin(b, 2.0 ** -10, 15 * 2.0 ** -10)
            qe.set_quant(b, c % 256, 15)
            qe.set_scale_min(b, j, 63, 63)
        elif kind == 4:  # only non-zero weight at c2
            nsb = K // 256
            for s in range(nsb):
                qe.set_d_dmin(qe.block(w, K, r, 256 * s), 0.0, 0.0)
            b2 = qe.block(w, K, r, c2)
            qe.set_d_dmin(b2, 1.0, 0.0)
            j2 = (c2 % 256) // 32
            for jj in range(8):
                qe.set_scale_min(b2, jj, 1 if jj == j2 else 0, 0)
            for k in range(32 * j2, 32 * j2 + 32):
                qe.set_quant(b2, k, 5 if k == c2 % 256 else 0)
    return w, kinds


def check_kinds(w, kinds, M, K):
    """The edits mean what they say, by the oracle's decoder."""
    w32, _ = oracle.dequant(oracle.Q4_K, w, M, K)
    c, c2 = _cols(K)
    for r in range(M):
        if kinds[r] in (1, 2, 5):
            assert w32[r, c] == 0.0, (r, kinds[r], w32[r, c])
        elif kinds[r] == 3:
            assert w32[r, c] != 0.0 and abs(w32[r, c]) < 1e-3 * np.abs(w32[r]).max()
        elif kinds[r] == 4:
            nz = np.flatnonzero(w32[r])
            assert nz.tolist() == [c2] and w32[r, c2] == 5.0




def adversarial_q8_0(workload, M, K):
    w = synth.q8_0_blocks(workload, 0, M, K)
    blk = w.reshape(M, K // 32, 34)
    c, c2 = _cols(K)
    for r in range(M):
        if r % 8 == 1:  # zero weight at c
            blk[r, c // 32, 2 + c % 32] = 0
        elif r % 8 == 4:  # only non-zero weight at c2: d = 1, q = 5
            blk[r, :, :] = 0
            blk[r, c2 // 32, 0:2] = np.array([1.0], "<f2").view(np.uint8)
            blk[r, c2 // 32, 2 + c2 % 32] = 5
    return w
