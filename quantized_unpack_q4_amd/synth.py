"""Seeded synthetic inputs: packed Q8_0 / Q4_K weight blocks and activations.

This module only draws random numbers and lays them out in the GGUF block
byte order; it contains none of the dequantization or matmul arithmetic.
Both the HIP path's tests and the reference oracle take their inputs from
here, so it is the one piece of code the two sides share.

Recipes (the synthetic stand-ins for the real checkpoints the pages run):

* Q8_0 block (34 B / 32 weights): ``d = binary16(|z| * 0.01)`` with z a
  standard normal (binary64, rounded once to binary16 by numpy), then 32
  int8 quants drawn uniformly from [-127, 127].
* Q4_K super-block (144 B / 256 weights): ``d, dmin = binary16(|z| * 1e-3)``
  each; the 12 scale/min bytes and the 128 quant bytes are uniform random
  bytes.  The 12-byte field packs sixteen 6-bit numbers into exactly 96
  bits, every bit used once, so uniform bytes give eight scales and eight
  mins that are independent and uniform on 0..63; likewise uniform quant
  bytes give independent 4-bit quants uniform on 0..15.
* Activations: standard normal binary32 (matrix-vector products), the same
  rounded to binary16 (matrix products, MoE), router logits standard normal
  binary32.

Every stream is ``numpy.random.default_rng([workload, tensor, role])`` with
role 0 = weights, 1 = activations, 2 = router logits.
"""
from __future__ import annotations

import numpy as np

ROLE_WEIGHTS = 0
ROLE_ACTIVATIONS = 1
ROLE_ROUTER = 2

Q8_0_BLOCK_BYTES = 34
Q8_0_BLOCK_WEIGHTS = 32
Q4_K_BLOCK_BYTES = 144
Q4_K_BLOCK_WEIGHTS = 256


def rng(workload: int, tensor: int, role: int) -> np.random.Generator:
    return np.random.default_rng([int(workload), int(tensor), int(role)])


def q8_0_bytes(M: int, K: int) -> int:
    assert K % Q8_0_BLOCK_WEIGHTS == 0
    return M * (K // Q8_0_BLOCK_WEIGHTS) * Q8_0_BLOCK_BYTES


def q4k_bytes(M: int, K: int) -> int:
    assert K % Q4_K_BLOCK_WEIGHTS == 0
    return M * (K // Q4_K_BLOCK_WEIGHTS) * Q4_K_BLOCK_BYTES


def q8_0_blocks(workload: int, tensor: int, M: int, K: int, scale: float = 0.01) -> np.ndarray:
    """Packed Q8_0 weights of an M x K matrix as a flat uint8 array."""
    g = rng(workload, tensor, ROLE_WEIGHTS)
    nb = M * (K // Q8_0_BLOCK_WEIGHTS)
    d = (np.abs(g.standard_normal(nb)) * scale).astype(np.float16)
    q = g.integers(-127, 128, size=(nb, Q8_0_BLOCK_WEIGHTS), dtype=np.int8)
    out = np.empty((nb, Q8_0_BLOCK_BYTES), np.uint8)
    out[:, 0:2] = d.astype("<f2").view(np.uint8).reshape(nb, 2)
    out[:, 2:] = q.view(np.uint8)
    return out.reshape(-1)


def q4k_blocks(workload: int, tensor: int, M: int, K: int, scale: float = 1e-3,
               out: np.ndarray | None = None) -> np.ndarray:
    """Packed Q4_K weights of an M x K matrix as a flat uint8 array.

    ``out`` (optional) is a preallocated flat uint8 array of the right size.
    """
    g = rng(workload, tensor, ROLE_WEIGHTS)
    nsb = M * (K // Q4_K_BLOCK_WEIGHTS)
    nbytes = nsb * Q4_K_BLOCK_BYTES
    if out is None:
        out = np.empty(nbytes, np.uint8)
    assert out.dtype == np.uint8 and out.size == nbytes
    # every byte uniform first (the 12 scale/min bytes and 128 quant bytes keep
    # these), then d and dmin overwrite bytes 0..3 of each super-block
    out[:] = g.integers(0, 256, size=nbytes, dtype=np.uint8)
    blk = out.reshape(nsb, Q4_K_BLOCK_BYTES)
    dd = (np.abs(g.standard_normal((nsb, 2))) * scale).astype("<f2")
    blk[:, 0:4] = dd.view(np.uint8).reshape(nsb, 4)
    return out


def activations_f32(workload: int, tensor: int, rows: int, K: int) -> np.ndarray:
    g = rng(workload, tensor, ROLE_ACTIVATIONS)
    return g.standard_normal((rows, K), dtype=np.float32)


def activations_f16(workload: int, tensor: int, rows: int, K: int) -> np.ndarray:
    g = rng(workload, tensor, ROLE_ACTIVATIONS)
    return g.standard_normal((rows, K), dtype=np.float32).astype(np.float16)


def router_logits(workload: int, tensor: int, T: int, E: int) -> np.ndarray:
    g = rng(workload, tensor, ROLE_ROUTER)
    return g.standard_normal((T, E), dtype=np.float32)
