"""Field edits of packed Q4_K super-blocks, for building adversarial weight rows
in tests (a weight that is exactly zero, or whose two terms d*sc*q and
dmin*m cancel).  Every caller checks the edited weights with the oracle's own
decoder, so a mistake here shows up as a failed assertion, not a wrong pin.

Byte layout of a 144-byte super-block (GGUF Q4_K): 0-1 d, 2-3 dmin (binary16),
4-15 the twelve scale/min bytes s[0..11], 16-143 the 128 quant bytes.  For
sub-blocks j < 4 the scale is the low 6 bits of s[j] and the min the low 6
bits of s[j+4]; for j >= 4 the scale is the low nibble of s[j+4] with the top
two bits of s[j-4] above it, the min the high nibble of s[j+4] with the top
two bits of s[j] above it.  Weight k sits in quant byte 32*(k//64) + k%32, in
the low nibble when k%64 < 32, else the high nibble.
"""
from __future__ import annotations

import numpy as np

SB = 144


def block(w: np.ndarray, K: int, row: int, col: int) -> np.ndarray:
    """The 144 bytes (a writable view) of the super-block holding (row, col)."""
    nsb = K // 256
    off = (row * nsb + col // 256) * SB
    return w[off:off + SB]


def set_quant(b: np.ndarray, k: int, q: int) -> None:
    i = 16 + 32 * (k // 64) + k % 32
    if k % 64 < 32:
        b[i] = (b[i] & 0xF0) | (q & 15)
    else:
        b[i] = (b[i] & 0x0F) | ((q & 15) << 4)


def set_scale_min(b: np.ndarray, j: int, sc: int, m: int) -> None:
    s = b[4:16]  # view
    if j < 4:
        s[j] = (s[j] & 0xC0) | (sc & 63)
        s[j + 4] = (s[j + 4] & 0xC0) | (m & 63)
    else:
        s[j + 4] = (sc & 15) | ((m & 15) << 4)
        s[j - 4] = (s[j - 4] & 0x3F) | ((sc >> 4) << 6)
        s[j] = (s[j] & 0x3F) | ((m >> 4) << 6)


def set_d_dmin(b: np.ndarray, d: float, dmin: float) -> None:
    b[0:4] = np.array([d, dmin], dtype="<f2").view(np.uint8)


def get_d_dmin(b: np.ndarray):
    v = b[0:4].copy().view("<f2")
    return float(v[0]), float(v[1])
