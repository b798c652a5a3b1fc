"""The seeded input generators: determinism and the recipe's distributions."""
import hashlib

import numpy as np

from quantized_unpack_q4_amd import synth


def _h(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_deterministic_and_seed_dependent():
    a = synth.q4k_blocks(1, 0, 8, 512)
    b = synth.q4k_blocks(1, 0, 8, 512)
    c = synth.q4k_blocks(1, 1, 8, 512)
    assert _h(a) == _h(b) and _h(a) != _h(c)
    assert a.size == synth.q4k_bytes(8, 512) == 8 * 2 * 144
    x = synth.activations_f32(1, 0, 2, 256)
    assert _h(x) == _h(synth.activations_f32(1, 0, 2, 256))
    q8 = synth.q8_0_blocks(1, 0, 4, 64)
    assert q8.size == synth.q8_0_bytes(4, 64) == 4 * 2 * 34
    out = np.empty(synth.q4k_bytes(8, 512), np.uint8)
    synth.q4k_blocks(1, 0, 8, 512, out=out)
    assert _h(out) == _h(a)


def test_q4k_recipe_distribution(orc):
    w = synth.q4k_blocks(2, 0, 64, 256 * 32)  # 2048 super-blocks
    blocks = w.reshape(-1, 144)
    d = blocks[:, 0:2].copy().view("<f2").astype(np.float64).ravel()
    dmin = blocks[:, 2:4].copy().view("<f2").astype(np.float64).ravel()
    assert np.all(d >= 0) and np.all(dmin >= 0)
    # |N(0,1)| * 1e-3 has mean sqrt(2/pi) * 1e-3
    assert abs(d.mean() / 1e-3 - np.sqrt(2 / np.pi)) < 0.05
    assert abs(dmin.mean() / 1e-3 - np.sqrt(2 / np.pi)) < 0.05
    scs, ms, qs = [], [], []
    for i in range(0, 2048, 8):
        _, _, sc, m, q = orc.q4k_fields(blocks[i])
        scs.append(sc)
        ms.append(m)
        qs.append(q)
    scs, ms, qs = map(np.concatenate, (scs, ms, qs))
    assert set(scs) == set(range(64)) and set(ms) == set(range(64))
    assert set(qs) == set(range(16))
    assert abs(scs.mean() - 31.5) < 1.5 and abs(qs.mean() - 7.5) < 0.2


def test_q8_0_recipe_distribution():
    w = synth.q8_0_blocks(3, 0, 16, 32 * 64).reshape(-1, 34)
    q = w[:, 2:].view(np.int8)
    assert q.min() >= -127 and q.max() <= 127
    assert q.min() == -127 and q.max() == 127
    d = w[:, 0:2].copy().view("<f2").astype(np.float64)
    assert np.all(d >= 0) and abs(d.mean() / 0.01 - np.sqrt(2 / np.pi)) < 0.05


def test_activation_dtypes():
    assert synth.activations_f32(0, 0, 3, 256).dtype == np.float32
    assert synth.activations_f16(0, 0, 3, 256).dtype == np.float16
    assert synth.router_logits(0, 0, 5, 64).shape == (5, 64)
