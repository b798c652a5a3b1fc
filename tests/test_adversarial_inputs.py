"""The adversarial weight rows used by the dynamic-range GPU tests decode as
built, by the oracle's own decoder (CPU only)."""
import numpy as np

import oracle
from tests._adversarial import _cols, adversarial_q4k, adversarial_q8_0, check_kinds


def test_q4k_rows_decode_as_built():
    for K in (1024, 4096, 14336, 16640):
        w, kinds = adversarial_q4k(90, K, 64, K)
        check_kinds(w, kinds, 64, K)
        assert sorted(set(kinds.tolist())) == [0, 1, 2, 3, 4, 5]


def test_q8_0_rows_decode_as_built():
    M, K = 64, 4096
    w = adversarial_q8_0(97, M, K)
    w32, _ = oracle.dequant(oracle.Q8_0, w, M, K)
    c, c2 = _cols(K)
    assert np.all(w32[1::8, c] == 0)
    for r in range(4, M, 8):
        assert np.flatnonzero(w32[r]).tolist() == [c2] and w32[r, c2] == 5.0
