"""Reference oracle for the fused block-dequant matmul (TEST INFRASTRUCTURE).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` import this package.  The HIP library never calls it, and it
shares no code with that library: the arithmetic lives in ``oracle.c`` (plain
C, binary64 accumulation), and this module only marshals numpy arrays.

What it computes is the plain definition of the method on the page "Building a
Rust Inference Engine That Matches Llama.cpp", section "Where the wins came
from": weights stored as GGUF quantized blocks are dequantized at the moment
they enter the dot product; the fused result equals dequantize-then-dot.

Parity pins: every function here is pinned by tests marked ``not gpu``
(hand-built blocks, closed forms, exhaustive binary16 decode against numpy,
an independently written numpy unpacker, brute force and invariants).  The
8-bit activation blocks (``quantize_q8k``) and the integer-dot product over
them (``gemv_q4k_q8k``) follow a reading of a block the pages name but do not
define, pinned by closed forms, rounding bounds and numpy.  The
MoE readings (SwiGLU between the expert projections, top-k softmax weights
used without renormalisation) are readings, not pinned by the pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

Q8_0 = 0
Q4_K = 1

_c_i64p = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc into liboracle.so (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        vp = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.orc_half_to_double.restype = ctypes.c_double
        L.orc_half_to_double.argtypes = [ctypes.c_uint16]
        L.orc_double_to_half.restype = ctypes.c_uint16
        L.orc_double_to_half.argtypes = [ctypes.c_double]
        L.orc_half_array_to_double.argtypes = [vp, i64, vp]
        L.orc_double_array_to_half.argtypes = [vp, i64, vp]
        L.orc_q4k_fields.argtypes = [vp, vp, vp, vp, vp, vp]
        L.orc_dequant.argtypes = [ctypes.c_int, vp, i64, i64, vp, vp]
        L.orc_gemv.argtypes = [ctypes.c_int, vp, vp, i64, i64, i64, vp, i64, vp, vp]
        L.orc_gemv_separate.argtypes = [ctypes.c_int, vp, vp, i64, i64, i64, vp]
        L.orc_gemm.argtypes = [ctypes.c_int, vp, vp, i64, i64, i64, vp, i64, vp, i64, vp, vp]
        L.orc_moe_route.argtypes = [vp, i64, i64, i64, vp, vp, ctypes.c_int]
        L.orc_swiglu.argtypes = [vp, vp, i64, vp]
        L.orc_moe_ffn.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                  vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int]
        L.orc_quantize_q8k.argtypes = [vp, i64, i64, vp, vp, vp]
        L.orc_gemv_q4k_q8k.argtypes = [vp, vp, vp, i64, i64, i64, vp, i64, vp, vp]
        L.orc_q4k_terms.argtypes = [vp, i64, i64, vp, vp]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _u8(w):
    w = np.ascontiguousarray(w)
    if w.dtype != np.uint8:
        w = w.view(np.uint8)
    return w.reshape(-1)


def _bits16(x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.float16:
        x = x.view(np.uint16)
    assert x.dtype == np.uint16
    return x


def _idx(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64).reshape(-1))


def row_bytes(fmt: int, K: int) -> int:
    return K // 32 * 34 if fmt == Q8_0 else K // 256 * 144


def _check(fmt, w, M, K):
    if fmt == Q8_0:
        assert K % 32 == 0
    else:
        assert K % 256 == 0
    assert w.size >= M * row_bytes(fmt, K)


# -- binary16 ---------------------------------------------------------------

def half_to_double(bits) -> np.ndarray:
    bits = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16).reshape(-1))
    out = np.empty(bits.size, dtype=np.float64)
    lib().orc_half_array_to_double(_p(bits), bits.size, _p(out))
    return out


def double_to_half(v) -> np.ndarray:
    """Round each value to binary16 (nearest, ties to even); returns bit patterns."""
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float64).reshape(-1))
    out = np.empty(v.size, dtype=np.uint16)
    lib().orc_double_array_to_half(_p(v), v.size, _p(out))
    return out


# -- block decode -------------------------------------------------------------

def q4k_fields(block):
    """(d, dmin, sc[8], m[8], q[256]) of one 144-byte Q4_K super-block."""
    block = _u8(block)
    assert block.size == 144
    d = ctypes.c_double()
    dmin = ctypes.c_double()
    sc = np.empty(8, np.int32)
    m = np.empty(8, np.int32)
    q = np.empty(256, np.int32)
    lib().orc_q4k_fields(_p(block), ctypes.byref(d), ctypes.byref(dmin), _p(sc), _p(m), _p(q))
    return d.value, dmin.value, sc, m, q


def dequant(fmt: int, w, M: int, K: int):
    """(w32 [M][K] float32, w16 [M][K] uint16 bits)."""
    w = _u8(w)
    _check(fmt, w, M, K)
    o32 = np.empty((M, K), np.float32)
    o16 = np.empty((M, K), np.uint16)
    lib().orc_dequant(fmt, _p(w), M, K, _p(o32), _p(o16))
    return o32, o16


# -- products -----------------------------------------------------------------

def gemv(fmt: int, w, x, M: int, K: int, rows=None):
    """y[b][i] = sum_k w32[rows[i]][k] x[b][k] (binary64) and its bound S."""
    w = _u8(w)
    _check(fmt, w, M, K)
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32).reshape(-1, K))
    B = x.shape[0]
    rows = _idx(rows)
    nr = M if rows is None else rows.size
    y = np.empty((B, nr), np.float64)
    S = np.empty((B, nr), np.float64)
    lib().orc_gemv(fmt, _p(w), _p(x), M, K, B, _p(rows), nr, _p(y), _p(S))
    return y, S


def gemv_separate(fmt: int, w, x, M: int, K: int):
    w = _u8(w)
    _check(fmt, w, M, K)
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32).reshape(-1, K))
    y = np.empty((x.shape[0], M), np.float64)
    lib().orc_gemv_separate(fmt, _p(w), _p(x), M, K, x.shape[0], _p(y))
    return y


def gemm(fmt: int, w, x16, M: int, K: int, rows=None, toks=None):
    """Y[t][i] = sum_k w32[rows[i]][k] x16[toks[t]][k] (binary64) and its bound S."""
    w = _u8(w)
    _check(fmt, w, M, K)
    x16 = _bits16(x16).reshape(-1, K)
    N = x16.shape[0]
    rows = _idx(rows)
    toks = _idx(toks)
    nr = M if rows is None else rows.size
    nt = N if toks is None else toks.size
    y = np.empty((nt, nr), np.float64)
    S = np.empty((nt, nr), np.float64)
    lib().orc_gemm(fmt, _p(w), _p(x16), M, K, N, _p(rows), nr, _p(toks), nt, _p(y), _p(S))
    return y, S


def gemm_matmul(fmt: int, w, x16, M: int, K: int, rows=None, toks=None):
    """The same result as ``gemm``, for large samples: each weight is decoded
    by the C decoder (``dequant``, binary32), every product and sum is taken in
    binary64 by numpy's matrix product (a library primitive in place of the
    plain loop; only the summation order differs, by ~1e-15 * S), and
    S = |X| |W|^T likewise.  Returns (Y [ntoks][nrows], S)."""
    w = _u8(w)
    _check(fmt, w, M, K)
    x16 = _bits16(x16).reshape(-1, K)
    rows = None if rows is None else np.asarray(rows, dtype=np.int64).reshape(-1)
    toks = None if toks is None else np.asarray(toks, dtype=np.int64).reshape(-1)
    rb = row_bytes(fmt, K)
    if rows is None:
        wsel, nr = w[:M * rb], M
    else:
        wsel = w[:M * rb].reshape(M, rb)[rows].reshape(-1)
        nr = rows.size
    w32, _ = dequant(fmt, wsel, nr, K)
    xs = x16 if toks is None else x16[toks]
    xd = xs.view(np.float16).astype(np.float64)
    wd = w32.astype(np.float64)
    return xd @ wd.T, np.abs(xd) @ np.abs(wd).T


def swiglu(g, u):
    """h = silu(g) * u elementwise in binary64 (silu(z) = z / (1 + e^-z))."""
    g = np.ascontiguousarray(np.asarray(g, dtype=np.float64))
    u = np.ascontiguousarray(np.asarray(u, dtype=np.float64))
    if g.shape != u.shape:
        raise ValueError("g and u differ in shape")
    h = np.empty_like(g)
    lib().orc_swiglu(_p(g), _p(u), g.size, _p(h))
    return h


def moe_route(logits, topk: int, renormalize: bool = False):
    """Top-k of the binary64 softmax of each row: (ids int32 [T][k], wts float64 [T][k]);
    with renormalize the chosen weights are divided by their sum."""
    logits = np.ascontiguousarray(np.asarray(logits, dtype=np.float32))
    T, E = logits.shape
    ids = np.empty((T, topk), np.int32)
    wts = np.empty((T, topk), np.float64)
    lib().orc_moe_route(_p(logits), T, E, topk, _p(ids), _p(wts), 1 if renormalize else 0)
    return ids, wts


def moe_ffn(w_gate, w_up, w_down, x16, ids, wts, H: int, I: int, E: int,
            weight_input: bool = False, fmt: int = Q4_K):
    """Binary64 MoE feed-forward; returns dict of g, u, h, d, out, Sg, Su, Sd.
    weight_input: each slot's weight scales the expert's input, not its output.
    fmt: format of all three weight stacks (Q4_K or Q8_0)."""
    x16 = _bits16(x16).reshape(-1, H)
    T = x16.shape[0]
    ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
    wts = np.ascontiguousarray(np.asarray(wts, dtype=np.float32))
    topk = ids.shape[1]
    assert ids.shape == (T, topk) and wts.shape == (T, topk)
    assert 0 <= ids.min() and ids.max() < E
    gu = I * row_bytes(fmt, H)
    dn = H * row_bytes(fmt, I)
    wg, wu, wd = _u8(w_gate), _u8(w_up), _u8(w_down)
    assert wg.size >= E * gu and wu.size >= E * gu and wd.size >= E * dn
    A = T * topk
    r = {k: np.empty((A, I)) for k in ("g", "u", "h", "Sg", "Su")}
    r.update({k: np.empty((A, H)) for k in ("d", "Sd")})
    r["out"] = np.empty((T, H))
    lib().orc_moe_ffn(fmt, _p(wg), _p(wu), _p(wd), _p(x16), _p(ids), _p(wts), T, H, I, E, topk,
                      _p(r["g"]), _p(r["u"]), _p(r["h"]), _p(r["d"]), _p(r["out"]),
                      _p(r["Sg"]), _p(r["Su"]), _p(r["Sd"]), 1 if weight_input else 0)
    return r


def quantize_q8k(x, K: int):
    """Activations as 8-bit blocks of 256: (q int8 [B][K], d float32 [B][K/256],
    bsum int32 [B][K/32]), every step in binary32."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32).reshape(-1, K))
    assert K % 256 == 0
    B = x.shape[0]
    q = np.empty((B, K), np.int8)
    d = np.empty((B, K // 256), np.float32)
    bs = np.empty((B, K // 32), np.int32)
    lib().orc_quantize_q8k(_p(x), B, K, _p(q), _p(d), _p(bs))
    return q, d, bs


def gemv_q4k_q8k(w, q, d, M: int, K: int, rows=None):
    """y[b][i] = sum_k w_exact[rows[i]][k] d_b q_b[k] (binary64) and its bound S."""
    w = _u8(w)
    _check(Q4_K, w, M, K)
    q = np.ascontiguousarray(np.asarray(q, dtype=np.int8).reshape(-1, K))
    B = q.shape[0]
    d = np.ascontiguousarray(np.asarray(d, dtype=np.float32).reshape(B, K // 256))
    rows = _idx(rows)
    nr = M if rows is None else rows.size
    y = np.empty((B, nr), np.float64)
    S = np.empty((B, nr), np.float64)
    lib().orc_gemv_q4k_q8k(_p(w), _p(q), _p(d), M, K, B, _p(rows), nr, _p(y), _p(S))
    return y, S


def q4k_terms(w, M: int, K: int, rows=None):
    """The exact terms a = d*sc*q and c = dmin*m of every weight (w = a - c),
    binary64 [nrows][K] each, for the given rows (all if None)."""
    w = _u8(w)
    _check(Q4_K, w, M, K)
    rb = row_bytes(Q4_K, K)
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64).reshape(-1)
        w = np.ascontiguousarray(w[:M * rb].reshape(M, rb)[rows]).reshape(-1)
        M = rows.size
    a = np.empty((M, K), np.float64)
    c = np.empty((M, K), np.float64)
    lib().orc_q4k_terms(_p(w), M, K, _p(a), _p(c))
    return a, c


def gemm_q4k_q8k(w, q, d, M: int, K: int, rows=None, toks=None):
    """Y[t][i] = sum_k w_exact[rows[i]][k] * d[toks[t]][k/256] * q[toks[t]][k]
    (binary64; the integer-dot product over 8-bit activation codes) and its
    bound S = sum_k (|d sc q4| + |dmin m|) * |d_x q| -- the plain loop of
    gemv_q4k_q8k with the tokens as its batch rows, Y laid out [tokens][rows]."""
    q = np.ascontiguousarray(np.asarray(q, dtype=np.int8).reshape(-1, K))
    d = np.ascontiguousarray(np.asarray(d, dtype=np.float32).reshape(q.shape[0], K // 256))
    if toks is not None:
        toks = np.asarray(toks, dtype=np.int64).reshape(-1)
        q, d = np.ascontiguousarray(q[toks]), np.ascontiguousarray(d[toks])
    return gemv_q4k_q8k(w, q, d, M, K, rows=rows)


def gemm_q4k_q8k_matmul(w, q, d, M: int, K: int, rows=None, toks=None):
    """gemm_q4k_q8k for large samples: the exact weight terms from q4k_terms
    (C), the activation values d_x * q exact in binary64, and every product and
    sum by numpy's binary64 matrix product (a library primitive in place of the
    loop; only the summation order differs)."""
    q = np.asarray(q, dtype=np.int8).reshape(-1, K)
    d = np.asarray(d, dtype=np.float32).reshape(q.shape[0], K // 256)
    if toks is not None:
        toks = np.asarray(toks, dtype=np.int64).reshape(-1)
        q, d = q[toks], d[toks]
    a, c = q4k_terms(w, M, K, rows=rows)
    xv = q.astype(np.float64) * np.repeat(d.astype(np.float64), 256, axis=1)
    return xv @ (a - c).T, np.abs(xv) @ (np.abs(a) + np.abs(c)).T
