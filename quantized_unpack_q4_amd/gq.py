"""ctypes binding of libgq.so: the same entry points as ``include/gq.h``.

Argument marshalling only: every step runs in the HIP kernels of libgq.so.
Tensors are torch tensors on the current HIP device (torch supplies device
memory and the current stream); binary16 data travels as ``torch.float16``
or ``torch.int16``/``torch.uint16`` bit patterns.  A missing library is an
error, never a fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgq.so")

GQ_OK = 0
GQ_EINVAL = 1
GQ_ESHAPE = 2
GQ_EALIGN = 3
GQ_EWORKSPACE = 4
GQ_EHIP = 5
MAX_BATCH = 16

EXPORTS = (
    "gq_gemv_q8_0", "gq_gemv_q4k", "gq_gemv_q4k_multi_table_bytes", "gq_gemv_q4k_multi_plan",
    "gq_gemv_q4k_multi", "gq_gemv_q4k_multi_batched", "gq_gemv_q4k_multi_batched_ws",
    "gq_gemv_q4k_multi_batched_ws_bytes", "gq_gemv_q4k_swiglu", "gq_gemv_q4k_swiglu_batched", "gq_gemm_q4k", "gq_gemm_q8_0", "gq_gemm_q4k_tiles", "gq_gemm_q8_0_tiles", "gq_gemm_q4k_kgroups", "gq_gemm_q4k_splitk",
    "gq_gemm_q4k_splitk_workspace_bytes", "gq_gemm_q4k_splitk_static",
    "gq_gemm_q4k_splitk_static_max_bytes",
    "gq_moe_gemm_q4k", "gq_moe_gemm_q4k_input_weighted", "gq_moe_gemm_q8_0",
    "gq_moe_gemm_q8_0_input_weighted", "gq_moe_route", "gq_quantize_q8k", "gq_gemv_q4k_q8k",
    "gq_gemm_q4k_q8k",
    "gq_moe_workspace_bytes", "gq_moe_workspace_offsets", "gq_dequant_q8_0",
    "gq_dequant_q4k", "gq_last_error", "gq_status_str", "gq_version",
)


class GQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libgq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libgq.so is not built (%s); run `python -m quantized_unpack_q4_amd.build`"
                % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        st = ctypes.c_int
        for name in ("gq_gemv_q8_0", "gq_gemv_q4k"):
            f = getattr(L, name)
            f.restype = st
            f.argtypes = [vp, vp, vp, i64, i64, i64, vp]
        L.gq_gemv_q4k_multi_table_bytes.restype = sz
        L.gq_gemv_q4k_multi_table_bytes.argtypes = [i64]
        L.gq_gemv_q4k_multi_plan.restype = st
        L.gq_gemv_q4k_multi_plan.argtypes = [vp, i64, vp, sz]
        L.gq_gemv_q4k_multi.restype = st
        L.gq_gemv_q4k_multi.argtypes = [vp, vp, vp]
        L.gq_gemv_q4k_multi_batched.restype = st
        L.gq_gemv_q4k_multi_batched.argtypes = [vp, vp, i64, vp]
        L.gq_gemm_q4k.restype = st
        L.gq_gemm_q4k.argtypes = [vp, vp, vp, i64, i64, i64, vp]
        L.gq_gemv_q4k_swiglu.restype = st
        L.gq_gemv_q4k_swiglu.argtypes = [vp, vp, vp, vp, i64, i64, vp]
        L.gq_gemm_q4k_splitk.restype = st
        L.gq_gemm_q4k_splitk.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp, sz, vp]
        L.gq_gemm_q4k_splitk_static.restype = st
        L.gq_gemm_q4k_splitk_static.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp]
        L.gq_gemm_q4k_splitk_static_max_bytes.restype = sz
        L.gq_gemm_q4k_splitk_static_max_bytes.argtypes = []
        L.gq_gemm_q4k_splitk_workspace_bytes.restype = sz
        L.gq_gemm_q4k_splitk_workspace_bytes.argtypes = [i64, i64, i64, i64]
        L.gq_gemm_q8_0.restype = st
        L.gq_gemm_q8_0.argtypes = [vp, vp, vp, i64, i64, i64, vp]
        L.gq_gemm_q4k_tiles.restype = st
        L.gq_gemm_q4k_tiles.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp]
        L.gq_gemm_q8_0_tiles.restype = st
        L.gq_gemm_q8_0_tiles.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp]
        L.gq_gemv_q4k_multi_batched_ws.restype = st
        L.gq_gemv_q4k_multi_batched_ws.argtypes = [vp, vp, i64, vp, sz, vp]
        L.gq_gemv_q4k_multi_batched_ws_bytes.restype = sz
        L.gq_gemv_q4k_multi_batched_ws_bytes.argtypes = [vp, i64]
        L.gq_gemv_q4k_swiglu_batched.restype = st
        L.gq_gemv_q4k_swiglu_batched.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
        L.gq_gemm_q4k_kgroups.restype = st
        L.gq_gemm_q4k_kgroups.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp]
        for name in ("gq_moe_gemm_q4k", "gq_moe_gemm_q4k_input_weighted", "gq_moe_gemm_q8_0",
                     "gq_moe_gemm_q8_0_input_weighted"):
            f = getattr(L, name)
            f.restype = st
            f.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, sz, vp]
        L.gq_quantize_q8k.restype = st
        L.gq_quantize_q8k.argtypes = [vp, vp, vp, vp, i64, i64, vp]
        L.gq_gemm_q4k_q8k.restype = st
        L.gq_gemm_q4k_q8k.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
        L.gq_gemv_q4k_q8k.restype = st
        L.gq_gemv_q4k_q8k.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp]
        L.gq_moe_route.restype = st
        L.gq_moe_route.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp]
        L.gq_moe_workspace_bytes.restype = sz
        L.gq_moe_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
        L.gq_moe_workspace_offsets.restype = st
        L.gq_moe_workspace_offsets.argtypes = [i64, i64, i64, i64, i64, ctypes.POINTER(sz)]
        for name in ("gq_dequant_q8_0", "gq_dequant_q4k"):
            f = getattr(L, name)
            f.restype = st
            f.argtypes = [vp, vp, vp, i64, i64, vp]
        L.gq_last_error.restype = ctypes.c_char_p
        L.gq_last_error.argtypes = []
        L.gq_status_str.restype = ctypes.c_char_p
        L.gq_status_str.argtypes = [st]
        L.gq_version.restype = ctypes.c_int
        L.gq_version.argtypes = []
        _lib = L
    return _lib


def last_error() -> str:
    return lib().gq_last_error().decode()


def _check(status: int) -> None:
    if status != GQ_OK:
        raise GQError(status, "%s: %s" % (lib().gq_status_str(status).decode(), last_error()))


def _ptr(t):
    """Device address of a tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libgq must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


# -- raw entry points (same names as the C ABI) ---------------------------------

def gq_gemv_q8_0(w, x, y, M, K, B, stream=None):
    _check(lib().gq_gemv_q8_0(_ptr(w), _ptr(x), _ptr(y), M, K, B, _stream(stream)))


def gq_gemv_q4k(w, x, y, M, K, B, stream=None):
    _check(lib().gq_gemv_q4k(_ptr(w), _ptr(x), _ptr(y), M, K, B, _stream(stream)))


class GemvDesc(ctypes.Structure):
    """Mirror of gq_gemv_desc."""
    _fields_ = [("w", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("K", ctypes.c_int64)]


def gq_gemv_q4k_multi_table_bytes(n) -> int:
    return int(lib().gq_gemv_q4k_multi_table_bytes(n))


def gq_gemv_q4k_multi_plan(descs, n, table, table_bytes):
    _check(lib().gq_gemv_q4k_multi_plan(descs, n, table, table_bytes))


def gq_gemv_q4k_multi(table, table_dev, stream=None):
    _check(lib().gq_gemv_q4k_multi(table, _ptr(table_dev), _stream(stream)))


def gq_gemv_q4k_multi_batched(table, table_dev, B, stream=None):
    _check(lib().gq_gemv_q4k_multi_batched(table, _ptr(table_dev), B, _stream(stream)))


class GemvTable:
    """A planned multi-product: host table + its device copy.

    ``items`` is a list of (w, x, y, M, K) with torch device tensors, x of
    shape [batch][K] and y [batch][M]; the tensors must stay alive while the
    table is used.
    """

    def __init__(self, items, batch=1, prestaged=False):
        import torch
        n = len(items)
        arr = (GemvDesc * n)()
        for i, (w, x, y, M, K) in enumerate(items):
            for t in (w, x, y):
                if not t.is_contiguous():
                    raise ValueError("tensors passed to libgq must be contiguous")
            arr[i] = GemvDesc(w.data_ptr(), x.data_ptr(), y.data_ptr(), M, K)
        nbytes = gq_gemv_q4k_multi_table_bytes(n)
        if nbytes == 0:
            raise ValueError("bad table size n=%d" % n)
        self.host = (ctypes.c_uint8 * nbytes)()
        gq_gemv_q4k_multi_plan(arr, n, self.host, nbytes)
        host_t = torch.frombuffer(bytearray(bytes(self.host)), dtype=torch.uint8)
        self.dev = host_t.to(items[0][0].device)
        self.items = items
        self.n = n
        self.batch = batch
        # prestaged: batch 2-16 with the activations staged once per product
        # into a workspace owned by the table (gq_gemv_q4k_multi_batched_ws)
        self.ws = None
        if prestaged and batch >= 2:
            nws = gq_gemv_q4k_multi_batched_ws_bytes(self.host, batch)
            if nws == 0:
                raise ValueError("table not valid at batch %d" % batch)
            self.ws = torch.empty(nws, dtype=torch.uint8, device=items[0][0].device)

    def run(self, stream=None):
        if self.batch == 1:
            gq_gemv_q4k_multi(self.host, self.dev, stream)
        elif self.ws is not None:
            gq_gemv_q4k_multi_batched_ws(self.host, self.dev, self.batch, self.ws,
                                         self.ws.numel(), stream)
        else:
            gq_gemv_q4k_multi_batched(self.host, self.dev, self.batch, stream)


def gq_gemv_q4k_multi_batched_ws_bytes(table, B) -> int:
    return lib().gq_gemv_q4k_multi_batched_ws_bytes(table, B)


def gq_gemv_q4k_multi_batched_ws(table, table_dev, B, ws, ws_bytes, stream=None):
    _check(lib().gq_gemv_q4k_multi_batched_ws(table, _ptr(table_dev), B, _ptr(ws), ws_bytes,
                                              _stream(stream)))


def gq_gemm_q4k(w, x, y, M, K, N, stream=None):
    _check(lib().gq_gemm_q4k(_ptr(w), _ptr(x), _ptr(y), M, K, N, _stream(stream)))


def gq_gemm_q8_0(w, x, y, M, K, N, stream=None):
    _check(lib().gq_gemm_q8_0(_ptr(w), _ptr(x), _ptr(y), M, K, N, _stream(stream)))


def gq_gemm_q4k_tiles(w, x, y, M, K, N, tile_rows, stream=None):
    _check(lib().gq_gemm_q4k_tiles(_ptr(w), _ptr(x), _ptr(y), M, K, N, tile_rows,
                                   _stream(stream)))


def gq_gemm_q8_0_tiles(w, x, y, M, K, N, tile_rows, stream=None):
    _check(lib().gq_gemm_q8_0_tiles(_ptr(w), _ptr(x), _ptr(y), M, K, N, tile_rows,
                                    _stream(stream)))


def gq_gemv_q4k_swiglu_batched(w_gate, w_up, x, h, M, K, B, stream=None):
    _check(lib().gq_gemv_q4k_swiglu_batched(_ptr(w_gate), _ptr(w_up), _ptr(x), _ptr(h), M, K, B,
                                            _stream(stream)))


def gq_gemm_q4k_kgroups(w, x, y, M, K, N, groups, stream=None):
    _check(lib().gq_gemm_q4k_kgroups(_ptr(w), _ptr(x), _ptr(y), M, K, N, groups,
                                     _stream(stream)))


def gq_gemv_q4k_swiglu(w_gate, w_up, x, h, M, K, stream=None):
    _check(lib().gq_gemv_q4k_swiglu(_ptr(w_gate), _ptr(w_up), _ptr(x), _ptr(h), M, K,
                                    _stream(stream)))


def gq_gemm_q4k_splitk_workspace_bytes(M, K, N, splits=0) -> int:
    return lib().gq_gemm_q4k_splitk_workspace_bytes(M, K, N, splits)


def gq_gemm_q4k_splitk(w, x, y, M, K, N, splits, ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().gq_gemm_q4k_splitk(_ptr(w), _ptr(x), _ptr(y), M, K, N, splits, _ptr(ws),
                                    ws_bytes, _stream(stream)))


def gq_gemm_q4k_splitk_static(w, x, y, M, K, N, splits=0, stream=None):
    _check(lib().gq_gemm_q4k_splitk_static(_ptr(w), _ptr(x), _ptr(y), M, K, N, splits,
                                           _stream(stream)))


def gq_gemm_q4k_splitk_static_max_bytes() -> int:
    return lib().gq_gemm_q4k_splitk_static_max_bytes()


def gq_moe_workspace_bytes(T, H, I, E, topk) -> int:
    return int(lib().gq_moe_workspace_bytes(T, H, I, E, topk))


def gq_moe_workspace_offsets(T, H, I, E, topk):
    off = (ctypes.c_size_t * 7)()
    _check(lib().gq_moe_workspace_offsets(T, H, I, E, topk, off))
    return list(off)


def gq_moe_gemm_q4k(w_gate, w_up, w_down, x, topk_ids, topk_w, out, T, H, I, E, topk, ws,
                    ws_bytes=None, stream=None, input_weighted=False):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    f = lib().gq_moe_gemm_q4k_input_weighted if input_weighted else lib().gq_moe_gemm_q4k
    _check(f(_ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(x), _ptr(topk_ids), _ptr(topk_w),
             _ptr(out), T, H, I, E, topk, _ptr(ws), ws_bytes, _stream(stream)))


def gq_moe_gemm_q8_0(w_gate, w_up, w_down, x, topk_ids, topk_w, out, T, H, I, E, topk, ws,
                     ws_bytes=None, stream=None, input_weighted=False):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    f = lib().gq_moe_gemm_q8_0_input_weighted if input_weighted else lib().gq_moe_gemm_q8_0
    _check(f(_ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(x), _ptr(topk_ids), _ptr(topk_w),
             _ptr(out), T, H, I, E, topk, _ptr(ws), ws_bytes, _stream(stream)))


def gq_quantize_q8k(x, q, d, bsum, B, K, stream=None):
    _check(lib().gq_quantize_q8k(_ptr(x), _ptr(q), _ptr(d), _ptr(bsum), B, K, _stream(stream)))


def gq_gemv_q4k_q8k(w, q, d, bsum, y, M, K, B, stream=None):
    _check(lib().gq_gemv_q4k_q8k(_ptr(w), _ptr(q), _ptr(d), _ptr(bsum), _ptr(y), M, K, B,
                                 _stream(stream)))


def gq_gemm_q4k_q8k(w, q, d, y, M, K, N, stream=None):
    _check(lib().gq_gemm_q4k_q8k(_ptr(w), _ptr(q), _ptr(d), _ptr(y), M, K, N, _stream(stream)))


def gq_dequant_q8_0(w, out32, out16, M, K, stream=None):
    _check(lib().gq_dequant_q8_0(_ptr(w), _ptr(out32), _ptr(out16), M, K, _stream(stream)))


def gq_dequant_q4k(w, out32, out16, M, K, stream=None):
    _check(lib().gq_dequant_q4k(_ptr(w), _ptr(out32), _ptr(out16), M, K, _stream(stream)))


def gq_version() -> int:
    return int(lib().gq_version())


# -- tensor-level helpers (allocate outputs with torch, then call the ABI) -------

def q4k_row_bytes(K: int) -> int:
    return K // 256 * 144


def q8_0_row_bytes(K: int) -> int:
    return K // 32 * 34


def gemv_q4k(w, x, M: int, K: int, out=None, stream=None):
    """y[B][M] = x[B][K] * W^T for packed Q4_K w (uint8 device tensor)."""
    import torch
    x2 = x.reshape(-1, K)
    B = x2.shape[0]
    y = out if out is not None else torch.empty((B, M), dtype=torch.float32, device=x.device)
    gq_gemv_q4k(w, x2, y, M, K, B, stream)
    return y


def gemv_q8_0(w, x, M: int, K: int, out=None, stream=None):
    import torch
    x2 = x.reshape(-1, K)
    B = x2.shape[0]
    y = out if out is not None else torch.empty((B, M), dtype=torch.float32, device=x.device)
    gq_gemv_q8_0(w, x2, y, M, K, B, stream)
    return y


def gemm_q4k(w, x16, M: int, K: int, out=None, stream=None):
    """Y[N][M] (float16) = X[N][K] (float16) * W^T."""
    import torch
    x2 = x16.reshape(-1, K)
    N = x2.shape[0]
    y = out if out is not None else torch.empty((N, M), dtype=torch.float16, device=x16.device)
    gq_gemm_q4k(w, x2, y, M, K, N, stream)
    return y


def gq_moe_route(logits, topk_ids, topk_w, T, E, topk, renormalize=0, stream=None):
    _check(lib().gq_moe_route(_ptr(logits), _ptr(topk_ids), _ptr(topk_w), T, E, topk,
                              int(renormalize), _stream(stream)))


def moe_route(logits, topk: int, renormalize=False, stream=None):
    """Top-k expert routing of logits [T][E] (float32): (ids int32, weights float32)."""
    import torch
    T, E = logits.shape
    ids = torch.empty((T, topk), dtype=torch.int32, device=logits.device)
    wts = torch.empty((T, topk), dtype=torch.float32, device=logits.device)
    gq_moe_route(logits, ids, wts, T, E, topk, renormalize, stream)
    return ids, wts


def moe_q4k(w_gate, w_up, w_down, x16, topk_ids, topk_w, H: int, I: int, E: int, ws=None,
            out=None, stream=None, input_weighted=False, q8_0=False):
    """Mixture-of-experts feed-forward; returns (out [T][H] float16, workspace).
    q8_0: the weight stacks are Q8_0 instead of Q4_K."""
    import torch
    T, topk = topk_ids.shape
    need = gq_moe_workspace_bytes(T, H, I, E, topk)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=x16.device)
    o = out if out is not None else torch.empty((T, H), dtype=torch.float16, device=x16.device)
    f = gq_moe_gemm_q8_0 if q8_0 else gq_moe_gemm_q4k
    f(w_gate, w_up, w_down, x16, topk_ids, topk_w, o, T, H, I, E, topk, ws, stream=stream,
      input_weighted=input_weighted)
    return o, ws


def dequant(fmt: str, w, M: int, K: int, want32=True, want16=True, stream=None):
    import torch
    dev = w.device
    o32 = torch.empty((M, K), dtype=torch.float32, device=dev) if want32 else None
    o16 = torch.empty((M, K), dtype=torch.float16, device=dev) if want16 else None
    if fmt == "q4k":
        gq_dequant_q4k(w, o32, o16, M, K, stream)
    elif fmt == "q8_0":
        gq_dequant_q8_0(w, o32, o16, M, K, stream)
    else:
        raise ValueError("unknown format %r" % fmt)
    return o32, o16


def quantize_q8k(x, stream=None):
    """x [B][K] float32 -> (q int8 [B][K], d float32 [B][K/256], bsum int32 [B][K/32])."""
    import torch
    B, K = x.shape
    q = torch.empty((B, K), dtype=torch.int8, device=x.device)
    d = torch.empty((B, K // 256), dtype=torch.float32, device=x.device)
    bs = torch.empty((B, K // 32), dtype=torch.int32, device=x.device)
    gq_quantize_q8k(x, q, d, bs, B, K, stream)
    return q, d, bs
