"""CPU oracle for MoE routing layout, dispatch copy and combine.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It wraps the plain C
definitions in ``ep_oracle.c`` (built with gcc; single-threaded unless
``set_threads`` asks for more on the token loops of dispatch and combine, for
the benchmark's all-cores leg) and shares no
code with the HIP library.  Arrays are numpy, on the host.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ep_oracle.c")
_LIB = os.path.join(_HERE, "libep_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-Wextra"]

ERR_CAPACITY = 1
ERR_ARGS = 2


def build(src: str = _SRC, out: str = _LIB, extra=()) -> str:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = f"{out}.tmp{os.getpid()}"
    subprocess.run(["gcc", *CFLAGS, *extra, "-o", tmp, src], check=True)
    os.replace(tmp, out)
    return out


_P = ctypes.c_void_p
_I = ctypes.c_int64


def _bind(lib):
    lib.oracle_set_threads.restype = None
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_capacity_bound.restype = _I
    lib.oracle_capacity_bound.argtypes = [_I, _I, _I, _I]
    lib.oracle_layout.restype = ctypes.c_int
    lib.oracle_layout.argtypes = [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]
    lib.oracle_dispatch.restype = None
    lib.oracle_dispatch.argtypes = [_I, _I, _I, _I, _P, _I, _P, _I, _I, _P,
                                    _P, _P, _P, _P, _P, _I, _I, _P, ctypes.c_int]
    lib.oracle_combine.restype = None
    lib.oracle_combine.argtypes = [_I, _I, _I, _P, _P, _P, _P, _P, _P]
    lib.oracle_combine_f64.restype = None
    lib.oracle_combine_f64.argtypes = [_I, _I, _I, _P, _P, _P, _P, _P, _P, _P]
    lib.oracle_combine_backward.restype = None
    lib.oracle_combine_backward.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P,
                                            _P, _P, _P, _P]
    lib.oracle_dispatch_backward.restype = None
    lib.oracle_dispatch_backward.argtypes = [_I, _I, _I, _P, _P, _P, _P, _P, _P]
    lib.oracle_rank_layout.restype = _I
    lib.oracle_rank_layout.argtypes = [_I, _I, _I, _P, _P, _P]
    lib.oracle_dispatch_rank.restype = None
    lib.oracle_dispatch_rank.argtypes = [_I, _I, _I, _I, _P, _I, _P, _I, _I, _P, _P, _P, _P,
                                         _P, _I, _I, _P, _P]
    lib.oracle_combine_rank.restype = None
    lib.oracle_combine_rank.argtypes = [_I, _I, _P, _P, _P, _P, _P]
    lib.oracle_combine_token_bias.restype = None
    lib.oracle_combine_token_bias.argtypes = [_I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.oracle_f32_to_e4m3.restype = None
    lib.oracle_f32_to_e4m3.argtypes = [_I, _P, _P]
    lib.oracle_sf_packs.restype = _I
    lib.oracle_sf_packs.argtypes = [_I, ctypes.c_int]
    lib.oracle_quantize_fp8.restype = None
    lib.oracle_quantize_fp8.argtypes = [_I, _I, _P, ctypes.c_int, _P, _P, _I, _I]
    lib.oracle_dispatch_quant.restype = None
    lib.oracle_dispatch_quant.argtypes = [_I, _I, _I, _I, _P, ctypes.c_int, _P, _P, _P, _P,
                                          _P, _P, _I, _I, _P, ctypes.c_int]
    return lib


_lib = None


def load(path: Optional[str] = None):
    """Load the built oracle (building it first if it is absent)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def set_threads(threads: int, lib=None) -> None:
    """Threads of the token loops of dispatch and the combines (1 = the plain
    sequential loops; results are identical for any count)."""
    (lib or load()).oracle_set_threads(int(threads))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class Layout:
    """Result of :func:`layout`; arrays are numpy int32, scalars Python ints."""

    def __init__(self, status, counts, psum, dst, src_meta, num_recv_tokens,
                 invalid_count, num_expanded):
        self.status = status
        self.counts = counts
        self.psum = psum
        self.dst = dst
        self.src_meta = src_meta
        self.num_recv_tokens = num_recv_tokens
        self.invalid_count = invalid_count
        self.num_expanded = num_expanded


def capacity_bound(T, K, E, A, lib=None) -> int:
    return int((lib or load()).oracle_capacity_bound(T, K, E, A))


def layout(topk_idx, num_experts: int, alignment: int, capacity: int,
           lib=None) -> Layout:
    """topk_idx: integer [T, K] (int32 is widened to int64)."""
    lib = lib or load()
    idx = _c(topk_idx, np.int64)
    T, K = idx.shape
    counts = np.zeros(num_experts, np.int32)
    psum = np.zeros(num_experts + 1, np.int32)
    dst = np.full(T * K, -7, np.int32)
    src = np.full(max(capacity, 1), -7, np.int32)
    sc = np.zeros(3, np.int64)
    st = lib.oracle_layout(T, K, num_experts, alignment, capacity, _ptr(idx),
                           _ptr(counts), _ptr(psum), _ptr(dst), _ptr(src),
                           _ptr(sc))
    return Layout(int(st), counts, psum, dst.reshape(T, K), src[:capacity],
                  int(sc[0]), int(sc[1]), int(sc[2]))


def dispatch(x_bytes: np.ndarray, lay: Layout, capacity: int,
             sf: Optional[np.ndarray] = None, sf_strides=None,
             weights: Optional[np.ndarray] = None, want_w: bool = False,
             zero_padding: bool = False, out_x=None, out_sf=None,
             out_sf_strides=None, out_w=None, num_sf_packs=None, lib=None):
    """x_bytes: uint8 [T, row_bytes] (the raw row bytes of bf16 or FP8 x).

    Outputs may be passed in (pre-filled, e.g. with a poison pattern) to show
    which rows are left untouched; otherwise they are zero-initialised.
    ``sf`` holds 4-byte scale packs (float32, or int32/uint32 packed
    exponents), addressed with (token, pack) element strides; there are
    ``num_sf_packs`` per token (default row_bytes / 128, one fp32 per block).
    """
    lib = lib or load()
    x = np.ascontiguousarray(x_bytes, dtype=np.uint8)
    T, row_bytes = x.shape
    K = lay.dst.shape[1]
    E = lay.counts.shape[0]
    if out_x is None:
        out_x = np.zeros((capacity, row_bytes), np.uint8)
    num_sf = 0
    ts = hs = ots = ohs = 0
    sf_arr = None
    if sf is not None:
        sf_arr = np.asarray(sf)
        assert sf_arr.dtype.itemsize == 4 and sf_arr.flags.c_contiguous
        ts, hs = sf_strides if sf_strides is not None else (sf_arr.shape[1], 1)
        num_sf = num_sf_packs or row_bytes // 128
        if out_sf is None:
            out_sf = np.zeros((capacity, num_sf), sf_arr.dtype)
        assert out_sf.dtype.itemsize == 4 and out_sf.flags.c_contiguous
        ots, ohs = out_sf_strides if out_sf_strides is not None else (num_sf, 1)
    if want_w and out_w is None:
        out_w = np.zeros(capacity, np.float32)
    w = None if weights is None else _c(weights, np.float32)
    lib.oracle_dispatch(T, K, E, row_bytes, _ptr(x), num_sf, _ptr(sf_arr),
                        ts, hs, _ptr(w), _ptr(lay.counts), _ptr(lay.psum),
                        _ptr(_c(lay.dst, np.int32)), _ptr(out_x),
                        _ptr(out_sf), ots, ohs, _ptr(out_w),
                        1 if zero_padding else 0)
    return out_x, out_sf, out_w


def combine(y_bits: np.ndarray, topk_idx, dst, weights=None, bias_bits=None,
            lib=None) -> np.ndarray:
    """y_bits: uint16 [rows, H] bf16 bit patterns; returns uint16 [T, H]."""
    lib = lib or load()
    y = _c(y_bits, np.uint16)
    idx = _c(topk_idx, np.int64)
    d = _c(dst, np.int32)
    T, K = idx.shape
    H = y.shape[1]
    out = np.zeros((T, H), np.uint16)
    w = None if weights is None else _c(weights, np.float32)
    b = None if bias_bits is None else _c(bias_bits, np.uint16)
    lib.oracle_combine(T, K, H, _ptr(y), _ptr(w), _ptr(b), _ptr(idx), _ptr(d),
                       _ptr(out))
    return out


def combine_f64(y_bits, topk_idx, dst, weights=None, bias_bits=None, lib=None):
    """binary64 weighted sums and sums of |term|, both float64 [T, H]."""
    lib = lib or load()
    y = _c(y_bits, np.uint16)
    idx = _c(topk_idx, np.int64)
    d = _c(dst, np.int32)
    T, K = idx.shape
    H = y.shape[1]
    out = np.zeros((T, H), np.float64)
    mag = np.zeros((T, H), np.float64)
    w = None if weights is None else _c(weights, np.float32)
    b = None if bias_bits is None else _c(bias_bits, np.uint16)
    lib.oracle_combine_f64(T, K, H, _ptr(y), _ptr(w), _ptr(b), _ptr(idx),
                           _ptr(d), _ptr(out), _ptr(mag))
    return out, mag


def combine_backward(g_bits, lay: Layout, topk_idx, weights=None, y_bits=None, bias_bits=None,
                     capacity=None, want_grad_y=True, want_grad_w=True, want_grad_bias=False,
                     grad_y=None, lib=None):
    """Backward of combine.  g_bits: uint16 [T, H] (bf16 gradient of out).
    Returns (grad_y uint16 [capacity, H] or None, grad_w float64 [T, K] or
    None, grad_bias float64 [E, H] or None); the float64 outputs are binary64
    reference sums.  grad_y may be passed pre-filled
    (rows without a slot keep their content)."""
    lib = lib or load()
    g = _c(g_bits, np.uint16)
    idx = _c(topk_idx, np.int64)
    T, K = idx.shape
    H = g.shape[1]
    E = lay.counts.shape[0]
    w = None if weights is None else _c(weights, np.float32)
    y = None if y_bits is None else _c(y_bits, np.uint16)
    b = None if bias_bits is None else _c(bias_bits, np.uint16)
    gy = None
    if want_grad_y:
        gy = grad_y if grad_y is not None else np.zeros((capacity, H), np.uint16)
    gw = np.zeros((T, K), np.float64) if want_grad_w else None
    gb = np.zeros((E, H), np.float64) if want_grad_bias else None
    if want_grad_w:
        assert y is not None, "grad_w needs the expert outputs y"
    src = _c(lay.src_meta, np.int32)
    lib.oracle_combine_backward(T, K, E, H, _ptr(g), _ptr(w), _ptr(y), _ptr(b), _ptr(idx),
                                _ptr(_c(lay.dst, np.int32)), _ptr(lay.counts), _ptr(lay.psum),
                                _ptr(src), _ptr(gy), _ptr(gw), _ptr(gb))
    return gy, gw, gb


def dispatch_backward(go_bits, topk_idx, dst, gw=None, lib=None):
    """Backward of dispatch.  go_bits: uint16 [capacity, H]; gw: float32
    [capacity] or None.  Returns (grad_x uint16 [T, H], grad_w float32 [T, K])."""
    lib = lib or load()
    go = _c(go_bits, np.uint16)
    idx = _c(topk_idx, np.int64)
    d = _c(dst, np.int32)
    T, K = idx.shape
    H = go.shape[1]
    gx = np.zeros((T, H), np.uint16)
    gwo = np.zeros((T, K), np.float32)
    g = None if gw is None else _c(gw, np.float32)
    lib.oracle_dispatch_backward(T, K, H, _ptr(go), _ptr(g), _ptr(idx), _ptr(d), _ptr(gx),
                                 _ptr(gwo))
    return gx, gwo


def rank_layout(topk_idx, num_experts: int, lib=None):
    """Returns (recv_row int32 [T], recv_src int32 [num_recv], num_recv)."""
    lib = lib or load()
    idx = _c(topk_idx, np.int64)
    T, K = idx.shape
    row = np.full(T, -7, np.int32)
    src = np.full(max(T, 1), -7, np.int32)
    n = int(lib.oracle_rank_layout(T, K, num_experts, _ptr(idx), _ptr(row), _ptr(src)))
    return row, src[:n], n


def dispatch_rank(x_bytes, topk_idx, num_experts, recv_row, rows, sf=None, sf_strides=None,
                  weights=None, out_x=None, out_sf=None, out_idx=None, out_w=None,
                  num_sf_packs=None, lib=None):
    """Rank-layout dispatch; outputs have ``rows`` rows (pre-fill to check
    untouched rows).  Returns (out_x, out_sf, out_idx int64 [rows, K],
    out_w float32 [rows, K])."""
    lib = lib or load()
    x = np.ascontiguousarray(x_bytes, dtype=np.uint8)
    idx = _c(topk_idx, np.int64)
    T, K = idx.shape
    R = x.shape[1]
    if out_x is None:
        out_x = np.zeros((rows, R), np.uint8)
    num_sf = ts = hs = ots = ohs = 0
    sf_arr = None
    if sf is not None:
        sf_arr = np.asarray(sf)
        assert sf_arr.dtype.itemsize == 4 and sf_arr.flags.c_contiguous
        ts, hs = sf_strides if sf_strides is not None else (sf_arr.shape[1], 1)
        num_sf = num_sf_packs or R // 128
        if out_sf is None:
            out_sf = np.zeros((rows, num_sf), sf_arr.dtype)
        ots, ohs = num_sf, 1
    if out_idx is None:
        out_idx = np.zeros((rows, K), np.int64)
    if out_w is None:
        out_w = np.zeros((rows, K), np.float32)
    w = None if weights is None else _c(weights, np.float32)
    lib.oracle_dispatch_rank(T, K, num_experts, R, _ptr(x), num_sf, _ptr(sf_arr), ts, hs,
                             _ptr(w), _ptr(idx), _ptr(_c(recv_row, np.int32)), _ptr(out_x),
                             _ptr(out_sf), ots, ohs, _ptr(out_idx), _ptr(out_w))
    return out_x, out_sf, out_idx, out_w


def combine_rank(x_bits, recv_row, b0_bits=None, b1_bits=None, lib=None):
    """x_bits: uint16 [rows, H]; returns uint16 [T, H]."""
    lib = lib or load()
    x = _c(x_bits, np.uint16)
    row = _c(recv_row, np.int32)
    T = row.shape[0]
    H = x.shape[1]
    out = np.zeros((T, H), np.uint16)
    b0 = None if b0_bits is None else _c(b0_bits, np.uint16)
    b1 = None if b1_bits is None else _c(b1_bits, np.uint16)
    lib.oracle_combine_rank(T, H, _ptr(x), _ptr(row), _ptr(b0), _ptr(b1), _ptr(out))
    return out


def combine_token_bias(y_bits, topk_idx, dst, weights=None, bias_bits=None, b0_bits=None,
                       b1_bits=None, lib=None):
    """Expanded combine plus per-token biases bias_0, bias_1 (uint16 [T, H])."""
    lib = lib or load()
    y = _c(y_bits, np.uint16)
    idx = _c(topk_idx, np.int64)
    d = _c(dst, np.int32)
    T, K = idx.shape
    H = y.shape[1]
    out = np.zeros((T, H), np.uint16)
    w = None if weights is None else _c(weights, np.float32)
    b = None if bias_bits is None else _c(bias_bits, np.uint16)
    b0 = None if b0_bits is None else _c(b0_bits, np.uint16)
    b1 = None if b1_bits is None else _c(b1_bits, np.uint16)
    lib.oracle_combine_token_bias(T, K, H, _ptr(y), _ptr(w), _ptr(b), _ptr(idx), _ptr(d),
                                  _ptr(b0), _ptr(b1), _ptr(out))
    return out


SF_F32 = 0
SF_UE8M0 = 1


def sf_packs(H: int, fmt: int, lib=None) -> int:
    lib = lib or load()
    return int(lib.oracle_sf_packs(H, fmt))


def f32_to_e4m3(values, lib=None) -> np.ndarray:
    """E4M3FN codes (uint8) of binary32 values, nearest with ties to even."""
    lib = lib or load()
    v = _c(values, np.float32)
    out = np.zeros(v.shape, np.uint8)
    lib.oracle_f32_to_e4m3(v.size, _ptr(v), _ptr(out))
    return out


def quantize_fp8(x_bits, fmt=SF_F32, lib=None):
    """x_bits: uint16 [T, H] bf16.  Returns (codes uint8 [T, H], packs uint32
    [T, sf_packs(H, fmt)])."""
    lib = lib or load()
    x = _c(x_bits, np.uint16)
    T, H = x.shape
    P = sf_packs(H, fmt, lib)
    q = np.zeros((T, H), np.uint8)
    sf = np.zeros((T, P), np.uint32)
    lib.oracle_quantize_fp8(T, H, _ptr(x), fmt, _ptr(q), _ptr(sf), P, 1)
    return q, sf


def dispatch_quant(x_bits, lay: Layout, capacity: int, fmt=SF_F32, weights=None,
                   want_w: bool = False, zero_padding: bool = False, out_x=None, out_sf=None,
                   out_sf_strides=None, out_w=None, lib=None):
    """Quantise bf16 rows then dispatch the codes and packs.  Outputs may be
    passed pre-filled (untouched rows keep their content)."""
    lib = lib or load()
    x = _c(x_bits, np.uint16)
    T, H = x.shape
    K = lay.dst.shape[1]
    E = lay.counts.shape[0]
    P = sf_packs(H, fmt, lib)
    if out_x is None:
        out_x = np.zeros((capacity, H), np.uint8)
    if out_sf is None:
        out_sf = np.zeros((capacity, P), np.uint32)
    assert out_sf.dtype.itemsize == 4 and out_sf.flags.c_contiguous
    ots, ohs = out_sf_strides if out_sf_strides is not None else (P, 1)
    if want_w and out_w is None:
        out_w = np.zeros(capacity, np.float32)
    w = None if weights is None else _c(weights, np.float32)
    lib.oracle_dispatch_quant(T, K, E, H, _ptr(x), fmt, _ptr(w), _ptr(lay.counts),
                              _ptr(lay.psum), _ptr(_c(lay.dst, np.int32)), _ptr(out_x),
                              _ptr(out_sf), ots, ohs, _ptr(out_w), 1 if zero_padding else 0)
    return out_x, out_sf, out_w

