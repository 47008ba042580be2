"""Independent brute-force statements of layout, dispatch and combine.

These are written separately from the C oracle (different language, different
formulation) and serve only to pin it: a mistake in the oracle shows up as a
disagreement with one of these on small inputs.  They follow the same pages:
DeepEP notes chapter 7 "V2: how dispatch builds expert inputs" (sections 7.1
to 7.5) and chapter 8 "V2: combine, handle and async overlap" (section 8.1).
"""
from __future__ import annotations

import numpy as np
import torch


def layout_sorted(topk_idx: np.ndarray, E: int, A: int):
    """Layout by sorting: valid slots ordered by (expert, slot index), each
    expert's run placed at the next multiple of A after the previous run.

    Returns (counts, psum, dst, src_meta_prefix, num_recv, invalid) where
    src_meta_prefix covers rows [0, psum[E]).
    """
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, K = idx.shape
    flat = idx.reshape(-1).tolist()
    valid = [(e, i) for i, e in enumerate(flat) if 0 <= e < E]
    invalid = sum(1 for e in flat if e != -1 and not (0 <= e < E))
    valid.sort()
    counts = [0] * E
    for e, _ in valid:
        counts[e] += 1
    psum = [0]
    for e in range(E):
        psum.append(psum[-1] + -(-counts[e] // A) * A)
    dst = [-1] * (T * K)
    src = [-1] * psum[-1]
    seen = [0] * E
    for e, i in valid:
        r = psum[e] + seen[e]
        seen[e] += 1
        dst[i] = r
        src[r] = i
    num_recv = sum(1 for t in range(T)
                   if any(0 <= flat[t * K + k] < E for k in range(K)))
    return (np.array(counts, np.int32), np.array(psum, np.int64),
            np.array(dst, np.int64).reshape(T, K), np.array(src, np.int64),
            num_recv, invalid)


def layout_argsort_a1(topk_idx: np.ndarray, E: int):
    """Alignment-1 special case through library routines: the expanded order
    is numpy's stable argsort of the expert ids over valid slots, and psum is
    the cumulative sum of bincount."""
    flat = np.asarray(topk_idx, np.int64).reshape(-1)
    ok = (flat >= 0) & (flat < E)
    slots = np.nonzero(ok)[0]
    order = slots[np.argsort(flat[slots], kind="stable")]
    counts = np.bincount(flat[slots], minlength=E)
    psum = np.concatenate([[0], np.cumsum(counts)])
    dst = np.full(flat.shape, -1, np.int64)
    dst[order] = np.arange(order.size)
    return counts, psum, dst.reshape(np.asarray(topk_idx).shape), order


def dispatch_expected(x_bytes, dst, counts, psum, capacity, poison=0xA5,
                      sf=None, weights=None, zero_padding=False):
    """Closed form of the expanded copy: row dst[t,k] equals row t of x, gap
    rows are zero when padding is requested, every other row keeps the poison
    byte.  Returns (out_x, out_sf, out_w)."""
    x = np.asarray(x_bytes, np.uint8)
    T, R = x.shape
    K = dst.shape[1]
    out = np.full((capacity, R), poison, np.uint8)
    pf = np.frombuffer(bytes([poison] * 4), np.float32)[0]
    nsf = 0 if sf is None else sf.shape[1]
    sdt = np.float32 if sf is None else sf.dtype          # 4-byte packs, kept as bits
    osf = np.full((capacity, nsf), np.frombuffer(bytes([poison] * 4), sdt)[0], sdt)
    ow = np.full(capacity, pf, np.float32)
    d = np.asarray(dst).reshape(T, K)
    tt, kk = np.nonzero(d >= 0)
    rows = d[tt, kk]
    out[rows] = x[tt]
    if nsf:
        osf[rows] = sf[tt]
    ow[rows] = 1.0 if weights is None else np.asarray(weights, np.float32)[tt, kk]
    if zero_padding:
        for e in range(len(counts)):
            g0, g1 = int(psum[e]) + int(counts[e]), int(psum[e + 1])
            out[g0:g1] = 0
            osf[g0:g1] = 0
            ow[g0:g1] = 0.0
    return out, osf, ow


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits_torch(a: np.ndarray) -> np.ndarray:
    """Round binary32 to bf16 with torch's conversion (nearest, ties to even)."""
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def combine_f32(y_bits, topk_idx, dst, weights=None, bias_bits=None):
    """Vectorised over tokens and channels, sequential over k, in numpy
    float32 (each operation rounded separately), rounded to bf16 by torch."""
    idx = np.asarray(topk_idx, np.int64)
    d = np.asarray(dst, np.int64).reshape(idx.shape)
    T, K = idx.shape
    yf = bf16_bits_to_f32(y_bits)
    H = yf.shape[1]
    bf = None if bias_bits is None else bf16_bits_to_f32(bias_bits)
    acc = np.zeros((T, H), np.float32)
    for k in range(K):
        rows = d[:, k]
        ok = rows >= 0
        v = yf[np.where(ok, rows, 0)]
        if bf is not None:
            v = (v + bf[np.where(ok, idx[:, k], 0)]).astype(np.float32)
        if weights is not None:
            v = (np.asarray(weights, np.float32)[:, k:k + 1] * v).astype(np.float32)
        acc = np.where(ok[:, None], (acc + v).astype(np.float32), acc)
    return f32_to_bf16_bits_torch(acc)


def combine_exact_sum(y_bits, topk_idx, dst, weights=None, bias_bits=None):
    """The weighted sum evaluated in binary64 (no bf16 rounding), and the sum
    of |terms|.  Its own rounding error is many orders of magnitude below the
    binary32 error bound that the oracle is checked against."""
    idx = np.asarray(topk_idx, np.int64)
    d = np.asarray(dst, np.int64).reshape(idx.shape)
    T, K = idx.shape
    yf = bf16_bits_to_f32(y_bits).astype(np.float64)
    bf = None if bias_bits is None else bf16_bits_to_f32(bias_bits).astype(np.float64)
    acc = np.zeros((T, yf.shape[1]))
    mag = np.zeros_like(acc)
    for k in range(K):
        rows = d[:, k]
        ok = rows >= 0
        v = yf[np.where(ok, rows, 0)]
        if bf is not None:
            v = v + bf[np.where(ok, idx[:, k], 0)]
        if weights is not None:
            v = np.asarray(weights, np.float64)[:, k:k + 1] * v
        acc += np.where(ok[:, None], v, 0.0)
        mag += np.where(ok[:, None], np.abs(v), 0.0)
    return acc, mag


def combine_backward_expected(g_bits, topk_idx, dst, weights, y_bits, bias_bits, counts,
                              psum, src_meta, E):
    """Backward of combine written out directly: grad_y rows as bf16 of the
    float32 product w * g, grad_w as a float64 dot product over channels,
    grad_bias as a float64 sum over each expert's rows."""
    idx = np.asarray(topk_idx, np.int64)
    T, K = idx.shape
    g = bf16_bits_to_f32(g_bits)
    H = g.shape[1]
    d = np.asarray(dst, np.int64).reshape(T, K)
    w = None if weights is None else np.asarray(weights, np.float32)
    rows = {}
    gw = np.zeros((T, K), np.float64)
    yf = bf16_bits_to_f32(y_bits).astype(np.float64)
    bf = None if bias_bits is None else bf16_bits_to_f32(bias_bits).astype(np.float64)
    for t in range(T):
        for k in range(K):
            r = d[t, k]
            if r < 0:
                continue
            s = g[t] if w is None else (w[t, k] * g[t]).astype(np.float32)
            rows[int(r)] = f32_to_bf16_bits_torch(s[None, :])[0]
            v = yf[r] + (bf[idx[t, k]] if bf is not None else 0.0)
            gw[t, k] = float(np.dot(g[t].astype(np.float64), v))
    gb = np.zeros((E, H), np.float64)
    for e in range(E):
        acc = np.zeros(H, np.float64)
        for r in range(int(psum[e]), int(psum[e]) + int(counts[e])):
            i = int(src_meta[r])
            t, k = divmod(i, K)
            gd = g[t].astype(np.float64)
            acc = acc + (gd if w is None else float(w[t, k]) * gd)
        gb[e] = acc
    return rows, gw, gb
