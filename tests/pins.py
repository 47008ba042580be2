"""Pins of the CPU oracle against things other than itself.

Each ``pin_*`` function takes a loaded oracle library (``oracle.load()`` or a
deliberately broken build of it) and raises AssertionError on disagreement.
The pins are: hand-worked golden fixtures (``tests/golden``), brute force on
tiny inputs (``bruteforce.py``), a special case that reduces to numpy's stable
argsort, closed forms (identity expert, exact gather) and invariants.

Run as ``python -m tests.pins <oracle.so>`` to get a one-line result per pin;
the mutation test uses that to show every planted mistake is caught.
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(_HERE))

import oracle  # noqa: E402
import ep_workloads as W  # noqa: E402

try:
    from . import bruteforce as BF  # noqa: E402
except ImportError:  # run as a script
    import bruteforce as BF  # type: ignore  # noqa: E402

GOLDEN = os.path.join(_HERE, "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16_bits(vals) -> np.ndarray:
    a = np.asarray(vals, np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)   # exact for these values


def _bits_to_float(bits) -> np.ndarray:
    return BF.bf16_bits_to_f32(bits)


# ----------------------------------------------------------------------------
# layout


def pin_capacity_golden(lib):
    g = _golden("capacity_bound.json")
    for c in g["cases"]:
        got = oracle.capacity_bound(c["T"], c["K"], c["E"], c["A"], lib=lib)
        assert got == c["bound"], (c, got)


def pin_layout_golden(lib):
    g = _golden("layout_hand.json")
    cap = g["capacity_bound"]
    assert oracle.capacity_bound(3, 2, 3, 2, lib=lib) == cap
    lay = oracle.layout(np.array(g["topk_idx"]), g["num_experts"], g["alignment"],
                        cap, lib=lib)
    assert lay.status == 0
    assert lay.counts.tolist() == g["counts"]
    assert lay.psum.tolist() == g["psum"]
    assert lay.dst.tolist() == g["dst"]
    assert lay.src_meta[:g["num_expanded"]].tolist() == g["src_meta"]
    assert lay.num_recv_tokens == g["num_recv_tokens"]
    assert lay.invalid_count == g["invalid_count"]
    assert lay.num_expanded == g["num_expanded"]


def _random_cases(n=300, seed=7):
    rng = np.random.default_rng(seed)
    for c in range(n):
        T = int(rng.integers(0, 40))
        K = int(rng.integers(1, 9))
        E = int(rng.integers(1, 33))
        A = int(rng.choice([1, 2, 3, 4, 8, 64, 128]))
        mode = c % 5
        if mode == 0:      # distinct experts when possible
            idx = np.stack([rng.permutation(max(E, K))[:K] for _ in range(T)]) \
                if T else np.zeros((0, K), np.int64)
            idx = np.where(idx < E, idx, -1)
        elif mode == 1:    # duplicates allowed
            idx = rng.integers(0, E, size=(T, K))
        elif mode == 2:    # invalid ids mixed in
            idx = rng.integers(-3, E + 3, size=(T, K))
        elif mode == 3:    # mostly empty
            idx = np.where(rng.random((T, K)) < 0.8, -1, rng.integers(0, E, size=(T, K)))
        else:              # all empty
            idx = np.full((T, K), -1)
        empty = rng.random((T, K)) < rng.choice([0.0, 0.1, 0.5])
        idx = np.where(empty, -1, idx).astype(np.int64).reshape(T, K)
        yield T, K, E, A, idx


def _check_layout_vs_sorted(lay, idx, E, A):
    counts, psum, dst, src, num_recv, invalid = BF.layout_sorted(idx, E, A)
    assert lay.status == 0
    np.testing.assert_array_equal(lay.counts, counts)
    np.testing.assert_array_equal(lay.psum, psum)
    np.testing.assert_array_equal(lay.dst, dst)
    np.testing.assert_array_equal(lay.src_meta[:psum[-1]], src)
    assert lay.num_recv_tokens == num_recv
    assert lay.invalid_count == invalid
    assert lay.num_expanded == psum[-1]


def pin_layout_bruteforce(lib):
    for T, K, E, A, idx in _random_cases():
        cap = T * K + (A - 1) * E + A          # room even with duplicates
        lay = oracle.layout(idx, E, A, cap, lib=lib)
        _check_layout_vs_sorted(lay, idx, E, A)


def pin_layout_argsort_alignment1(lib):
    rng = np.random.default_rng(11)
    for _ in range(40):
        T, K, E = int(rng.integers(1, 200)), int(rng.integers(1, 9)), int(rng.integers(1, 64))
        idx = rng.integers(-1, E, size=(T, K))
        lay = oracle.layout(idx, E, 1, T * K, lib=lib)
        counts, psum, dst, order = BF.layout_argsort_a1(idx, E)
        np.testing.assert_array_equal(lay.counts, counts)
        np.testing.assert_array_equal(lay.psum, psum)
        np.testing.assert_array_equal(lay.dst, dst)
        np.testing.assert_array_equal(lay.src_meta[:order.size], order)


def check_layout_invariants(lay, idx, E, A, capacity):
    """Invariants any correct layout satisfies (also used on GPU results)."""
    idx = np.asarray(idx, np.int64)
    T, K = idx.shape
    flat = idx.reshape(-1)
    ok = (flat >= 0) & (flat < E)
    counts = lay.counts.astype(np.int64)
    psum = lay.psum.astype(np.int64)
    assert counts.sum() == ok.sum()
    np.testing.assert_array_equal(counts, np.bincount(flat[ok], minlength=E))
    assert psum[0] == 0 and np.all(psum % A == 0)
    np.testing.assert_array_equal(np.diff(psum), -(-counts // A) * A)
    assert psum[-1] <= capacity
    dst = lay.dst.reshape(-1).astype(np.int64)
    assert np.all(dst[~ok] == -1)
    d = dst[ok]
    assert np.unique(d).size == d.size                       # injective
    e = flat[ok]
    assert np.all(d >= psum[e]) and np.all(d < psum[e] + counts[e])
    src = lay.src_meta.astype(np.int64)
    np.testing.assert_array_equal(src[d], np.nonzero(ok)[0])
    gap = np.ones(psum[-1], bool)
    gap[d] = False
    assert np.all(src[:psum[-1]][gap] == -1)
    for ee in range(E):                                       # stability
        seg = src[psum[ee]:psum[ee] + counts[ee]]
        assert np.all(np.diff(seg) > 0)
    assert lay.num_recv_tokens == int(ok.reshape(T, K).any(axis=1).sum())


def pin_layout_invariants_configs(lib):
    for name, cfg in W.CONFIGS.items():
        idx, _ = W.routing(cfg)
        cap = oracle.capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment, lib=lib)
        lay = oracle.layout(idx, cfg.experts, cfg.alignment, cap, lib=lib)
        assert lay.status == 0, name
        check_layout_invariants(lay, idx, cfg.experts, cfg.alignment, cap)


def pin_layout_capacity_error(lib):
    idx = np.array([[0, 1], [1, 2], [2, 0]])
    lay = oracle.layout(idx, 3, 4, 11, lib=lib)      # needs 12 rows
    assert lay.status == oracle.ERR_CAPACITY
    assert lay.num_expanded == 12
    lay = oracle.layout(idx, 3, 4, 12, lib=lib)
    assert lay.status == 0


# ----------------------------------------------------------------------------
# dispatch


def pin_dispatch_golden(lib):
    g = _golden("layout_hand.json")
    d = g["dispatch"]
    cap = g["capacity_bound"]
    lay = oracle.layout(np.array(g["topk_idx"]), g["num_experts"], g["alignment"], cap, lib=lib)
    out_x = np.full((cap, 4), 0xA5, np.uint8)
    out_w = np.full(cap, -9.0, np.float32)
    ox, _, ow = oracle.dispatch(np.array(d["x"], np.uint8), lay, cap,
                                weights=np.array(d["weights"], np.float32),
                                want_w=True, zero_padding=True, out_x=out_x,
                                out_w=out_w, lib=lib)
    assert ox[:8].tolist() == d["out_x"]
    assert np.all(ox[8:] == 0xA5)
    assert ow[:8].tolist() == d["out_w"]
    assert np.all(ow[8:] == -9.0)


def _dispatch_case(lib, T, K, E, A, row_bytes, fp8, zero_padding, with_w,
                   rng, sf_layout="row"):
    idx = rng.integers(-1, E, size=(T, K))
    cap = T * K + (A - 1) * E + 2 * A
    lay = oracle.layout(idx, E, A, cap, lib=lib)
    x = rng.integers(0, 256, size=(T, row_bytes), dtype=np.uint8)
    w = rng.random((T, K), dtype=np.float32) if with_w else None
    sf = sf_strides = out_sf = out_sf_strides = None
    nsf = row_bytes // 128 if fp8 else 0
    if fp8:
        sf = rng.random((T, nsf), dtype=np.float32) + 0.5
        sf_strides = (nsf, 1)
        if sf_layout == "col":        # source scales stored [nsf, T]
            sf = np.ascontiguousarray(sf.T)
            sf_strides = (1, T)
        out_sf = np.full((cap, nsf), np.frombuffer(b"\xa5" * 4, np.float32)[0], np.float32)
        out_sf_strides = (nsf, 1)
    out_x = np.full((cap, row_bytes), 0xA5, np.uint8)
    out_w = np.full(cap, np.frombuffer(b"\xa5" * 4, np.float32)[0], np.float32)
    ox, osf, ow = oracle.dispatch(x, lay, cap, sf=sf, sf_strides=sf_strides,
                                  weights=w, want_w=True,
                                  zero_padding=zero_padding, out_x=out_x,
                                  out_sf=out_sf, out_sf_strides=out_sf_strides,
                                  out_w=out_w, lib=lib)
    sf_rows = None
    if fp8:
        sf_rows = sf if sf_layout == "row" else np.ascontiguousarray(sf.T)
    ex, esf, ew = BF.dispatch_expected(x, lay.dst, lay.counts, lay.psum, cap,
                                       sf=sf_rows, weights=w,
                                       zero_padding=zero_padding)
    np.testing.assert_array_equal(ox, ex)
    np.testing.assert_array_equal(ow.view(np.uint32), ew.view(np.uint32))
    if fp8:
        np.testing.assert_array_equal(osf.view(np.uint32), esf.view(np.uint32))


def pin_dispatch_closed_form(lib):
    rng = np.random.default_rng(3)
    for fp8 in (False, True):
        for zp in (False, True):
            for with_w in (False, True):
                for sf_layout in (("row", "col") if fp8 else ("row",)):
                    _dispatch_case(lib, int(rng.integers(1, 50)), int(rng.integers(1, 9)),
                                   int(rng.integers(1, 20)), int(rng.choice([1, 4, 16])),
                                   256 if fp8 else 2 * 24, fp8, zp, with_w, rng,
                                   sf_layout)


def pin_dispatch_scale_packs(lib):
    """Scale packs are 4-byte words copied as bits (one fp32 per block, or four
    UE8M0 exponent bytes; DeepEP notes ch.7 s7.3 passes the pack count and
    both strides): random words, many of them NaN patterns as floats, go to a
    column-major output whose pack stride is the row count rounded up to 4
    (16-byte aligned columns), and equal the closed form bit for bit."""
    rng = np.random.default_rng(29)
    for zp in (False, True):
        T, K, E, A, row_bytes = 37, 5, 11, 8, 640
        packs = (row_bytes // 128 + 3) // 4                  # four exponents per word
        idx = rng.integers(-1, E, size=(T, K))
        cap = T * K + (A - 1) * E + A
        lay = oracle.layout(idx, E, A, cap, lib=lib)
        x = rng.integers(0, 256, size=(T, row_bytes), dtype=np.uint8)
        sf = rng.integers(0, 2 ** 32, size=(T, packs), dtype=np.uint64).astype(np.uint32)
        sf[::3, 0] = 0x7FC00001                               # a NaN payload must survive
        tma = (cap + 3) // 4 * 4
        store = np.full((packs, tma), 0xA5A5A5A5, np.uint32)
        _, osf, _ = oracle.dispatch(x, lay, cap, sf=sf, zero_padding=zp, out_sf=store,
                                    out_sf_strides=(1, tma), num_sf_packs=packs, lib=lib)
        _, esf, _ = BF.dispatch_expected(x, lay.dst, lay.counts, lay.psum, cap, sf=sf,
                                         zero_padding=zp)
        np.testing.assert_array_equal(osf[:, :cap].T, esf)
        assert np.all(osf[:, cap:] == 0xA5A5A5A5)


# ----------------------------------------------------------------------------
# combine


def pin_combine_golden(lib):
    g = _golden("combine_hand.json")
    idx = np.array(g["topk_idx"])
    lay = oracle.layout(idx, g["num_experts"], g["alignment"], 8, lib=lib)
    assert lay.dst.tolist() == g["dst"]
    y = _bf16_bits(g["y"])
    out = oracle.combine(y, idx, lay.dst, np.array(g["weights"], np.float32),
                         _bf16_bits(g["bias"]), lib=lib)
    assert _bits_to_float(out).tolist() == g["expected_with_bias"]
    out = oracle.combine(y, idx, lay.dst, lib=lib)
    assert _bits_to_float(out).tolist() == g["no_bias_no_weights"]["expected"]
    t = g["ties"]
    out = oracle.combine(_bf16_bits(t["y"]), np.array(t["topk_idx"]),
                         np.array(t["dst"]), lib=lib)
    assert out.tolist() == t["expected_bits"]
    o = g["order"]
    out = oracle.combine(_bf16_bits(o["y"]), np.array(o["topk_idx"]),
                         np.array(o["dst"]), np.array(o["weights"], np.float32),
                         lib=lib)
    assert out.tolist() == o["expected_bits"]


def _bf16_from_normal(rng, shape, scale=1.0):
    return BF.f32_to_bf16_bits_torch(rng.standard_normal(shape, dtype=np.float32) * scale)


def _combine_inputs(rng, T, K, E, H, empty=0.2, bias=True, weights=True):
    """Random routing (layout by brute force, not by the oracle), bf16 expert
    rows, signed weights and an optional [E, H] bias.  Token 0 has no slot."""
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    idx = np.where(rng.random((T, K)) < empty, -1, idx)
    idx[0] = -1
    dst = BF.layout_sorted(idx, E, 4)[2]
    rows = T * K + 4 * E
    y = _bf16_from_normal(rng, (rows, H), 3.0)
    w = (rng.random((T, K), dtype=np.float32) * 2 - 0.5) if weights else None
    b = _bf16_from_normal(rng, (E, H), 0.5) if bias else None
    return idx, dst, y, w, b


def pin_combine_numpy_f32(lib):
    rng = np.random.default_rng(5)
    for bias in (False, True):
        for weights in (False, True):
            for (T, K, E, H) in ((37, 8, 16, 64), (20, 3, 5, 40), (9, 1, 2, 8)):
                idx, dst, y, w, b = _combine_inputs(rng, T, K, E, H, bias=bias,
                                                    weights=weights)
                got = oracle.combine(y, idx, dst, w, b, lib=lib)
                exp = BF.combine_f32(y, idx, dst, w, b)
                np.testing.assert_array_equal(got, exp)
                assert np.all(got[0] == 0)             # empty token -> +0.0


def pin_combine_f64_bound(lib):
    """The bf16 result is within the binary32 error bound of the binary64 sum:
    |got - exact| <= 2^-8 |result| (final bf16 rounding, unit roundoff 2^-8)
    + (K + 2) 2^-24 sum_k |term_k| (bias add, multiply and K - 1 adds in
    binary32, first order).  The oracle's own binary64 path must agree with
    the independent binary64 sum."""
    rng = np.random.default_rng(9)
    for bias in (False, True):
        idx, dst, y, w, b = _combine_inputs(rng, 50, 8, 16, 96, bias=bias)
        got = _bits_to_float(oracle.combine(y, idx, dst, w, b, lib=lib)).astype(np.float64)
        exact, mag = BF.combine_exact_sum(y, idx, dst, w, b)
        K = idx.shape[1]
        bound = 2.0 ** -8 * np.maximum(np.abs(got), np.abs(exact)) \
            + (K + 2) * 2.0 ** -24 * mag * 1.01
        assert np.all(np.abs(got - exact) <= bound)
        o64, omag = oracle.combine_f64(y, idx, dst, w, b, lib=lib)
        np.testing.assert_allclose(o64, exact, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(omag, mag, rtol=1e-12, atol=1e-12)


def pin_combine_identity_expert(lib):
    """y = dispatch(x) (identity expert), weights None: out[t] = bf16(c_t*x[t])
    exactly, where c_t is the number of valid slots of token t (the sum of c_t
    copies of one bf16 value needs at most 8 + log2(K) significant bits)."""
    import torch
    cfg = W.CONFIGS["tiny"]
    wl = W.make(cfg)
    idx = wl.topk_idx.copy()
    idx[-1] = -1
    cap = oracle.capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment, lib=lib)
    lay = oracle.layout(idx, cfg.experts, cfg.alignment, cap, lib=lib)
    x_bits = wl.x.contiguous().view(torch.int16).numpy().view(np.uint16)
    y_bytes, _, _ = oracle.dispatch(x_bits.view(np.uint8), lay, cap, lib=lib)
    out = oracle.combine(y_bytes.view(np.uint16), idx, lay.dst, lib=lib)
    c = (idx >= 0).sum(axis=1).astype(np.float32)
    prod = c[:, None] * _bits_to_float(x_bits)
    prod = np.where(prod == 0, np.float32(0), prod)     # the sum starts at +0.0
    exp = BF.f32_to_bf16_bits_torch(prod)
    np.testing.assert_array_equal(out, exp)
    assert np.all(out[-1] == 0)


def pin_combine_single_slot_gather(lib):
    """One valid slot per token and no weights: the output row is the expert
    row itself, except that -0.0 becomes +0.0 (the sum starts at +0.0)."""
    rng = np.random.default_rng(21)
    T, K, E, H = 30, 6, 12, 16
    idx = np.full((T, K), -1, np.int64)
    idx[np.arange(T), rng.integers(0, K, T)] = rng.integers(0, E, T)
    dst = BF.layout_sorted(idx, E, 2)[2]
    y = _bf16_from_normal(rng, (T * K + 2 * E, H))
    y[:, 3] = 0x8000                                   # -0.0 entries
    out = oracle.combine(y, idx, dst, lib=lib)
    exp = y[dst.max(axis=1)]
    exp = np.where(exp == 0x8000, 0, exp)
    np.testing.assert_array_equal(out, exp)


# ----------------------------------------------------------------------------
# backward pair


def _backward_case(rng, T=40, K=5, E=9, H=48, A=4, bias=True, weights=True):
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    idx = np.where(rng.random((T, K)) < 0.2, -1, idx)
    idx[1] = -1
    cap = T * K + A * E
    lay = oracle.layout(idx, E, A, cap, lib=None)
    g = _bf16_from_normal(rng, (T, H))
    y = _bf16_from_normal(rng, (cap, H), 2.0)
    w = (rng.random((T, K), dtype=np.float32) * 2 - 0.5) if weights else None
    b = _bf16_from_normal(rng, (E, H), 0.3) if bias else None
    return idx, lay, cap, g, y, w, b


def pin_combine_backward_bruteforce(lib):
    rng = np.random.default_rng(31)
    for bias in (False, True):
        for weights in (False, True):
            idx, lay, cap, g, y, w, b = _backward_case(rng, bias=bias, weights=weights)
            gy, gw, gb = oracle.combine_backward(g, lay, idx, w, y, b, capacity=cap,
                                                 want_grad_bias=True, lib=lib)
            rows, egw, egb = BF.combine_backward_expected(
                g, idx, lay.dst, w, y, b, lay.counts, lay.psum, lay.src_meta, len(lay.counts))
            for r, v in rows.items():
                np.testing.assert_array_equal(gy[r], v)
            np.testing.assert_allclose(gw, egw, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(gb, egb, rtol=1e-12, atol=1e-12)


def pin_combine_backward_adjoint(lib):
    """Without bias, combine is linear in y and in w:
    <g, sum_k w_k y_k> = sum_r <grad_y_r, y_r> up to grad_y's bf16 rounding,
    and sum_{t,k} w_k * grad_w[t,k] = <g, sum_k w_k y_k> (binary64)."""
    rng = np.random.default_rng(37)
    idx, lay, cap, g, y, w, _ = _backward_case(rng, bias=False)
    gy, gw, _ = oracle.combine_backward(g, lay, idx, w, y, None, capacity=cap, lib=lib)
    gf = _bits_to_float(g).astype(np.float64)
    yf = _bits_to_float(y).astype(np.float64)
    d = lay.dst
    out = np.zeros_like(gf)
    for k in range(idx.shape[1]):
        ok = d[:, k] >= 0
        out[ok] += w[ok, k:k + 1].astype(np.float64) * yf[d[ok, k]]
    lhs = float((gf * out).sum())
    valid = d[d >= 0]
    rhs = float((_bits_to_float(gy[valid]).astype(np.float64) * yf[valid]).sum())
    mag = float(np.abs(gf * out).sum()) + float(np.abs(_bits_to_float(gy[valid]) * yf[valid]).sum())
    assert abs(lhs - rhs) <= 2.0 ** -8 * mag
    assert abs(float((w.astype(np.float64) * gw).sum()) - lhs) <= 1e-9 * mag


def pin_dispatch_backward(lib):
    """grad_x is the plain combine of the gradient rows (adjoint of the copy:
    <go, dispatch(x)> = <grad_x, x> up to bf16 rounding) and grad_w gathers
    the per-row weight gradient of each slot."""
    rng = np.random.default_rng(41)
    idx, lay, cap, _, go, _, _ = _backward_case(rng)
    x = _bf16_from_normal(rng, (idx.shape[0], go.shape[1]))
    gwr = rng.standard_normal(cap).astype(np.float32)
    gx, gw = oracle.dispatch_backward(go, idx, lay.dst, gwr, lib=lib)
    np.testing.assert_array_equal(gx, BF.combine_f32(go, idx, lay.dst))
    exp_w = np.where(lay.dst >= 0, gwr[np.maximum(lay.dst, 0)], 0.0).astype(np.float32)
    np.testing.assert_array_equal(gw, exp_w)
    xd, _, _ = oracle.dispatch(x.view(np.uint8), lay, cap, lib=lib)
    valid = lay.dst[lay.dst >= 0]
    gof = _bits_to_float(go).astype(np.float64)
    lhs = float((gof[valid] * _bits_to_float(xd.view(np.uint16)[valid])).sum())
    rhs = float((_bits_to_float(gx).astype(np.float64) * _bits_to_float(x)).sum())
    mag = float(np.abs(gof[valid] * _bits_to_float(xd.view(np.uint16)[valid])).sum())
    assert abs(lhs - rhs) <= 2.0 ** -7 * mag


# ----------------------------------------------------------------------------
# rank layout and per-token biases


def pin_rank_layout_golden(lib):
    g = _golden("layout_hand.json")["rank_layout"]
    idx = np.array(g["topk_idx"])
    row, src, n = oracle.rank_layout(idx, g["num_experts"], lib=lib)
    assert row.tolist() == g["recv_row"] and src.tolist() == g["recv_src"] and n == 2
    x = np.arange(4 * 16, dtype=np.uint8).reshape(4, 16)
    ox, _, oi, ow = oracle.dispatch_rank(x, idx, g["num_experts"], row, 2,
                                         weights=np.array(g["weights"], np.float32), lib=lib)
    assert oi.tolist() == g["recv_topk_idx"]
    assert ow.tolist() == g["recv_topk_weights"]
    assert ox.tolist() == x[[1, 3]].tolist()


def pin_rank_layout_cumsum(lib):
    """Rank rows are the running count of received tokens (numpy cumsum)."""
    rng = np.random.default_rng(43)
    for _ in range(30):
        T, K, E = int(rng.integers(0, 90)), int(rng.integers(1, 6)), int(rng.integers(1, 12))
        idx = rng.integers(-3, E + 2, size=(T, K))
        idx = np.where(rng.random((T, K)) < 0.5, -1, idx)
        row, src, n = oracle.rank_layout(idx, E, lib=lib)
        ok = ((idx >= 0) & (idx < E)).any(axis=1) if T else np.zeros(0, bool)
        np.testing.assert_array_equal(row, np.where(ok, np.cumsum(ok) - 1, -1))
        np.testing.assert_array_equal(src, np.nonzero(ok)[0])
        assert n == int(ok.sum())


def pin_dispatch_rank_closed_form(lib):
    rng = np.random.default_rng(47)
    T, K, E, H = 60, 4, 10, 256
    idx = np.where(rng.random((T, K)) < 0.6, -1, rng.integers(0, E + 2, size=(T, K)))
    row, src, n = oracle.rank_layout(idx, E, lib=lib)
    x = rng.integers(0, 256, size=(T, H), dtype=np.uint8)
    sf = rng.random((T, H // 128), dtype=np.float32)
    w = rng.random((T, K), dtype=np.float32)
    rows = n + 3
    ox = np.full((rows, H), 0xA5, np.uint8)
    ox, osf, oi, ow = oracle.dispatch_rank(x, idx, E, row, rows, sf=sf, weights=w, out_x=ox,
                                           lib=lib)
    np.testing.assert_array_equal(ox[:n], x[src])
    assert np.all(ox[n:] == 0xA5)
    np.testing.assert_array_equal(osf[:n], sf[src])
    valid = (idx >= 0) & (idx < E)
    np.testing.assert_array_equal(oi[:n], np.where(valid, idx, -1)[src])
    np.testing.assert_array_equal(ow[:n], np.where(valid, w, 0.0).astype(np.float32)[src])


def _f32_bf16(rng, shape, scale=1.0):
    return _bf16_from_normal(rng, shape, scale)


def pin_combine_rank_numpy(lib):
    rng = np.random.default_rng(53)
    T, K, E, H = 50, 3, 7, 40
    idx = np.where(rng.random((T, K)) < 0.5, -1, rng.integers(0, E, size=(T, K)))
    row, src, n = oracle.rank_layout(idx, E, lib=lib)
    x = _f32_bf16(rng, (max(n, 1), H), 2.0)
    b0, b1 = _f32_bf16(rng, (T, H)), _f32_bf16(rng, (T, H), 0.5)
    for bb0, bb1 in ((None, None), (b0, None), (b0, b1), (None, b1)):
        got = oracle.combine_rank(x, row, bb0, bb1, lib=lib)
        acc = np.where((row >= 0)[:, None], _bits_to_float(x)[np.maximum(row, 0)], np.float32(0))
        for b in (bb0, bb1):
            if b is not None:
                acc = (acc + _bits_to_float(b)).astype(np.float32)
        np.testing.assert_array_equal(got, BF.f32_to_bf16_bits_torch(acc))


def pin_combine_rank_golden(lib):
    g = _golden("combine_hand.json")["rank_combine"]
    got = oracle.combine_rank(_bf16_bits(g["x"]), np.array(g["recv_row"], np.int32),
                              _bf16_bits(g["bias_0"]), _bf16_bits(g["bias_1"]), lib=lib)
    assert got.tolist() == g["expected_bits"]


def pin_combine_token_bias(lib):
    """Zero-bias special case equals the plain combine; with biases it equals
    a numpy float32 sum that adds bias_0 then bias_1 after the slots; and the
    hand-worked order cases."""
    rng = np.random.default_rng(59)
    idx, dst, y, w, b = _combine_inputs(rng, 33, 6, 11, 24)
    np.testing.assert_array_equal(oracle.combine_token_bias(y, idx, dst, w, b, lib=lib),
                                  oracle.combine(y, idx, dst, w, b, lib=lib))
    T, H = idx.shape[0], y.shape[1]
    b0, b1 = _f32_bf16(rng, (T, H)), _f32_bf16(rng, (T, H), 0.1)
    got = oracle.combine_token_bias(y, idx, dst, w, b, b0, b1, lib=lib)
    yf = _bits_to_float(y)
    bf = _bits_to_float(b)
    acc = np.zeros((T, H), np.float32)
    for k in range(idx.shape[1]):
        ok = dst[:, k] >= 0
        v = (yf[np.maximum(dst[:, k], 0)] + bf[np.maximum(idx[:, k], 0)]).astype(np.float32)
        v = (w[:, k:k + 1] * v).astype(np.float32)
        acc = np.where(ok[:, None], (acc + v).astype(np.float32), acc)
    acc = (acc + _bits_to_float(b0)).astype(np.float32)
    acc = (acc + _bits_to_float(b1)).astype(np.float32)
    np.testing.assert_array_equal(got, BF.f32_to_bf16_bits_torch(acc))
    g = _golden("combine_hand.json")["token_bias"]
    got = oracle.combine_token_bias(_bf16_bits(g["y"]), np.array(g["topk_idx"]),
                                    np.array(g["dst"]), b0_bits=_bf16_bits(g["bias_0"]),
                                    b1_bits=_bf16_bits(g["bias_1"]), lib=lib)
    assert got.tolist() == g["expected_bits"]


# ----------------------------------------------------------------------------
# FP8 quantiser (reading R23: the per-128-channel recipe of the workload inputs)


def _torch_e4m3(vals_f32: np.ndarray) -> np.ndarray:
    """torch's binary32 -> float8_e4m3fn conversion (nearest, ties to even) of
    values already inside [-448, 448]."""
    t = torch.from_numpy(np.ascontiguousarray(vals_f32, np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_e4m3_conversion_matches_torch(lib):
    """Every bf16 value in [-448, 448], every midpoint between neighbouring
    E4M3FN magnitudes and the binary32 neighbours of each midpoint convert
    like torch's float8_e4m3fn cast (a library routine)."""
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448)]
    e = np.arange(16)[:, None]
    m = np.arange(8)[None, :]
    mags = np.where(e == 0, m * 2.0 ** -9, (8 + m) * 2.0 ** (e - 10)).reshape(-1)[:127]
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)),
                           np.nextafter(mids, np.float32(1000))]).astype(np.float32)
    vals = np.concatenate([v, near, -near, mags.astype(np.float32)]).astype(np.float32)
    np.testing.assert_array_equal(oracle.f32_to_e4m3(vals, lib=lib), _torch_e4m3(vals))
    big = np.array([448.5, 464.0, 1e30, np.inf, -np.inf, -500.0], np.float32)
    np.testing.assert_array_equal(oracle.f32_to_e4m3(big, lib=lib),
                                  _torch_e4m3(np.clip(big, -448, 448)))
    assert oracle.f32_to_e4m3(np.array([np.nan], np.float32), lib=lib)[0] == 0x7F


def _quant_inputs(rng, T, H):
    """bf16 rows whose blocks span many magnitudes, with an all-zero block,
    a block below 1e-12 and blocks whose largest magnitude is negative."""
    x = rng.standard_normal((T, H)).astype(np.float32)
    x *= (10.0 ** rng.integers(-8, 6, size=(T, H // 128, 1))).repeat(128, axis=2).reshape(T, H)
    x[0, :128] = 0.0
    x[1, 128:256] *= 1e-14
    x[2, :128] = -np.abs(x[2, :128])
    return BF.f32_to_bf16_bits_torch(x)


def pin_quantize_f32_matches_torch_recipe(lib):
    """F32 scales: the same recipe written with torch ops (amax per block,
    clamp_min(1e-12) / 448, division, clamp, float8_e4m3fn cast)."""
    rng = np.random.default_rng(53)
    T, H = 24, 1280
    xb = _quant_inputs(rng, T, H)
    q, sf = oracle.quantize_fp8(xb, oracle.SF_F32, lib=lib)
    xf = torch.from_numpy(_bits_to_float(xb)).reshape(T, H // 128, 128)
    s = xf.abs().amax(dim=2).clamp_min(1e-12) / 448.0
    codes = (xf / s[:, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    np.testing.assert_array_equal(q, codes.view(torch.uint8).numpy().reshape(T, H))
    np.testing.assert_array_equal(sf, s.numpy().view(np.uint32))


def pin_quantize_ue8m0_power_of_two(lib):
    """UE8M0: the scale byte is 127 + ceil(log2(s)) (numpy frexp: s = f * 2^k,
    f in [0.5, 1)), four bytes per pack from the lowest block up, and the
    codes are torch's cast of x / 2^(byte - 127)."""
    rng = np.random.default_rng(59)
    T, H = 20, 1664                                   # 13 blocks: a partial last pack
    xb = _quant_inputs(rng, T, H)
    q, sf = oracle.quantize_fp8(xb, oracle.SF_UE8M0, lib=lib)
    xf = _bits_to_float(xb).reshape(T, H // 128, 128)
    s = np.maximum(np.abs(xf).max(axis=2), np.float32(1e-12)).astype(np.float32) / np.float32(448)
    f, k = np.frexp(s.astype(np.float64))
    ex = np.where(f == 0.5, k - 1, k) + 127
    packs = np.zeros((T, (H // 128 + 3) // 4), np.uint64)
    for j in range(H // 128):
        packs[:, j // 4] |= ex[:, j].astype(np.uint64) << np.uint64(8 * (j % 4))
    np.testing.assert_array_equal(sf, packs.astype(np.uint32))
    div = np.ldexp(np.float32(1), (ex - 127).astype(np.int32)).astype(np.float32)
    vals = np.clip(xf / div[:, :, None], -448, 448).astype(np.float32)
    np.testing.assert_array_equal(q, _torch_e4m3(vals.reshape(T, H)))


def pin_quantize_golden(lib):
    g = _golden("quant_hand.json")
    H = g["hidden"]
    x = np.zeros((1, H), np.float32)
    for c, v in g["nonzero"].items():
        x[0, int(c)] = np.nan if v == "nan" else v
    xb = _bf16_bits(x)
    q, sf = oracle.quantize_fp8(xb, oracle.SF_F32, lib=lib)
    for c, code in g["f32_codes"].items():
        assert q[0, int(c)] == code, (c, q[0, int(c)], code)
    assert np.count_nonzero(q) == len(g["f32_codes"]) - sum(1 for v in g["f32_codes"].values()
                                                             if v == 0)
    amax = np.array(g["block_amax"], np.float32)
    want = np.maximum(amax, np.float32(1e-12)) / np.float32(448)
    np.testing.assert_array_equal(sf[0], want.astype(np.float32).view(np.uint32))
    q, sf = oracle.quantize_fp8(xb, oracle.SF_UE8M0, lib=lib)
    for c, code in g["ue8m0_codes"].items():
        assert q[0, int(c)] == code, (c, q[0, int(c)], code)
    assert sf[0].tolist() == g["ue8m0_packs"]
    for j, e in enumerate(g["ue8m0_exponents"]):
        assert (int(sf[0, j // 4]) >> (8 * (j % 4))) & 0xFF == e


def pin_dispatch_quant_is_quantize_then_copy(lib):
    """The quantising dispatch equals the closed-form copy of the quantised
    rows and their packs (both formats, with and without zero padding)."""
    rng = np.random.default_rng(61)
    for fmt in (oracle.SF_F32, oracle.SF_UE8M0):
        for zp in (False, True):
            T, K, E, A, H = 30, 4, 9, 8, 640
            idx = rng.integers(-1, E, size=(T, K))
            cap = T * K + (A - 1) * E + A
            lay = oracle.layout(idx, E, A, cap, lib=lib)
            xb = _quant_inputs(rng, T, H)
            w = rng.random((T, K), dtype=np.float32)
            P = oracle.sf_packs(H, fmt, lib=lib)
            ox = np.full((cap, H), 0xA5, np.uint8)
            osf = np.full((cap, P), 0xA5A5A5A5, np.uint32)
            ow = np.full(cap, np.frombuffer(b"\xa5" * 4, np.float32)[0], np.float32)
            oracle.dispatch_quant(xb, lay, cap, fmt, weights=w, zero_padding=zp, out_x=ox,
                                  out_sf=osf, out_w=ow, lib=lib)
            q, sf = oracle.quantize_fp8(xb, fmt, lib=lib)
            ex, esf, ew = BF.dispatch_expected(q, lay.dst, lay.counts, lay.psum, cap, sf=sf,
                                               weights=w, zero_padding=zp)
            np.testing.assert_array_equal(ox, ex)
            np.testing.assert_array_equal(osf, esf)
            np.testing.assert_array_equal(ow.view(np.uint32), ew.view(np.uint32))


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


def run_all(lib):
    """Return {pin name: None or failure text}."""
    res = {}
    for p in PINS:
        try:
            p(lib)
            res[p.__name__] = None
        except Exception as e:  # noqa: BLE001 - report every failing pin
            res[p.__name__] = f"{type(e).__name__}: {str(e)[:200]}"
    return res


if __name__ == "__main__":
    lib = oracle.load(sys.argv[1]) if len(sys.argv) > 1 else oracle.load()
    out = run_all(lib)
    print(json.dumps(out))
