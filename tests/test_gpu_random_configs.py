"""Seeded random configurations end to end: layout, dispatch and combine on
the GPU against the CPU oracle, bit-exact, each configuration mixing options
that the targeted tests vary one at a time - token counts from 0 to 2500,
top-k 1 to 12 with duplicate experts (K may exceed E), 1 to 300 experts,
alignment 1 to 128, bf16 rows of any 16-byte multiple or FP8 rows with
row- or column-major scales, int32 or int64 ids, empty and out-of-range
ids, weights or none, an expert bias or none, zero padding or none.  Whole
output buffers start from the same poison bytes on both sides."""
import numpy as np
import pytest
import torch

import oracle
from tests import bruteforce as BF
from tests.gpu_util import POISON, gpu_layout, needs_gpu, poison_, say, u8, u16
from tests.tolerance import check_sum

pytestmark = [pytest.mark.gpu, needs_gpu]

N_CONFIGS = 40


def _config(seed):
    rng = np.random.default_rng(seed)
    c = dict(T=int(rng.choice([0, 1, 7, 64, 300, 1000, 2500])), K=int(rng.integers(1, 13)),
             E=int(rng.choice([1, 3, 16, 64, 256, 300])),
             A=int(rng.choice([1, 2, 16, 64, 128])), fp8=bool(rng.random() < 0.5),
             idx32=bool(rng.random() < 0.3), empty=float(rng.choice([0.0, 0.1, 0.5, 1.0])),
             invalid=bool(rng.random() < 0.2), weights=bool(rng.random() < 0.7),
             bias=bool(rng.random() < 0.4), zp=bool(rng.random() < 0.4),
             sf_cols=bool(rng.random() < 0.3))
    c["H"] = int(rng.choice([128, 256, 1152, 2048])) if c["fp8"] else 8 * int(rng.integers(1, 300))
    return rng, c


@pytest.mark.parametrize("seed", range(N_CONFIGS))
def test_random_config_end_to_end(seed):
    rng, c = _config(9000 + seed)
    T, K, E, A, H = c["T"], c["K"], c["E"], c["A"], c["H"]
    idx = rng.integers(0, E, size=(T, K))
    idx[rng.random((T, K)) < c["empty"]] = -1
    if c["invalid"] and T:
        bad = rng.random((T, K)) < 0.05
        idx[bad] = rng.choice([-2, E, E + 7], size=int(bad.sum()))
    cap = T * K + (A - 1) * E + A                  # enough with duplicates and K > E
    say("random config", seed, c)
    h, rc, dst, src = gpu_layout(idx, E, A, cap,
                                 idx_dtype=torch.int32 if c["idx32"] else torch.int64)
    lay = oracle.layout(idx, E, A, cap)
    n = lay.num_expanded
    assert rc["num_expanded"] == n and rc["num_recv_tokens"] == lay.num_recv_tokens
    np.testing.assert_array_equal(h.counts.cpu().numpy(), lay.counts)
    np.testing.assert_array_equal(h.psum.cpu().numpy(), lay.psum)
    np.testing.assert_array_equal(dst.reshape(-1)[:T * K], lay.dst.reshape(-1))
    np.testing.assert_array_equal(src[:n], lay.src_meta[:n])

    w = rng.random((T, K), dtype=np.float32) if c["weights"] else None
    w_dev = None if w is None else torch.from_numpy(w).cuda()
    pf = np.frombuffer(bytes([POISON] * 4), np.float32)[0]
    if c["fp8"]:
        x = torch.from_numpy(rng.integers(0, 256, size=(T, H), dtype=np.uint8))
        sf = rng.random((T, H // 128), dtype=np.float32)
        sf_dev = torch.from_numpy(sf).cuda()
        if c["sf_cols"]:
            sf_dev = sf_dev.t().contiguous().t()
        out_sf = poison_(torch.empty((cap, H // 128), dtype=torch.float32, device="cuda"))
        o_sf = np.full((cap, H // 128), pf, np.float32)
    else:
        x = torch.from_numpy(BF.f32_to_bf16_bits_torch(
            rng.standard_normal((T, H)).astype(np.float32)).view(np.int16)).view(torch.bfloat16)
        sf = sf_dev = out_sf = o_sf = None
    out_x = poison_(torch.empty((cap, H), dtype=x.dtype, device="cuda"))
    out_w = poison_(torch.empty(cap, dtype=torch.float32, device="cuda"))
    h.dispatch(x.cuda(), sf=sf_dev, topk_weights=w_dev, zero_padding=c["zp"], out_x=out_x,
               out_sf=out_sf, out_w=out_w)
    torch.cuda.synchronize()
    o_x = np.full((cap, u8(x[:1]).shape[1] if T else (H if c["fp8"] else 2 * H)), POISON,
                  np.uint8)
    o_w = np.full(cap, pf, np.float32)
    x_bytes = u8(x) if T else np.zeros((0, o_x.shape[1]), np.uint8)
    oracle.dispatch(x_bytes, lay, cap, sf=sf, weights=w, want_w=True, zero_padding=c["zp"],
                    out_x=o_x, out_sf=o_sf, out_w=o_w)
    np.testing.assert_array_equal(u8(out_x), o_x)
    np.testing.assert_array_equal(out_w.cpu().numpy().view(np.uint32), o_w.view(np.uint32))
    if o_sf is not None:
        np.testing.assert_array_equal(out_sf.cpu().numpy().view(np.uint32), o_sf.view(np.uint32))

    y = BF.f32_to_bf16_bits_torch(rng.standard_normal((cap, H)).astype(np.float32))
    bias = (BF.f32_to_bf16_bits_torch((rng.standard_normal((E, H)) * 0.02).astype(np.float32))
            if c["bias"] else None)
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    out = h.combine(to_dev(y), topk_weights=w_dev, bias=None if bias is None else to_dev(bias))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(u16(out), oracle.combine(y, idx, lay.dst, w, bias))


def _bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("seed", range(0, N_CONFIGS, 2))
def test_random_config_other_calls(seed):
    """The same kind of configurations through the backward pair (grad_y and
    grad_x bit-exact; weight and bias gradients within one binary32 rounding
    of the oracle's binary64 sums plus the reordering bound), the rank layout
    (dispatch_rank and combine_rank with both per-token biases, bit-exact)
    and, for bf16 rows of whole 128-channel blocks, the quantising dispatch
    (codes and packs bit-exact)."""
    rng, c = _config(9000 + seed)
    T, K, E, A, H = c["T"], c["K"], c["E"], c["A"], c["H"]
    idx = rng.integers(0, E, size=(T, K))
    idx[rng.random((T, K)) < c["empty"]] = -1
    if c["invalid"] and T:
        bad = rng.random((T, K)) < 0.05
        idx[bad] = rng.choice([-2, E, E + 7], size=int(bad.sum()))
    cap = T * K + (A - 1) * E + A
    say("random config, other calls", seed, c)
    h, rc, _, _ = gpu_layout(idx, E, A, cap, idx_dtype=torch.int32 if c["idx32"] else torch.int64)
    lay = oracle.layout(idx, E, A, cap)
    bf = lambda shape, s=1.0: BF.f32_to_bf16_bits_torch(
        (rng.standard_normal(shape) * s).astype(np.float32))
    w = rng.random((T, K), dtype=np.float32) if c["weights"] else None
    w_dev = None if w is None else torch.from_numpy(w).cuda()
    g, y = bf((T, H)), bf((cap, H))
    bias = bf((E, H), 0.02) if c["bias"] else None

    # combine backward
    gy = poison_(torch.empty((cap, H), dtype=torch.bfloat16, device="cuda"))
    _, gw, gb = h.combine_backward(_bf16_dev(g), topk_weights=w_dev, y=_bf16_dev(y),
                                   bias=None if bias is None else _bf16_dev(bias), grad_y=gy,
                                   want_grad_y=True, want_grad_weights=True, want_grad_bias=True)
    torch.cuda.synchronize()
    o_gy = np.full((cap, H), np.uint16(POISON | POISON << 8), np.uint16)
    o_gy, o_gw, o_gb = oracle.combine_backward(g, lay, idx, w, y, bias, capacity=cap,
                                               want_grad_bias=True, grad_y=o_gy)
    np.testing.assert_array_equal(u16(gy), o_gy)
    gf = BF.bf16_bits_to_f32(g).astype(np.float64)
    yf = BF.bf16_bits_to_f32(y).astype(np.float64)
    bfl = None if bias is None else BF.bf16_bits_to_f32(bias).astype(np.float64)
    wa = np.ones((T, K)) if w is None else np.abs(w.astype(np.float64))
    mw = np.zeros((T, K))
    mb = np.zeros((E, H))
    for k in range(K):
        ok = lay.dst[:, k] >= 0
        v = yf[np.maximum(lay.dst[:, k], 0)]
        if bfl is not None:
            v = v + bfl[np.clip(idx[:, k], 0, E - 1)]
        mw[:, k] = np.where(ok, np.abs(gf * v).sum(axis=1), 0.0)
        np.add.at(mb, idx[ok, k], wa[ok, k:k + 1] * np.abs(gf[ok]))
    check_sum(gw.cpu().numpy(), o_gw, mw, max(H, 1))
    check_sum(gb.cpu().numpy(), o_gb, mb, int(lay.counts.max(initial=1)))

    # dispatch backward
    gow = rng.standard_normal(cap).astype(np.float32)
    gx, gxw = h.dispatch_backward(_bf16_dev(y), grad_out_w=torch.from_numpy(gow).cuda(),
                                  want_grad_weights=True)
    torch.cuda.synchronize()
    o_gx, o_gxw = oracle.dispatch_backward(y, idx, lay.dst, gow)
    np.testing.assert_array_equal(u16(gx), o_gx)
    np.testing.assert_array_equal(gxw.cpu().numpy().view(np.uint32), o_gxw.view(np.uint32))

    # rank layout: dispatch_rank then combine_rank with both per-token biases
    row, _, nrecv = oracle.rank_layout(idx, E)
    pf = np.frombuffer(bytes([POISON] * 4), np.float32)[0]
    xr = bf((T, H))
    o_x = np.full((T, 2 * H), POISON, np.uint8)
    o_i = np.full((T, K), -9, np.int64)
    o_w = np.full((T, K), pf, np.float32)
    oracle.dispatch_rank(xr.view(np.uint8).reshape(T, 2 * H), idx, E, row, T, weights=w,
                         out_x=o_x, out_idx=o_i, out_w=o_w)
    r_x = poison_(torch.empty((T, H), dtype=torch.bfloat16, device="cuda"))
    r_i = torch.full((T, K), -9, dtype=torch.int32 if c["idx32"] else torch.int64, device="cuda")
    r_w = poison_(torch.empty((T, K), dtype=torch.float32, device="cuda"))
    h.dispatch_rank(_bf16_dev(xr), topk_weights=w_dev, out_x=r_x, out_topk_idx=r_i,
                    out_topk_weights=r_w)
    b0, b1 = bf((T, H)), bf((T, H))
    xrr = bf((T, H))
    out_r = h.combine_rank(_bf16_dev(xrr), bias_0=_bf16_dev(b0), bias_1=_bf16_dev(b1))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(u8(r_x).reshape(T, 2 * H), o_x)
    np.testing.assert_array_equal(r_i.cpu().numpy().astype(np.int64), o_i)
    np.testing.assert_array_equal(r_w.cpu().numpy().view(np.uint32), o_w.view(np.uint32))
    np.testing.assert_array_equal(u16(out_r), oracle.combine_rank(xrr, row, b0, b1))
    assert rc["num_recv_tokens"] == nrecv

    # quantising dispatch (bf16 rows of whole 128-channel blocks)
    if H % 128 == 0:
        name, fmt = (("ue8m0", oracle.SF_UE8M0) if seed % 4 == 0 else ("f32", oracle.SF_F32))
        P = oracle.sf_packs(H, fmt)
        xq = bf((T, H), 10.0)
        q_x = poison_(torch.empty((cap, H), dtype=torch.uint8, device="cuda"))
        q_sf = poison_(torch.empty((cap, P), dtype=torch.int32, device="cuda"))
        q_w = poison_(torch.empty(cap, dtype=torch.float32, device="cuda"))
        h.dispatch_quant(_bf16_dev(xq), name, topk_weights=w_dev, zero_padding=c["zp"],
                         out_x=q_x, out_sf=q_sf.view(torch.float32) if name == "f32" else q_sf,
                         out_w=q_w)
        torch.cuda.synchronize()
        oq_x = np.full((cap, H), POISON, np.uint8)
        oq_sf = np.full((cap, P), np.uint32(0xA5A5A5A5), np.uint32)
        oq_w = np.full(cap, pf, np.float32)
        oracle.dispatch_quant(xq, lay, cap, fmt, weights=w, zero_padding=c["zp"], out_x=oq_x,
                              out_sf=oq_sf, out_w=oq_w)
        np.testing.assert_array_equal(u8(q_x), oq_x)
        np.testing.assert_array_equal(q_sf.cpu().numpy().view(np.uint32), oq_sf)
        np.testing.assert_array_equal(q_w.cpu().numpy().view(np.uint32), oq_w.view(np.uint32))


def test_empty_batch_every_call():
    """A batch of no tokens through every call.  With expert_alignment 1 the
    capacity is 0, so every output tensor is empty (a NULL data pointer):
    each call must accept it and succeed.  With alignment 4 and zero padding
    the expanded buffer exists but the layout has no rows, so nothing may be
    written; the bias gradient is all zeros."""
    import combine_ep_layout_08_amd as ep
    K, E, H = 4, 8, 256
    for A in (1, 4):
        say("empty batch, every call, alignment", A)
        h = ep.Handle(0, K, E, A)
        h.layout(torch.zeros((0, K), dtype=torch.int64, device="cuda"))
        cap = h.capacity
        xb = torch.zeros((0, H), dtype=torch.bfloat16, device="cuda")
        x8 = torch.zeros((0, H), dtype=torch.uint8, device="cuda")
        sf = torch.zeros((0, H // 128), dtype=torch.float32, device="cuda")
        out_x = poison_(torch.empty((cap, H), dtype=torch.bfloat16, device="cuda"))
        out_w = poison_(torch.empty(cap, dtype=torch.float32, device="cuda"))
        h.dispatch(xb, out_x=out_x, out_w=out_w, zero_padding=True)
        o8 = poison_(torch.empty((cap, H), dtype=torch.uint8, device="cuda"))
        osf = poison_(torch.empty((cap, H // 128), dtype=torch.float32, device="cuda"))
        h.dispatch(x8, sf=sf, out_x=o8, out_sf=osf, zero_padding=True)
        oq = poison_(torch.empty((cap, H), dtype=torch.uint8, device="cuda"))
        oqs = poison_(torch.empty((cap, H // 128), dtype=torch.float32, device="cuda"))
        h.dispatch_quant(xb, "f32", out_x=oq, out_sf=oqs, zero_padding=True)
        y = torch.zeros((cap, H), dtype=torch.bfloat16, device="cuda")
        out = h.combine(y)
        gy, gw, gb = h.combine_backward(xb, y=y, want_grad_weights=True, want_grad_bias=True)
        gx, gxw = h.dispatch_backward(y, want_grad_weights=True)
        r = h.dispatch_rank(xb)
        rq = h.dispatch_rank_quant(xb, "ue8m0")
        out_r = h.combine_rank(xb)
        q, qs = ep.quantize_fp8(xb)
        torch.cuda.synchronize()
        assert out.shape == (0, H) and gx.shape == (0, H) and out_r.shape == (0, H)
        assert gw.shape == (0, K) and gxw.shape == (0, K) and r[0].shape == (0, H)
        assert rq[0].shape == (0, H) and rq[1].shape == (0, ep.ep_sf_packs(H, ep.EP_SF_UE8M0))
        assert q.shape == (0, H) and qs.shape == (0, H // 128)
        assert np.all(gb.cpu().numpy() == 0)
        for t in (out_x, out_w, o8, osf, oq, oqs):
            assert np.all(u8(t) == POISON)
        rc = h.read_counts()
        assert rc["num_expanded"] == 0 and rc["num_recv_tokens"] == 0
