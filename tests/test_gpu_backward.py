"""Backward pair on the GPU against the CPU oracle.

grad_y (combine backward) and grad_x (dispatch backward) are bf16 results of
separately rounded binary32 operations: bit-exact.  The weight and bias
gradients are binary64 sums of exact terms rounded once to binary32; their
summation order differs from the oracle's, so they are compared with
|gpu - ref| <= 2^-24 |ref| + n 2^-52 sum|terms| (one binary32 rounding plus
the binary64 reordering bound over n terms)."""
import numpy as np
import pytest
import torch

import combine_ep_layout_08_amd as ep
import ep_workloads as W
import oracle
from tests import bruteforce as BF
from tests.gpu_util import (POISON, assert_layout_equal, assert_rows_equal, gpu_layout, needs_gpu,
                            poison_, say, u16)
from tests.tolerance import check_sum

pytestmark = [pytest.mark.gpu, needs_gpu]


def _magnitudes(g, idx, dst, w, y, b):
    """sum_h |g (y + b)| per slot and sum over rows |w g| per (expert, channel)."""
    gf = BF.bf16_bits_to_f32(g).astype(np.float64)
    yf = BF.bf16_bits_to_f32(y).astype(np.float64)
    bf = None if b is None else BF.bf16_bits_to_f32(b).astype(np.float64)
    T, K = idx.shape
    mw = np.zeros((T, K))
    for k in range(K):
        ok = dst[:, k] >= 0
        v = yf[np.maximum(dst[:, k], 0)]
        if bf is not None:
            v = v + bf[np.maximum(idx[:, k], 0)]
        mw[:, k] = np.where(ok, np.abs(gf * v).sum(axis=1), 0.0)
    return mw


_check_sum = check_sum


def _run(idx, E, A, cap, g, y, w=None, b=None, want_bias=True, want_y=True, want_w=True):
    T, K = idx.shape
    H = g.shape[1]
    h, rc, dst, src = gpu_layout(idx, E, A, cap)
    lay = oracle.layout(idx, E, A, cap)
    assert_layout_equal(rc, dst, src, lay)      # a gradient mismatch below is then not the layout's
    gy = poison_(torch.empty((cap, H), dtype=torch.bfloat16, device="cuda")) if want_y else None
    wd = None if w is None else torch.from_numpy(w).cuda()
    bd = None if b is None else b.cuda()
    r_gy, gw, gb = h.combine_backward(g.cuda(), topk_weights=wd, y=y.cuda(), bias=bd, grad_y=gy,
                                      want_grad_y=want_y, want_grad_weights=want_w,
                                      want_grad_bias=want_bias)
    torch.cuda.synchronize()
    assert (r_gy is None) == (not want_y) and (gw is None) == (not want_w)
    o_gy = np.full((cap, H), np.uint16(POISON | POISON << 8), np.uint16)
    o_gy, o_gw, o_gb = oracle.combine_backward(u16(g), lay, idx, w, u16(y),
                                               None if b is None else u16(b), capacity=cap,
                                               want_grad_bias=want_bias, grad_y=o_gy)
    if want_y:
        np.testing.assert_array_equal(u16(gy), o_gy)
    if want_w:
        mw = _magnitudes(u16(g), idx, lay.dst, w, u16(y), None if b is None else u16(b))
        _check_sum(gw.cpu().numpy(), o_gw, mw, H)
        assert np.all(gw.cpu().numpy()[lay.dst < 0] == 0)
    if want_bias:
        gf = np.abs(BF.bf16_bits_to_f32(u16(g)).astype(np.float64))
        wa = np.ones(idx.shape) if w is None else np.abs(w.astype(np.float64))
        mb = np.zeros((E, H))
        for k in range(K):
            ok = lay.dst[:, k] >= 0
            np.add.at(mb, idx[ok, k], wa[ok, k:k + 1] * gf[ok])
        _check_sum(gb.cpu().numpy(), o_gb, mb, int(lay.counts.max(initial=1)))
    return h, lay


@pytest.mark.parametrize("K,H,weights,bias", [(4, 256, True, False), (8, 1024, True, True),
                                              (3, 200, False, True), (12, 72, True, True),
                                              (1, 8, False, False)])
def test_combine_backward_small(K, H, weights, bias):
    rng = np.random.default_rng(K * 100 + H)
    T, E, A = 300, 24, 8
    idx = rng.integers(-1, E, size=(T, K))
    idx[5] = -1
    cap = T * K + A * E
    g = torch.randn((T, H), generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    y = torch.randn((cap, H), generator=torch.Generator().manual_seed(2)).to(torch.bfloat16)
    w = (rng.random((T, K), dtype=np.float32) * 2 - 0.5) if weights else None
    b = torch.randn((E, H), generator=torch.Generator().manual_seed(3)).mul(0.1).to(
        torch.bfloat16) if bias else None
    say("combine backward", K, H, weights, bias)
    _run(idx, E, A, cap, g, y, w, b)


@pytest.mark.parametrize("want_y,want_w,bias", [(True, False, True), (False, True, True),
                                                (False, True, False), (True, False, False),
                                                (False, False, True)])
def test_combine_backward_partial_outputs(want_y, want_w, bias):
    """Each output on its own (the row pass has grad_y-only and weight-only forms)."""
    rng = np.random.default_rng(int(want_y) * 4 + int(want_w) * 2 + int(bias))
    T, K, E, A, H = 257, 20, 40, 4, 1160
    idx = rng.integers(-1, E, size=(T, K))
    cap = T * K + A * E
    g = torch.randn((T, H), generator=torch.Generator().manual_seed(11)).to(torch.bfloat16)
    y = torch.randn((cap, H), generator=torch.Generator().manual_seed(12)).to(torch.bfloat16)
    w = rng.random((T, K), dtype=np.float32)
    b = torch.randn((E, H), generator=torch.Generator().manual_seed(13)).mul(0.1).to(
        torch.bfloat16) if bias else None
    say("combine backward partial", want_y, want_w, bias)
    _run(idx, E, A, cap, g, y, w, b, want_bias=bias, want_y=want_y, want_w=want_w)


@pytest.mark.parametrize("name", ["prefill", "skewed"])
def test_combine_backward_workloads(name):
    cfg = W.CONFIGS[name]
    cap = ep.ep_capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment)
    wl = W.make(cfg, y_rows=cap, with_x=False)
    g = W.payload_bf16(cfg.tokens, cfg.hidden, 77, 3)
    say("combine backward", name)
    _run(wl.topk_idx, cfg.experts, cfg.alignment, cap, g, wl.y, wl.topk_weights, wl.bias,
         want_bias=wl.bias is not None)


def test_dispatch_backward():
    cfg = W.CONFIGS["prefill"]
    cap = ep.ep_capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment)
    wl = W.make(cfg, y_rows=cap, with_x=False)
    go = wl.y                                        # any bf16 [capacity, H]
    gwr = torch.randn(cap, generator=torch.Generator().manual_seed(5))
    say("dispatch backward")
    h, rc, dst, src = gpu_layout(wl.topk_idx, cfg.experts, cfg.alignment, cap)
    lay = oracle.layout(wl.topk_idx, cfg.experts, cfg.alignment, cap)
    assert_layout_equal(rc, dst, src, lay)      # a grad_x mismatch below is then not the layout's
    gx, gw = h.dispatch_backward(go.cuda(), grad_out_w=gwr.cuda(), want_grad_weights=True)
    torch.cuda.synchronize()
    o_gx, o_gw = oracle.dispatch_backward(u16(go), wl.topk_idx, lay.dst, gwr.numpy())
    assert_rows_equal(u16(gx), o_gx, "grad_x")
    np.testing.assert_array_equal(gw.cpu().numpy(), o_gw)
    gx2, gw2 = h.dispatch_backward(go.cuda(), want_grad_weights=True)   # no weight gradient in
    torch.cuda.synchronize()
    np.testing.assert_array_equal(u16(gx2), o_gx)
    assert np.all(gw2.cpu().numpy() == 0)


def test_backward_after_capacity_error_writes_nothing():
    idx = np.array([[0, 1], [1, 2], [2, 0]])
    h, rc, _, _ = gpu_layout(idx, 3, 4, 11)
    assert rc["status"] == ep.EP_ERR_CAPACITY
    g = torch.ones((3, 64), dtype=torch.bfloat16, device="cuda")
    y = torch.ones((11, 64), dtype=torch.bfloat16, device="cuda")
    gy = poison_(torch.empty((11, 64), dtype=torch.bfloat16, device="cuda"))
    say("backward after capacity error")
    h.combine_backward(g, y=y, grad_y=gy)
    gx, _ = h.dispatch_backward(y)
    torch.cuda.synchronize()
    assert np.all(u16(gy) == np.uint16(POISON | POISON << 8))
