"""Combine on the GPU against the CPU oracle, bit-exact (same binary32 slot
order, separately rounded multiply and add, bf16 round-to-nearest-even).
Covers the workloads (identity expert, softmax and sigmoid weights, fused
bias), hand-worked golden values, more than one 8-slot chunk, empty tokens,
no weights, capacity errors, and the largest workload on sampled tokens."""
import json
import os

import numpy as np
import pytest
import torch

import combine_ep_layout_08_amd as ep
import ep_workloads as W
import oracle
from tests.gpu_util import (assert_layout_equal, assert_rows_equal, gpu_layout, needs_gpu, POISON,
                            poison_, say, u16, u8)

pytestmark = [pytest.mark.gpu, needs_gpu]

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "combine_hand.json")


def _bf16(vals) -> torch.Tensor:
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16)


def _gpu_combine(h, y, w=None, bias=None):
    out = poison_(torch.empty((h.num_tokens, y.shape[1]), dtype=torch.bfloat16, device="cuda"))
    h.combine(y.cuda(), topk_weights=None if w is None else torch.from_numpy(w).cuda(),
              bias=None if bias is None else bias.cuda(), out=out)
    torch.cuda.synchronize()
    return u16(out)


def _check(idx, E, A, cap, y, w=None, bias=None):
    h, rc, dst, src = gpu_layout(idx, E, A, cap)
    lay = oracle.layout(idx, E, A, cap)
    assert_layout_equal(rc, dst, src, lay)      # a combine mismatch below is then not the layout's
    got = _gpu_combine(h, y, w, bias)
    exp = oracle.combine(u16(y), idx, lay.dst, w, None if bias is None else u16(bias))
    assert_rows_equal(got, exp, "combine")
    return got


def test_combine_tiny_identity_expert():
    cfg = W.CONFIGS["tiny"]
    wl = W.make(cfg)
    idx = wl.topk_idx.copy()
    idx[-1] = -1                                  # one token with no slot
    cap = ep.ep_capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment)
    say("combine tiny identity")
    h, rc, dst, _ = gpu_layout(idx, cfg.experts, cfg.alignment, cap)
    y, _, _ = h.dispatch(wl.x.cuda())             # identity expert: y = dispatched x
    lay = oracle.layout(idx, cfg.experts, cfg.alignment, cap)
    for w in (None, wl.topk_weights):
        got = _gpu_combine(h, y, w)
        exp = oracle.combine(u16(y), idx, lay.dst, w)
        np.testing.assert_array_equal(got, exp)
    # unit weights: out[t] = bf16(count_t * x[t]) exactly, +0.0 for the empty token
    got = _gpu_combine(h, y, None)
    c = (idx >= 0).sum(axis=1).astype(np.float32)
    prod = c[:, None] * wl.x.float().numpy()
    prod = np.where(prod == 0, np.float32(0), prod)
    exp = u16(torch.from_numpy(prod).to(torch.bfloat16))
    np.testing.assert_array_equal(got, exp)


@pytest.mark.parametrize("name", ["decode", "prefill", "skewed"])
def test_combine_configs_full(name):
    cfg = W.CONFIGS[name]
    cap = ep.ep_capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment)
    wl = W.make(cfg, y_rows=cap, with_x=False)
    say("combine", name, cap, "bias" if wl.bias is not None else "")
    _check(wl.topk_idx, cfg.experts, cfg.alignment, cap, wl.y, wl.topk_weights, wl.bias)


def _pad8(vals) -> torch.Tensor:
    """bf16 rows padded with zero columns to the 8-element (16-byte) row unit."""
    v = torch.tensor(vals, dtype=torch.float32)
    out = torch.zeros((v.shape[0], 8), dtype=torch.float32)
    out[:, :v.shape[1]] = v
    return out.to(torch.bfloat16)


def test_combine_golden_hand_values():
    g = json.load(open(GOLDEN))
    idx = np.array(g["topk_idx"])
    say("combine golden")
    h, rc, dst, _ = gpu_layout(idx, g["num_experts"], g["alignment"], 8)
    assert dst.tolist() == g["dst"]
    y = torch.zeros((8, 8), dtype=torch.bfloat16)
    y[:7] = _pad8(g["y"])
    got = _gpu_combine(h, y, np.array(g["weights"], np.float32), _pad8(g["bias"]))
    assert got[:, :2].tolist() == u16(_bf16(g["expected_with_bias"])).tolist()
    assert np.all(got[:, 2:] == 0)
    got = _gpu_combine(h, y)
    assert got[:, :2].tolist() == u16(_bf16(g["no_bias_no_weights"]["expected"])).tolist()
    t = g["ties"]
    h, _, dst, _ = gpu_layout(np.array(t["topk_idx"]), 1, 1, 4)
    assert dst.tolist() == t["dst"]
    assert _gpu_combine(h, _pad8(t["y"]))[:, :1].tolist() == t["expected_bits"]
    o = g["order"]
    h, _, dst, _ = gpu_layout(np.array(o["topk_idx"]), 1, 1, 5)
    assert dst.tolist() == o["dst"]
    got = _gpu_combine(h, _pad8(o["y"]), np.array(o["weights"], np.float32))
    assert got[:, :1].tolist() == o["expected_bits"]


@pytest.mark.parametrize("K", [1, 3, 8, 9, 12, 20, 64])
@pytest.mark.parametrize("H", [8, 24, 200, 2056])
def test_combine_ragged(K, H):
    rng = np.random.default_rng(K * 1000 + H)
    T, E, A = 45, 24, 4
    idx = rng.integers(-1, E, size=(T, K))
    idx[3] = -1
    cap = T * K + A * E
    y = torch.randn((cap, H), generator=torch.Generator().manual_seed(H)).mul(4).to(torch.bfloat16)
    w = (rng.random((T, K), dtype=np.float32) * 2 - 0.5)
    b = torch.randn((E, H), generator=torch.Generator().manual_seed(K)).to(torch.bfloat16)
    for ww, bb in ((None, None), (w, None), (None, b), (w, b)):
        say("combine ragged", K, H, ww is not None, bb is not None)
        got = _check(idx, E, A, cap, y, ww, bb)
        assert np.all(got[3] == 0)


def test_combine_after_capacity_error_writes_nothing():
    idx = np.array([[0, 1], [1, 2], [2, 0]])
    h, rc, _, _ = gpu_layout(idx, 3, 4, 11)
    assert rc["status"] == ep.EP_ERR_CAPACITY
    y = torch.ones((11, 64), dtype=torch.bfloat16, device="cuda")
    say("combine after capacity error")
    out = poison_(torch.empty((3, 64), dtype=torch.bfloat16, device="cuda"))
    h.combine(y, out=out)
    torch.cuda.synchronize()
    assert np.all(u8(out) == POISON)


def test_combine_large_sampled():
    """32768 x 7168, 294656-row expert buffer, 20% empty slots: the GPU runs
    the whole batch; 384 sampled tokens are recomputed by the oracle from
    their own expert rows."""
    cfg = W.CONFIGS["large"]
    cap = ep.ep_capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment)
    wl = W.make(cfg, device="cuda", y_rows=cap, with_x=False)
    say("combine large", cap)
    h, rc, dst, _ = gpu_layout(wl.topk_idx, cfg.experts, cfg.alignment, cap)
    w = torch.from_numpy(wl.topk_weights).cuda()
    out = h.combine(wl.y, topk_weights=w)
    torch.cuda.synchronize()
    lay = oracle.layout(wl.topk_idx, cfg.experts, cfg.alignment, cap)
    np.testing.assert_array_equal(dst, lay.dst)
    rng = np.random.default_rng(1)
    toks = np.sort(rng.choice(cfg.tokens, 384, replace=False))
    sub_dst = lay.dst[toks]
    rows = np.unique(sub_dst[sub_dst >= 0])
    remap = np.full(cap, -1, np.int64)
    remap[rows] = np.arange(rows.size)
    y_rows = u16(wl.y[torch.from_numpy(rows).cuda()])
    mini_dst = np.where(sub_dst >= 0, remap[np.maximum(sub_dst, 0)], -1)
    exp = oracle.combine(y_rows, wl.topk_idx[toks], mini_dst, wl.topk_weights[toks])
    got = u16(out[torch.from_numpy(toks).cuda()])
    np.testing.assert_array_equal(got, exp)
