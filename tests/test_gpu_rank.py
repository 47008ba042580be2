"""Rank (non-expanded) layout and per-token biases on the GPU against the CPU
oracle, bit-exact: rank dispatch (rows, FP8 scales, received top-k ids and
weights; unwritten rows poison-checked), rank combine with bias_0 / bias_1,
the expanded combine with per-token biases, and the hand-worked order cases."""
import json
import os

import numpy as np
import pytest
import torch

import combine_ep_layout_08_amd as ep
import ep_workloads as W
import oracle
from tests.gpu_util import (POISON, assert_rank_equal, gpu_layout, needs_gpu, poison_, say,
                            u16, u8)

pytestmark = [pytest.mark.gpu, needs_gpu]
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(shape, seed, scale=1.0):
    return torch.randn(shape, generator=torch.Generator().manual_seed(seed)).mul(scale).to(
        torch.bfloat16)


@pytest.mark.parametrize("fp8,H,idx32", [(False, 264, False), (True, 1024, False),
                                         (False, 7168, True), (True, 7168, True)])
def test_dispatch_rank(fp8, H, idx32):
    rng = np.random.default_rng(H + fp8)
    T, K, E = 700, 6, 20
    idx = np.where(rng.random((T, K)) < 0.55, -1, rng.integers(-2, E + 2, size=(T, K)))
    w = rng.random((T, K), dtype=np.float32)
    h, rc, _, _ = gpu_layout(idx, E, 4, T * K + 4 * E,
                             idx_dtype=torch.int32 if idx32 else torch.int64)
    assert_rank_equal(rc, idx, E)
    if fp8:
        x = torch.from_numpy(rng.integers(0, 256, size=(T, H), dtype=np.uint8))
        sf = torch.from_numpy(rng.random((T, H // 128), dtype=np.float32))
    else:
        x, sf = _bf16((T, H), 1), None
    out_x = poison_(torch.empty((T, H), dtype=x.dtype, device="cuda"))
    out_sf = poison_(torch.empty((T, H // 128), dtype=torch.float32, device="cuda")) if fp8 \
        else None
    out_i = poison_(torch.empty((T, K), dtype=torch.int32 if idx32 else torch.int64,
                                device="cuda"))
    out_w = poison_(torch.empty((T, K), dtype=torch.float32, device="cuda"))
    say("dispatch rank", fp8, H, idx32)
    h.dispatch_rank(x.cuda(), sf=None if sf is None else sf.cuda(),
                    topk_weights=torch.from_numpy(w).cuda(), out_x=out_x, out_sf=out_sf,
                    out_topk_idx=out_i, out_topk_weights=out_w)
    torch.cuda.synchronize()
    row, src, n = oracle.rank_layout(idx, E)
    pf = np.frombuffer(bytes([POISON] * 4), np.float32)[0]
    ox = np.full((T, u8(x[:1]).shape[1]), POISON, np.uint8)
    osf = np.full((T, H // 128), pf, np.float32) if fp8 else None
    oi = np.full((T, K), np.frombuffer(bytes([POISON] * 8), np.int64)[0], np.int64)
    ow = np.full((T, K), pf, np.float32)
    oracle.dispatch_rank(u8(x), idx, E, row, T, sf=None if sf is None else sf.numpy(),
                         weights=w, out_x=ox, out_sf=osf, out_idx=oi, out_w=ow)
    np.testing.assert_array_equal(u8(out_x), ox)
    if fp8:
        np.testing.assert_array_equal(out_sf.cpu().numpy().view(np.uint32), osf.view(np.uint32))
    gi = out_i.cpu().numpy().astype(np.int64)
    np.testing.assert_array_equal(gi[:n], oi[:n])
    np.testing.assert_array_equal(out_w.cpu().numpy()[:n], ow[:n])
    assert np.all(u8(out_w)[n:] == POISON)


@pytest.mark.parametrize("name,fmt", [("f32", oracle.SF_F32), ("ue8m0", oracle.SF_UE8M0)])
@pytest.mark.parametrize("H,idx32,col,weights", [(1152, False, False, True),
                                                 (7168, True, True, True),
                                                 (2176, False, True, False)])
def test_dispatch_rank_quant(name, fmt, H, idx32, col, weights):
    """Quantising rank dispatch: the oracle's quantiser followed by its rank
    dispatch of the codes and packs, bit-exact, with empty tokens, invalid
    ids, row- or column-major scales (2176 channels: a partial UE8M0 pack),
    and unwritten rows poison-checked."""
    rng = np.random.default_rng(H * 3 + fmt + idx32)
    T, K, E = 700, 6, 20
    idx = np.where(rng.random((T, K)) < 0.55, -1, rng.integers(-2, E + 2, size=(T, K)))
    w = rng.random((T, K), dtype=np.float32) if weights else None
    h, rc, _, _ = gpu_layout(idx, E, 4, T * K + 4 * E,
                             idx_dtype=torch.int32 if idx32 else torch.int64)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x *= (10.0 ** rng.integers(-6, 5, size=(T, H // 128, 1))).repeat(128, axis=2).reshape(T, H)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    P = ep.ep_sf_packs(H, fmt)
    out_x = poison_(torch.empty((T, H), dtype=torch.uint8, device="cuda"))
    if col:
        store = poison_(torch.empty((P, ep.ep_tma_aligned_rows(T)), dtype=torch.int32,
                                    device="cuda"))
        out_sf = store[:, :T].t()
    else:
        out_sf = poison_(torch.empty((T, P), dtype=torch.int32, device="cuda"))
    if name == "f32":
        out_sf = out_sf.view(torch.float32)
    out_i = poison_(torch.empty((T, K), dtype=torch.int32 if idx32 else torch.int64,
                                device="cuda"))
    out_w = poison_(torch.empty((T, K), dtype=torch.float32, device="cuda"))
    say("dispatch rank quant", name, H, idx32, col, weights)
    h.dispatch_rank_quant(xb.cuda(), name,
                          topk_weights=None if w is None else torch.from_numpy(w).cuda(),
                          out_x=out_x, out_sf=out_sf, out_topk_idx=out_i, out_topk_weights=out_w)
    torch.cuda.synchronize()
    q, sf = oracle.quantize_fp8(u16(xb), fmt)
    row, _, n = oracle.rank_layout(idx, E)
    pf = np.frombuffer(bytes([POISON] * 4), np.float32)[0]
    ox = np.full((T, H), POISON, np.uint8)
    osf = np.full((T, P), np.uint32(0xA5A5A5A5), np.uint32)
    oi = np.full((T, K), np.frombuffer(bytes([POISON] * 8), np.int64)[0], np.int64)
    ow = np.full((T, K), pf, np.float32)
    oracle.dispatch_rank(q, idx, E, row, T, sf=sf, weights=w, out_x=ox, out_sf=osf, out_idx=oi,
                         out_w=ow, num_sf_packs=P)
    np.testing.assert_array_equal(u8(out_x), ox)
    np.testing.assert_array_equal(out_sf.contiguous().view(torch.int32).cpu().numpy()
                                  .view(np.uint32), osf)
    np.testing.assert_array_equal(out_i.cpu().numpy().astype(np.int64)[:n], oi[:n])
    np.testing.assert_array_equal(out_w.cpu().numpy()[:n], ow[:n])
    assert np.all(u8(out_w)[n:] == POISON)


@pytest.mark.parametrize("idx32", [False, True])
@pytest.mark.parametrize("give_ids,give_weights", [(True, True), (True, False), (False, True),
                                                   (False, False)])
def test_dispatch_rank_quant_limits(idx32, give_ids, give_weights):
    """Quantising rank dispatch at the limits (E = 1024, K = 64: every lane of
    the quantising wave writes an id and a weight) through the C ABI, with
    either metadata output NULL: the given ones match the oracle bit for bit,
    the codes and scales do too, and nothing else is written."""
    rng = np.random.default_rng(641 + 2 * idx32 + give_ids + 4 * give_weights)
    T, K, E, H = 300, 64, 1024, 512
    idx = np.where(rng.random((T, K)) < 0.5, -1, rng.integers(-3, E + 3, size=(T, K)))
    idx[:7] = -1                                       # tokens with no slot
    w = rng.random((T, K), dtype=np.float32)
    h, _, _, _ = gpu_layout(idx, E, 1, T * K, idx_dtype=torch.int32 if idx32 else torch.int64)
    xb = _bf16((T, H), 642)
    fmt = oracle.SF_F32
    P = ep.ep_sf_packs(H, fmt)
    out_x = poison_(torch.empty((T, H), dtype=torch.uint8, device="cuda"))
    out_sf = poison_(torch.empty((T, P), dtype=torch.int32, device="cuda"))
    out_i = poison_(torch.empty((T, K), dtype=torch.int32 if idx32 else torch.int64,
                                device="cuda"))
    out_w = poison_(torch.empty((T, K), dtype=torch.float32, device="cuda"))
    x = xb.cuda()
    wt = torch.from_numpy(w).cuda()
    say("dispatch rank quant limits", idx32, give_ids, give_weights)
    st = ep.ep_dispatch_rank_quant(h.h, x.data_ptr(), H, ep.EP_SF_F32, wt.data_ptr(),
                                   out_x.data_ptr(), out_sf.data_ptr(), P, 1,
                                   out_i.data_ptr() if give_ids else None,
                                   out_w.data_ptr() if give_weights else None,
                                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == ep.EP_OK
    q, sf = oracle.quantize_fp8(u16(xb), fmt)
    row, _, n = oracle.rank_layout(idx, E)
    ox = np.full((T, H), POISON, np.uint8)
    osf = np.full((T, P), np.uint32(0xA5A5A5A5), np.uint32)
    oi = np.zeros((T, K), np.int64)
    ow = np.zeros((T, K), np.float32)
    oracle.dispatch_rank(q, idx, E, row, T, sf=sf, weights=w, out_x=ox, out_sf=osf, out_idx=oi,
                         out_w=ow, num_sf_packs=P)
    np.testing.assert_array_equal(u8(out_x), ox)
    np.testing.assert_array_equal(out_sf.cpu().numpy().view(np.uint32), osf)
    if give_ids:
        np.testing.assert_array_equal(out_i.cpu().numpy().astype(np.int64)[:n], oi[:n])
        assert np.all(u8(out_i)[n:] == POISON)
    else:
        assert np.all(u8(out_i) == POISON)
    if give_weights:
        np.testing.assert_array_equal(out_w.cpu().numpy()[:n], ow[:n])
        assert np.all(u8(out_w)[n:] == POISON)
    else:
        assert np.all(u8(out_w) == POISON)


def test_dispatch_rank_packed_scales_column_major():
    """Rank dispatch with int32 scale packs into a column-major, 16-byte
    aligned scale buffer, bit-exact with the oracle."""
    rng = np.random.default_rng(77)
    T, K, E, H = 333, 4, 16, 2048
    packs = H // 512
    idx = np.where(rng.random((T, K)) < 0.6, -1, rng.integers(0, E, size=(T, K)))
    h, rc, _, _ = gpu_layout(idx, E, 4, T * K + 4 * E)
    x = torch.from_numpy(rng.integers(0, 256, size=(T, H), dtype=np.uint8))
    sf = rng.integers(0, 2 ** 32, size=(T, packs), dtype=np.uint64).astype(np.uint32)
    tma = ep.ep_tma_aligned_rows(T)
    store = poison_(torch.empty((packs, tma), dtype=torch.int32, device="cuda"))
    out_x = poison_(torch.empty((T, H), dtype=torch.uint8, device="cuda"))
    say("dispatch rank packed scales")
    h.dispatch_rank(x.cuda(), sf=torch.from_numpy(sf.view(np.int32)).cuda(), out_x=out_x,
                    out_sf=store[:, :T].t())
    torch.cuda.synchronize()
    row, _, n = oracle.rank_layout(idx, E)
    ox = np.full((T, H), POISON, np.uint8)
    o_store = np.full((packs, tma), np.uint32(0xA5A5A5A5), np.uint32)
    oracle.dispatch_rank(u8(x), idx, E, row, T, sf=sf, out_x=ox, num_sf_packs=packs)
    np.testing.assert_array_equal(u8(out_x), ox)
    # the oracle's rank dispatch writes row-major scales: compare through the view
    o_rows = oracle.dispatch_rank(u8(x), idx, E, row, T, sf=sf, num_sf_packs=packs)[1]
    got = store.cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(got[:, :n].T, o_rows[:n])
    assert np.all(got[:, n:] == 0xA5A5A5A5)


@pytest.mark.parametrize("biases", [(False, False), (True, False), (True, True), (False, True)])
def test_combine_rank(biases):
    rng = np.random.default_rng(7)
    T, K, E, H = 900, 4, 16, 2056
    idx = np.where(rng.random((T, K)) < 0.6, -1, rng.integers(0, E, size=(T, K)))
    h, rc, _, _ = gpu_layout(idx, E, 1, T * K)
    x = _bf16((T, H), 2, 3.0)
    b0 = _bf16((T, H), 3) if biases[0] else None
    b1 = _bf16((T, H), 4, 0.1) if biases[1] else None
    say("combine rank", biases)
    out = h.combine_rank(x.cuda(), bias_0=None if b0 is None else b0.cuda(),
                         bias_1=None if b1 is None else b1.cuda())
    torch.cuda.synchronize()
    row, _, _ = oracle.rank_layout(idx, E)
    exp = oracle.combine_rank(u16(x), row, None if b0 is None else u16(b0),
                              None if b1 is None else u16(b1))
    np.testing.assert_array_equal(u16(out), exp)


@pytest.mark.parametrize("name", ["prefill", "skewed"])
def test_combine_token_biases(name):
    cfg = W.CONFIGS[name]
    cap = ep.ep_capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment)
    wl = W.make(cfg, y_rows=cap, with_x=False)
    b0 = W.payload_bf16(cfg.tokens, cfg.hidden, 11, 3, std=0.5)
    b1 = W.payload_bf16(cfg.tokens, cfg.hidden, 12, 3, std=0.1)
    say("combine token biases", name)
    h, rc, dst, _ = gpu_layout(wl.topk_idx, cfg.experts, cfg.alignment, cap)
    out = h.combine(wl.y.cuda(), topk_weights=torch.from_numpy(wl.topk_weights).cuda(),
                    bias=None if wl.bias is None else wl.bias.cuda(), bias_0=b0.cuda(),
                    bias_1=b1.cuda())
    torch.cuda.synchronize()
    lay = oracle.layout(wl.topk_idx, cfg.experts, cfg.alignment, cap)
    exp = oracle.combine_token_bias(u16(wl.y), wl.topk_idx, lay.dst, wl.topk_weights,
                                    None if wl.bias is None else u16(wl.bias), u16(b0), u16(b1))
    np.testing.assert_array_equal(u16(out), exp)


def _pad8(vals) -> torch.Tensor:
    v = torch.tensor(vals, dtype=torch.float32)
    out = torch.zeros((v.shape[0], 8), dtype=torch.float32)
    out[:, :v.shape[1]] = v
    return out.to(torch.bfloat16)


def test_golden_bias_order():
    g = json.load(open(os.path.join(GOLDEN, "combine_hand.json")))
    tb = g["token_bias"]
    h, _, dst, _ = gpu_layout(np.array(tb["topk_idx"]), 1, 1, 3)
    assert dst.tolist() == tb["dst"]
    say("golden token bias")
    out = h.combine(_pad8(tb["y"]).cuda(), bias_0=_pad8(tb["bias_0"]).cuda(),
                    bias_1=_pad8(tb["bias_1"]).cuda())
    torch.cuda.synchronize()
    assert u16(out)[:, :1].tolist() == tb["expected_bits"]
    rk = g["rank_combine"]
    idx = np.array([[0], [-1]])                    # token 0 received (row 0), token 1 not
    h, rc, _, _ = gpu_layout(idx, 1, 1, 1)
    assert rc["recv_row"].tolist() == rk["recv_row"]
    x = torch.zeros((2, 8), dtype=torch.bfloat16)
    x[:1] = _pad8(rk["x"])
    out = h.combine_rank(x.cuda(), bias_0=_pad8(rk["bias_0"]).cuda(),
                         bias_1=_pad8(rk["bias_1"]).cuda())
    torch.cuda.synchronize()
    assert u16(out)[:, :1].tolist() == rk["expected_bits"]


def test_imported_layout_has_rank_rows():
    rng = np.random.default_rng(3)
    T, K, E = 500, 4, 12
    idx = np.where(rng.random((T, K)) < 0.7, -1, rng.integers(0, E, size=(T, K)))
    lay = oracle.layout(idx, E, 2, T * K + 2 * E)
    h = ep.Handle(T, K, E, 2, T * K + 2 * E)
    say("import rank rows")
    h.import_layout(torch.from_numpy(idx).cuda(), lay.counts, lay.psum, lay.dst,
                    lay.src_meta[:lay.num_expanded], lay.num_recv_tokens)
    row, src, n = oracle.rank_layout(idx, E)
    np.testing.assert_array_equal(h.recv_row.cpu().numpy(), row)
    np.testing.assert_array_equal(h.recv_src.cpu().numpy()[:n], src)


@pytest.mark.parametrize("name", ["prefill", "skewed"])
def test_rank_dispatch_after_import_equals_after_layout(name):
    """The imported layout's rank rows come from the device's numbering of
    its slot rows: a rank dispatch after ep_handle_import of the oracle's
    layout writes the same bytes (rows, scales, received ids and weights) as
    one after ep_layout on the same ids."""
    cfg = W.CONFIGS[name]
    wl = W.make(cfg, device="cuda")
    idx = torch.from_numpy(wl.topk_idx).cuda()
    w = torch.from_numpy(wl.topk_weights).cuda()
    cap = ep.ep_capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment)
    lay = oracle.layout(wl.topk_idx, cfg.experts, cfg.alignment, cap)
    outs = []
    for how in ("layout", "import"):
        h = ep.Handle(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment, cap)
        say("rank dispatch after", how, name)
        if how == "layout":
            h.layout(idx)
        else:
            h.import_layout(idx, lay.counts, lay.psum, lay.dst, lay.src_meta[:lay.num_expanded],
                            lay.num_recv_tokens)
        rx = poison_(torch.empty((cfg.tokens, cfg.hidden), dtype=wl.x.dtype, device="cuda"))
        rsf = (poison_(torch.empty((cfg.tokens, cfg.hidden // 128), dtype=torch.float32,
                                   device="cuda")) if cfg.fp8 else None)
        ri = poison_(torch.empty((cfg.tokens, cfg.topk), dtype=torch.int64, device="cuda"))
        rw = poison_(torch.empty((cfg.tokens, cfg.topk), dtype=torch.float32, device="cuda"))
        h.dispatch_rank(wl.x, sf=wl.sf, topk_weights=w, out_x=rx, out_sf=rsf, out_topk_idx=ri,
                        out_topk_weights=rw)
        torch.cuda.synchronize()
        assert h.read_counts(check=False)["num_recv_tokens"] == lay.num_recv_tokens
        outs.append([u8(t) for t in (rx, rsf, ri, rw) if t is not None] +
                    [h.recv_row.cpu().numpy().copy()])
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)


def test_import_with_wrong_received_count_is_refused():
    rng = np.random.default_rng(11)
    T, K, E = 300, 4, 9
    idx = np.where(rng.random((T, K)) < 0.5, -1, rng.integers(0, E, size=(T, K)))
    lay = oracle.layout(idx, E, 2, T * K + 2 * E)
    h = ep.Handle(T, K, E, 2, T * K + 2 * E)
    say("import wrong received count")
    with pytest.raises(ep.EpError) as err:
        h.import_layout(torch.from_numpy(idx).cuda(), lay.counts, lay.psum, lay.dst,
                        lay.src_meta[:lay.num_expanded], lay.num_recv_tokens + 1)
    assert err.value.status == ep.EP_ERR_SHAPE
    assert h.h.laid_out == 0
    with pytest.raises(ep.EpError) as err:
        h.read_counts()
    assert err.value.status == ep.EP_ERR_NOT_LAID_OUT
    # the right count is taken
    h.import_layout(torch.from_numpy(idx).cuda(), lay.counts, lay.psum, lay.dst,
                    lay.src_meta[:lay.num_expanded], lay.num_recv_tokens)
    assert h.read_counts(check=False)["num_recv_tokens"] == lay.num_recv_tokens
