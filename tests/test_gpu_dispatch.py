"""Dispatch copy on the GPU against the CPU oracle, bit-exact over whole
output buffers (both sides start from the same poison bytes, so rows that
must stay untouched are checked too).  Covers bf16 and FP8 + scales, zero
padding, per-row weights, strided scale factors, ragged row sizes, cached
re-dispatch, an imported oracle layout, and capacity errors.  The largest
workload (4.2 GB output) is checked on sampled tokens and rows."""
import numpy as np
import pytest
import torch

import combine_ep_layout_08_amd as ep
import ep_workloads as W
import oracle
from tests.gpu_util import POISON, gpu_layout, needs_gpu, poison_, say, u8

pytestmark = [pytest.mark.gpu, needs_gpu]


def _run_both(idx, E, A, cap, x, sf=None, w=None, zero_padding=False, want_w=True,
              sf_cols=False, handle=None, streaming=False):
    """GPU layout + dispatch, and the oracle on the same inputs."""
    T, K = idx.shape
    h, rc, dst, _ = gpu_layout(idx, E, A, cap, handle=handle)
    H = x.shape[1]
    out_x = poison_(torch.empty((cap, H), dtype=x.dtype, device="cuda"))
    out_sf = None
    sf_dev = None
    if sf is not None:
        out_sf = poison_(torch.empty((cap, H // 128), dtype=torch.float32, device="cuda"))
        sf_dev = sf.cuda()
        if sf_cols:                          # same values, column-major storage
            sf_dev = sf_dev.t().contiguous().t()
    out_w = poison_(torch.empty(cap, dtype=torch.float32, device="cuda")) if want_w else None
    w_dev = None if w is None else torch.from_numpy(w).cuda()
    h.dispatch(x.cuda(), sf=sf_dev, topk_weights=w_dev, zero_padding=zero_padding,
               out_x=out_x, out_sf=out_sf, out_w=out_w, streaming=streaming)
    torch.cuda.synchronize()
    lay = oracle.layout(idx, E, A, cap)
    o_x = np.full((cap, u8(x[:1]).shape[1]), POISON, np.uint8)
    pf = np.frombuffer(bytes([POISON] * 4), np.float32)[0]
    o_sf = np.full((cap, H // 128), pf, np.float32) if sf is not None else None
    o_w = np.full(cap, pf, np.float32) if want_w else None
    sf_np = None if sf is None else sf.numpy()
    oracle.dispatch(u8(x), lay, cap, sf=sf_np, weights=w, want_w=want_w,
                    zero_padding=zero_padding, out_x=o_x, out_sf=o_sf, out_w=o_w)
    return h, (out_x, out_sf, out_w), (o_x, o_sf, o_w), lay


def _assert_same(gpu, ref):
    gx, gsf, gw = gpu
    ox, osf, ow = ref
    np.testing.assert_array_equal(u8(gx), ox)
    if osf is not None:
        np.testing.assert_array_equal(gsf.cpu().numpy().view(np.uint32), osf.view(np.uint32))
    if ow is not None:
        np.testing.assert_array_equal(gw.cpu().numpy().view(np.uint32), ow.view(np.uint32))


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skewed"])
def test_dispatch_configs_full(name):
    cfg = W.CONFIGS[name]
    wl = W.make(cfg)
    cap = ep.ep_capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment)
    say("dispatch", name, cap)
    _, g, o, _ = _run_both(wl.topk_idx, cfg.experts, cfg.alignment, cap, wl.x, sf=wl.sf,
                           w=wl.topk_weights, zero_padding=cfg.zero_padding)
    _assert_same(g, o)


@pytest.mark.parametrize("name,zp", [("decode", True), ("prefill", False), ("prefill", True),
                                     ("skewed", True)])
def test_dispatch_streaming_stores(name, zp):
    """EP_DISPATCH_STREAMING changes only how the rows are stored: the same
    bytes as the oracle over the whole poisoned buffers."""
    cfg = W.CONFIGS[name]
    wl = W.make(cfg)
    cap = ep.ep_capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment)
    say("dispatch streaming", name, zp)
    _, g, o, _ = _run_both(wl.topk_idx, cfg.experts, cfg.alignment, cap, wl.x, sf=wl.sf,
                           w=wl.topk_weights, zero_padding=zp, streaming=True)
    _assert_same(g, o)


@pytest.mark.parametrize("fp8,H", [(False, 8), (False, 200), (False, 1032), (False, 8200),
                                   (True, 128), (True, 1152), (True, 16384)])
@pytest.mark.parametrize("zp", [False, True])
def test_dispatch_ragged_rows(fp8, H, zp):
    rng = np.random.default_rng(H + 7 * zp)
    T, K, E, A = 77, 3, 9, 4
    idx = rng.integers(-1, E, size=(T, K))
    if fp8:
        x = torch.from_numpy(rng.integers(0, 256, size=(T, H), dtype=np.uint8))
        sf = torch.from_numpy(rng.random((T, H // 128), dtype=np.float32))
    else:
        x = torch.from_numpy(rng.integers(0, 1 << 16, size=(T, H), dtype=np.uint16)
                             .view(np.int16)).view(torch.bfloat16)
        sf = None
    w = rng.random((T, K), dtype=np.float32)
    cap = T * K + A * E
    say("dispatch ragged", fp8, H, zp)
    _, g, o, _ = _run_both(idx, E, A, cap, x, sf=sf, w=w if H % 2 else None,
                           zero_padding=zp)
    _assert_same(g, o)


def test_dispatch_strided_scales_and_no_weights():
    cfg = W.CONFIGS["decode"]
    wl = W.make(cfg)
    cap = ep.ep_capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment)
    say("dispatch column-major scales")
    _, g, o, _ = _run_both(wl.topk_idx, cfg.experts, cfg.alignment, cap, wl.x, sf=wl.sf,
                           w=None, zero_padding=True, sf_cols=True)
    _assert_same(g, o)


@pytest.mark.parametrize("zp", [False, True])
def test_dispatch_packed_scales_column_major(zp):
    """Four UE8M0 exponents per 4-byte pack (hidden 7168: 14 packs), read from
    a column-major source and copied as bits into a column-major scale buffer
    whose columns are 16-byte aligned (the grouped-GEMM layout)."""
    rng = np.random.default_rng(31 + zp)
    T, K, E, A, H = 300, 8, 64, 32, 7168
    packs = H // 512
    idx = rng.integers(-1, E, size=(T, K))
    cap = ep.ep_capacity_bound(T, K, E, A)
    x = torch.from_numpy(rng.integers(0, 256, size=(T, H), dtype=np.uint8))
    sf_np = rng.integers(0, 2 ** 32, size=(T, packs), dtype=np.uint64).astype(np.uint32)
    sf_np[::5, 3] = 0x7FC00001                      # NaN payload as a float
    sf_cols = np.ascontiguousarray(sf_np.T)         # stored [packs, T]
    sf_dev = torch.from_numpy(sf_cols.view(np.int32)).cuda().t()
    h, rc, dst, _ = gpu_layout(idx, E, A, cap)
    tma = ep.ep_tma_aligned_rows(cap)
    store = poison_(torch.empty((packs, tma), dtype=torch.int32, device="cuda"))
    out_x = poison_(torch.empty((cap, H), dtype=torch.uint8, device="cuda"))
    say("dispatch packed scales", zp)
    h.dispatch(x.cuda(), sf=sf_dev, zero_padding=zp, out_x=out_x, out_sf=store[:, :cap].t())
    _, osf2, _ = h.dispatch(x.cuda(), sf=sf_dev, zero_padding=zp, col_major_sf=True)
    torch.cuda.synchronize()
    lay = oracle.layout(idx, E, A, cap)
    o_x = np.full((cap, H), POISON, np.uint8)
    o_store = np.full((packs, tma), np.uint32(0xA5A5A5A5), np.uint32)
    oracle.dispatch(u8(x), lay, cap, sf=sf_cols, sf_strides=(1, T), zero_padding=zp,
                    out_x=o_x, out_sf=o_store, out_sf_strides=(1, tma), num_sf_packs=packs)
    np.testing.assert_array_equal(u8(out_x), o_x)
    np.testing.assert_array_equal(store.cpu().numpy().view(np.uint32), o_store)
    assert osf2.shape == (cap, packs) and osf2.stride() == (1, tma)
    n = lay.num_expanded
    written = np.nonzero(lay.src_meta[:n] >= 0)[0] if not zp else np.arange(n)
    np.testing.assert_array_equal(osf2.cpu().numpy().view(np.uint32)[written],
                                  o_store[:, :cap].T[written])


def test_dispatch_many_slots_per_token():
    rng = np.random.default_rng(2)
    T, K, E, A = 50, 40, 16, 8          # K > E: duplicates, 40 stores per row
    idx = rng.integers(-1, E, size=(T, K))
    x = torch.from_numpy(rng.integers(0, 1 << 16, size=(T, 264), dtype=np.uint16)
                         .view(np.int16)).view(torch.bfloat16)
    say("dispatch K=40")
    _, g, o, _ = _run_both(idx, E, A, T * K + A * E, x, w=rng.random((T, K), dtype=np.float32),
                           zero_padding=True)
    _assert_same(g, o)


def test_dispatch_cached_handle_matches_fresh():
    cfg = W.CONFIGS["prefill"]
    wl = W.make(cfg)
    cap = ep.ep_capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment)
    say("dispatch cached")
    h, g, o, lay = _run_both(wl.topk_idx, cfg.experts, cfg.alignment, cap, wl.x, sf=wl.sf,
                             w=wl.topk_weights)
    _assert_same(g, o)
    x2, sf2 = W.payload_fp8(cfg.tokens, cfg.hidden, 77, 3)
    out2 = poison_(torch.empty_like(g[0]))
    osf2 = poison_(torch.empty_like(g[1]))
    h.dispatch(x2.cuda(), sf=sf2.cuda(), out_x=out2, out_sf=osf2)     # reuse the handle
    torch.cuda.synchronize()
    o_x = np.full_like(o[0], POISON)
    o_sf = np.full_like(o[1], np.frombuffer(bytes([POISON] * 4), np.float32)[0])
    oracle.dispatch(u8(x2), lay, cap, sf=sf2.numpy(), out_x=o_x, out_sf=o_sf)
    np.testing.assert_array_equal(u8(out2), o_x)
    np.testing.assert_array_equal(osf2.cpu().numpy().view(np.uint32), o_sf.view(np.uint32))


def test_dispatch_with_imported_oracle_layout():
    cfg = W.CONFIGS["skewed"]
    wl = W.make(cfg)
    cap = ep.ep_capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment)
    lay = oracle.layout(wl.topk_idx, cfg.experts, cfg.alignment, cap)
    h = ep.Handle(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment, cap)
    idx_dev = torch.from_numpy(wl.topk_idx).cuda()
    say("dispatch imported layout")
    h.import_layout(idx_dev, lay.counts, lay.psum, lay.dst, lay.src_meta[:lay.num_expanded],
                    lay.num_recv_tokens)
    out_x = poison_(torch.empty((cap, cfg.hidden), dtype=torch.bfloat16, device="cuda"))
    h.dispatch(wl.x.cuda(), zero_padding=True, out_x=out_x)
    torch.cuda.synchronize()
    o_x = np.full((cap, 2 * cfg.hidden), POISON, np.uint8)
    oracle.dispatch(u8(wl.x), lay, cap, zero_padding=True, out_x=o_x)
    np.testing.assert_array_equal(u8(out_x), o_x)


@pytest.mark.parametrize("streaming", [False, True])
def test_dispatch_after_capacity_error_writes_nothing(streaming):
    idx = np.array([[0, 1], [1, 2], [2, 0]])
    x = torch.arange(3 * 64, dtype=torch.float32).reshape(3, 64).to(torch.bfloat16)
    h, rc, _, _ = gpu_layout(idx, 3, 4, 11)
    assert rc["status"] == ep.EP_ERR_CAPACITY
    out = poison_(torch.empty((11, 64), dtype=torch.bfloat16, device="cuda"))
    say("dispatch after capacity error", streaming)
    h.dispatch(x.cuda(), zero_padding=True, out_x=out, streaming=streaming)
    torch.cuda.synchronize()
    assert np.all(u8(out) == POISON)


def test_dispatch_large_sampled():
    """Largest workload: 32768 x 7168 bf16, 294656-row output sized at the
    bound, 20% empty slots.  Checked on 512 sampled tokens, on rows past
    psum[E] (untouched) and on gap rows (untouched without zero padding)."""
    cfg = W.CONFIGS["large"]
    cap = ep.ep_capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment)
    wl = W.make(cfg, device="cuda")
    say("dispatch large", cap)
    h, rc, dst, src = gpu_layout(wl.topk_idx, cfg.experts, cfg.alignment, cap)
    lay = oracle.layout(wl.topk_idx, cfg.experts, cfg.alignment, cap)
    np.testing.assert_array_equal(dst, lay.dst)
    out_x = poison_(torch.empty((cap, cfg.hidden), dtype=torch.bfloat16, device="cuda"))
    out_w = poison_(torch.empty(cap, dtype=torch.float32, device="cuda"))
    w = torch.from_numpy(wl.topk_weights).cuda()
    h.dispatch(wl.x, topk_weights=w, out_x=out_x, out_w=out_w)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    toks = rng.choice(cfg.tokens, 512, replace=False)
    xs = u8(wl.x[torch.from_numpy(toks).cuda()])
    for n, t in enumerate(toks):
        for k in range(cfg.topk):
            r = lay.dst[t, k]
            if r >= 0:
                np.testing.assert_array_equal(u8(out_x[r]), xs[n])
                assert out_w[r].item() == wl.topk_weights[t, k]
    n = lay.num_expanded
    tail = rng.integers(n, cap, 64)
    assert np.all(u8(out_x[torch.from_numpy(tail).cuda()]) == POISON)
    gaps = np.nonzero(lay.src_meta[:n] == -1)[0]
    if gaps.size:
        pick = torch.from_numpy(rng.choice(gaps, min(64, gaps.size), replace=False)).cuda()
        assert np.all(u8(out_x[pick]) == POISON)


@pytest.mark.parametrize("zp", [False, True])
def test_dispatch_scale_copy_both_orders(zp):
    """The scale packs move in expanded-row order when routed rows fill at
    least a quarter of the buffer (slots * 4 >= capacity), else with each
    token's rows; the same routing and inputs through a dense handle and one
    with eight times the capacity give the oracle's bytes either way."""
    rng = np.random.default_rng(91 + zp)
    T, K, E, A, H = 700, 8, 48, 16, 2048
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    idx = np.where(rng.random((T, K)) < 0.1, -1, idx)
    x = torch.from_numpy(rng.integers(0, 256, size=(T, H), dtype=np.uint8))
    sf = torch.from_numpy(rng.random((T, H // 128), dtype=np.float32))
    w = rng.random((T, K), dtype=np.float32)
    bound = ep.ep_capacity_bound(T, K, E, A)
    for cap in (bound, 8 * bound):                   # row order, then token order
        say("dispatch scale copy order", zp, cap)
        _, g, o, _ = _run_both(idx, E, A, cap, x, sf=sf, w=w, zero_padding=zp)
        _assert_same(g, o)


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_layout_dispatch_equals_layout_then_dispatch(name):
    """ep_layout_dispatch (the uncached dispatch: layout, then the copy, in one
    call) writes exactly what ep_layout followed by ep_dispatch writes: the
    whole layout, every output row, scale pack and weight (poison-filled
    buffers on both sides, compared on the device).  At decode and prefill
    the one-call form stores its rows with streaming stores."""
    cfg = W.CONFIGS[name]
    cap = ep.ep_capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment)
    wl = W.make(cfg, device="cuda")
    idx = torch.from_numpy(wl.topk_idx).cuda()
    w = torch.from_numpy(wl.topk_weights).cuda()
    outs = []
    for fused in (False, True):
        h = ep.Handle(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment, cap)
        ox = poison_(torch.empty((cap, cfg.hidden), dtype=wl.x.dtype, device="cuda"))
        osf = (poison_(torch.empty((cap, cfg.hidden // 128), dtype=torch.float32, device="cuda"))
               if cfg.fp8 else None)
        ow = poison_(torch.empty(cap, dtype=torch.float32, device="cuda"))
        say("layout_dispatch", name, "fused" if fused else "two calls")
        if fused:
            h.layout_dispatch(idx, wl.x, sf=wl.sf, topk_weights=w, zero_padding=cfg.zero_padding,
                              out_x=ox, out_sf=osf, out_w=ow,
                              streaming=name in ("decode", "prefill"))
        else:
            h.layout(idx)
            h.dispatch(wl.x, sf=wl.sf, topk_weights=w, zero_padding=cfg.zero_padding, out_x=ox,
                       out_sf=osf, out_w=ow)
        rc = h.read_counts(check=False)
        n = rc["num_expanded"]
        outs.append((rc, h.dst_slot.clone(), h.src_meta[:n].clone(), h.recv_row.clone(),
                     ox, osf, ow))
    (rc1, d1, s1, r1, x1, sf1, w1), (rc2, d2, s2, r2, x2, sf2, w2) = outs
    for k in ("num_expanded", "num_recv_tokens", "error_bits", "invalid_count"):
        assert rc1[k] == rc2[k], k
    np.testing.assert_array_equal(rc1["counts"], rc2["counts"])
    np.testing.assert_array_equal(rc1["psum"], rc2["psum"])
    for a, b in ((d1, d2), (s1, s2), (r1, r2), (x1, x2), (sf1, sf2), (w1, w2)):
        if a is not None:
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
