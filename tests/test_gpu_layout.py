"""Routing layout on the GPU against the CPU oracle, bit-exact: counts, psum,
slot index, source metadata, received-token count, invalid-id count and error
bits.  Covers the five workloads at full size, tile boundaries, ragged and
empty inputs, invalid ids, duplicates, K > E, the limits (E = 1024, K = 64),
int32 ids, capacity errors, handle reuse and determinism."""
import numpy as np
import pytest
import torch

import combine_ep_layout_08_amd as ep
import ep_workloads as W
import oracle
from tests import pins
from tests.gpu_util import (POISON, assert_layout_equal, assert_rank_equal, gpu_layout,
                             needs_gpu, poison_, say, u8)

pytestmark = [pytest.mark.gpu, needs_gpu]


def _check(idx, E, A, capacity, **kw):
    lay = oracle.layout(idx, E, A, capacity)
    h, rc, dst, src = gpu_layout(idx, E, A, capacity, **kw)
    assert_layout_equal(rc, dst, src, lay)
    assert_rank_equal(rc, idx, E)
    return h, lay


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_layout_configs(name):
    cfg = W.CONFIGS[name]
    idx, _ = W.routing(cfg)
    cap = ep.ep_capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment)
    say("layout", name, idx.shape, cfg.experts, cfg.alignment, cap)
    _, lay = _check(idx, cfg.experts, cfg.alignment, cap)
    pins.check_layout_invariants(lay, idx, cfg.experts, cfg.alignment, cap)


def test_layout_random_small_cases():
    for n, (T, K, E, A, idx) in enumerate(pins._random_cases(n=200, seed=17)):
        cap = T * K + (A - 1) * E + A
        say("layout random", n, T, K, E, A)
        _check(idx, E, A, cap)


@pytest.mark.parametrize("slots", [1, 63, 64, 65, 1024, 1025, 2047, 2048, 2049, 4096, 4097,
                                   2048 * 7 + 5])
@pytest.mark.parametrize("K,E", [(8, 256), (1, 1024), (4, 1), (3, 5)])
def test_layout_tile_boundaries(slots, K, E):
    T = max(1, slots // K)
    rng = np.random.default_rng(slots * 31 + K)
    idx = rng.integers(-1, E, size=(T, K))
    say("layout tiles", T, K, E)
    _check(idx, E, 4, T * K + 4 * E)


@pytest.mark.parametrize("T,K,E", [(128, 8, 256), (129, 8, 256), (256, 8, 256), (257, 8, 256),
                                   (8192, 8, 256), (8193, 8, 256), (10880, 6, 64),
                                   (10881, 6, 64), (102400, 8, 256), (102401, 8, 256),
                                   (8229, 64, 1024)])
def test_layout_forms_meet(T, K, E):
    """A batch within one tile (up to 2048 slots) is laid out by one block in
    one launch; up to 64 short tiles (1024 slots) by count + place over short
    tiles, up to 400 tiles of 2048 slots over long ones; beyond that by the
    single-pass lookback.  Both sides of each switch, bit-exact, with empty
    and invalid ids."""
    rng = np.random.default_rng(T + K)
    idx = rng.integers(-1, E, size=(T, K))
    idx[::101, 0] = E + 3                               # invalid ids
    say("layout forms", T, K, E)
    _check(idx, E, 16, T * K + 16 * E)


def test_layout_limits_and_skew():
    rng = np.random.default_rng(5)
    T, K, E = 3000, 64, 1024
    idx = rng.integers(-1, E, size=(T, K))
    say("layout E=1024 K=64")
    _check(idx, E, 16, T * K + 16 * E)
    idx = np.zeros((5000, 8), np.int64)          # every slot on expert 0
    say("layout one hot expert")
    _check(idx, 256, 128, 5000 * 8 + 128 * 256)


def test_layout_special_inputs():
    say("layout T=0")
    _check(np.zeros((0, 8), np.int64), 16, 4, 64)
    say("layout all empty")
    _check(np.full((300, 8), -1), 16, 4, 64)
    rng = np.random.default_rng(8)
    idx = rng.integers(-5, 40, size=(700, 6))    # ids beyond E and below -1
    say("layout invalid ids")
    _, lay = _check(idx, 32, 8, 700 * 6 + 8 * 32)
    assert lay.invalid_count > 0
    say("layout K > E duplicates")
    _check(rng.integers(0, 3, size=(333, 7)), 3, 2, 333 * 7 + 6)
    say("layout int32 ids")
    _check(rng.integers(-1, 64, size=(999, 8)), 64, 32, 999 * 8 + 32 * 64,
           idx_dtype=torch.int32)


def test_layout_golden_hand_example():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "layout_hand.json")))
    idx = np.array(g["topk_idx"])
    say("layout golden")
    h, rc, dst, src = gpu_layout(idx, g["num_experts"], g["alignment"], g["capacity_bound"])
    assert rc["counts"].tolist() == g["counts"]
    assert rc["psum"].tolist() == g["psum"]
    assert dst.tolist() == g["dst"]
    assert src[:g["num_expanded"]].tolist() == g["src_meta"]
    assert rc["num_recv_tokens"] == g["num_recv_tokens"]


def test_layout_capacity_error():
    idx = np.array([[0, 1], [1, 2], [2, 0]])
    say("layout capacity error")
    _check(idx, 3, 4, 11)                        # needs 12 rows
    _check(idx, 3, 4, 12)


@pytest.mark.parametrize("T", [100, 5000, 40000, 110000])     # every layout form
def test_layout_capacity_in_every_form(T):
    """A capacity one row short of what the routing needs is reported as
    EP_ERR_CAPACITY and dispatch and combine then write nothing; the exact
    capacity succeeds bit-exactly."""
    K, E, A, H = 8, 64, 4, 64
    idx = np.random.default_rng(T + 1).integers(-1, E, size=(T, K))
    need = oracle.layout(idx, E, A, T * K + A * E).num_expanded
    for cap in (need - 1, need):
        say("layout capacity", T, cap, need)
        lay = oracle.layout(idx, E, A, cap)
        h, rc, dst, src = gpu_layout(idx, E, A, cap)
        assert_layout_equal(rc, dst, src, lay)
        out_x = poison_(torch.empty((cap, H), dtype=torch.bfloat16, device="cuda"))
        out = poison_(torch.empty((T, H), dtype=torch.bfloat16, device="cuda"))
        h.dispatch(torch.ones((T, H), dtype=torch.bfloat16, device="cuda"), out_x=out_x,
                   zero_padding=True)
        h.combine(torch.ones((cap, H), dtype=torch.bfloat16, device="cuda"), out=out)
        torch.cuda.synchronize()
        if cap < need:
            assert rc["status"] == ep.EP_ERR_CAPACITY
            assert np.all(u8(out_x) == POISON) and np.all(u8(out) == POISON)
        else:
            assert not np.any(u8(out) == POISON)


@pytest.mark.parametrize("T", [64, 4096, 110000])     # one-tile, count + place, lookback forms
def test_layout_timeout_bit_is_sticky(T):
    """Once a layout scan's bounded wait has given up, the handle stays void
    until it is set up again.  The timeout bit is set here from the host in the
    handle's error word (no wait has to time out): a later layout still
    reports EP_ERR_TIMEOUT, dispatch and combine write nothing, and a new
    ep_handle_init on the same workspace clears it."""
    K, E, A, H = 8, 64, 4, 64
    idx = torch.from_numpy(np.random.default_rng(T).integers(-1, E, size=(T, K))).cuda()
    h = ep.Handle(T, K, E, A)
    h.scalars[ep.EP_SCALAR_ERROR_BITS] = ep.EP_ERRBIT_SCAN_TIMEOUT
    say("layout sticky timeout", T)
    h.layout(idx)
    assert h.read_counts(check=False)["status"] == ep.EP_ERR_TIMEOUT
    out_x = poison_(torch.empty((h.capacity, H), dtype=torch.bfloat16, device="cuda"))
    out = poison_(torch.empty((T, H), dtype=torch.bfloat16, device="cuda"))
    h.dispatch(torch.ones((T, H), dtype=torch.bfloat16, device="cuda"), out_x=out_x,
               zero_padding=True)
    h.combine(torch.ones((h.capacity, H), dtype=torch.bfloat16, device="cuda"), out=out)
    torch.cuda.synchronize()
    assert np.all(u8(out_x) == POISON) and np.all(u8(out) == POISON)
    assert ep.ep_handle_init(h.h, T, K, E, A, h.capacity, h.workspace.data_ptr(),
                             h.workspace.numel(), ep._stream()) == ep.EP_OK
    h.layout(idx)
    assert h.read_counts(check=False)["status"] in (ep.EP_OK, ep.EP_ERR_INVALID_ID)


def test_layout_handle_reuse_and_determinism():
    cfg = W.CONFIGS["prefill"]
    cap = ep.ep_capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment)
    h = ep.Handle(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment, cap)
    first = None
    for rep in range(12):
        seed = 1003 if rep % 2 == 0 else 2000 + rep
        idx, _ = W.routing(cfg, seed)
        ntok = cfg.tokens if rep % 3 else cfg.tokens - 7 * rep   # fewer tokens than max
        idx = idx[:ntok]
        say("layout reuse", rep, seed, ntok)
        lay = oracle.layout(idx, cfg.experts, cfg.alignment, cap)
        _, rc, dst, src = gpu_layout(idx, cfg.experts, cfg.alignment, cap, handle=h)
        assert_layout_equal(rc, dst, src, lay)
        assert_rank_equal(rc, idx, cfg.experts)
        if seed == 1003 and ntok == cfg.tokens:
            if first is None:
                first = dst.copy()
            np.testing.assert_array_equal(dst, first)


def test_layout_forms_alternate_on_one_handle():
    """One handle sized for 110000 tokens lays out batches that take every form
    in turn - lookback (110000 x 8), count + place over long tiles (40000) and
    short tiles (8192, 5000), one launch (256, 100) and the empty batch - in
    an order that switches form on every call, so each form starts from the
    call tags, counters and status words another form left behind."""
    K, E, A, Tmax = 8, 64, 4, 110000
    cap = ep.ep_capacity_bound(Tmax, K, E, A)
    h = ep.Handle(Tmax, K, E, A, cap)
    rng = np.random.default_rng(77)
    for n, T in enumerate([110000, 256, 40000, 100, 8192, 0, 110000, 5000, 256, 40000, 110000]):
        idx = rng.integers(-1, E, size=(T, K))
        if T:
            idx[rng.integers(0, T, size=3), 0] = E + 1          # a few invalid ids
        say("layout forms on one handle", n, T)
        lay = oracle.layout(idx, E, A, cap)
        _, rc, dst, src = gpu_layout(idx, E, A, cap, handle=h)
        assert_layout_equal(rc, dst, src, lay)
        assert_rank_equal(rc, idx, E)


@pytest.mark.parametrize("T,K", [(500, 4), (5000, 4), (40000, 8), (110000, 8)])   # every form
def test_layout_cumulative_stats(T, K):
    rng = np.random.default_rng(12)
    E = 40
    h = ep.Handle(T, K, E, 8)
    stats = torch.zeros(E, dtype=torch.int32, device="cuda")
    total = np.zeros(E, np.int64)
    for rep in range(3):
        idx = rng.integers(-1, E, size=(T, K))
        say("layout stats", T, K, rep)
        h.layout(torch.from_numpy(idx).cuda(), cumulative_stats=stats)
        total += oracle.layout(idx, E, 8, h.capacity).counts
    torch.cuda.synchronize()
    np.testing.assert_array_equal(stats.cpu().numpy(), total)


@pytest.mark.parametrize("name,reps", [("prefill", 300), ("skewed", 60), ("large", 30)])
def test_layout_count_place_repeated(name, reps):
    """The count + place form many times over on one handle and on fresh
    handles, every slot row and source row against the oracle.  Each thread
    of the count kernel reads the in-tile offsets of its slots' buckets, which
    other threads write, so the ranking ends with a block barrier; without it
    a few slots per call were placed by up to a wave's count too far, now and
    then (42 of 32768 prefill slots, off by at most 5, in one run)."""
    cfg = W.CONFIGS[name]
    cap = ep.ep_capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment)
    idx_np, _ = W.routing(cfg, cfg.seed)
    lay = oracle.layout(idx_np, cfg.experts, cfg.alignment, cap)
    n = lay.num_expanded
    idx = torch.from_numpy(idx_np).cuda()
    exp_dst = torch.from_numpy(lay.dst.astype(np.int32)).cuda()
    exp_src = torch.from_numpy(lay.src_meta[:n].astype(np.int32)).cuda()
    say("count + place repeated", name, reps)
    keep = ep.Handle(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment, cap)
    bad = []
    for rep in range(reps):
        h = keep if rep % 2 else ep.Handle(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment, cap)
        h.layout(idx)
        d_ok = bool(torch.equal(h.dst_slot, exp_dst.view(cfg.tokens, cfg.topk)))
        s_ok = bool(torch.equal(h.src_meta[:n], exp_src))
        if not (d_ok and s_ok):
            bad.append(rep)
    rc = keep.read_counts()
    assert rc["num_expanded"] == n
    assert not bad, f"{len(bad)} of {reps} layouts differ from the oracle (calls {bad[:10]})"
