"""FP8 quantiser and quantising dispatch on the GPU against the CPU oracle,
bit-exact: codes, fp32 scales and packed UE8M0 exponents, over whole output
buffers (poison-filled on both sides).  Covers every bf16 value in
[-448, 448] through a unit scale, rows of several passes, column-major
scales, NaN / infinity / zero / tiny blocks, zero padding, weights, the
prefill workload at full size, and capacity errors."""
import numpy as np
import pytest
import torch

import combine_ep_layout_08_amd as ep
import ep_workloads as W
import oracle
from tests import bruteforce as BF
from tests.gpu_util import POISON, gpu_layout, needs_gpu, poison_, say, u8, u16

pytestmark = [pytest.mark.gpu, needs_gpu]

FORMATS = [("f32", oracle.SF_F32), ("ue8m0", oracle.SF_UE8M0)]


def _inputs(rng, T, H):
    """bf16 rows with blocks of many magnitudes, a zero block, a block below
    1e-12, a negative-dominated block, NaN and infinity entries."""
    x = rng.standard_normal((T, H)).astype(np.float32)
    x *= (10.0 ** rng.integers(-8, 6, size=(T, H // 128, 1))).repeat(128, axis=2).reshape(T, H)
    x[0, :128] = 0.0
    if T > 1:
        x[1, :128] *= 1e-14
    if T > 2:
        x[2, :128] = -np.abs(x[2, :128])
    if T > 3:
        x[3, 5] = np.nan
        x[3, 130] = np.inf
        x[3, 131] = -np.inf
    return BF.f32_to_bf16_bits_torch(x)


def _sf_np(t):
    return t.contiguous().view(torch.int32).cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("name,fmt", FORMATS)
def test_quantize_every_bf16_value_at_unit_scale(name, fmt):
    """Blocks led by 448 have scale 1 in both forms, so every code is the
    plain conversion of a bf16 value: all 65536 patterns in [-448, 448]."""
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448)]
    per_block = 127
    nb = -(-v.size // per_block)
    x = np.zeros((nb, 128), np.float32)
    x[:, 0] = 448.0
    flat = np.zeros(nb * per_block, np.float32)
    flat[:v.size] = v
    x[:, 1:] = flat.reshape(nb, per_block)
    H = 1024
    xb = (x.reshape(-1).view(np.uint32) >> 16).astype(np.uint16)
    xb = np.concatenate([xb, np.zeros((-xb.size) % H, np.uint16)]).reshape(-1, H)
    say("quantize every bf16", name)
    q, sf = ep.quantize_fp8(torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda(),
                            name)
    torch.cuda.synchronize()
    oq, osf = oracle.quantize_fp8(xb, fmt)
    np.testing.assert_array_equal(u8(q), oq)
    np.testing.assert_array_equal(_sf_np(sf), osf)


@pytest.mark.parametrize("name,fmt", FORMATS)
def test_quantize_every_block_maximum(name, fmt):
    """One block for every finite bf16 magnitude as its maximum (0 through
    0x7F7F, so every scale the quantiser can derive from finite input,
    including the 1e-12 floor), the other 127 entries random bf16 values of
    either sign no larger in magnitude: every divisor meets many quotients."""
    rng = np.random.default_rng(11 + fmt)
    amax = np.arange(0x7F80, dtype=np.uint32)
    rest = (rng.random((amax.size, 127)) * (amax[:, None] + 1)).astype(np.uint32)
    blocks = np.concatenate([amax[:, None], rest], axis=1)
    perm = rng.permuted(np.tile(np.arange(128), (amax.size, 1)), axis=1)
    blocks = np.take_along_axis(blocks, perm, axis=1)
    blocks |= rng.integers(0, 2, size=blocks.shape, dtype=np.uint32) << 15
    xb = blocks.astype(np.uint16).reshape(-1, 1024)
    say("quantize every block maximum", name)
    q, sf = ep.quantize_fp8(torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda(),
                            name)
    torch.cuda.synchronize()
    oq, osf = oracle.quantize_fp8(xb, fmt)
    np.testing.assert_array_equal(u8(q), oq)
    np.testing.assert_array_equal(_sf_np(sf), osf)


@pytest.mark.parametrize("name,fmt", FORMATS)
@pytest.mark.parametrize("T,H", [(1, 128), (37, 640), (300, 1664), (64, 7168), (9, 8320),
                                 (0, 256)])
def test_quantize_matches_oracle(name, fmt, T, H):
    rng = np.random.default_rng(T * 7 + H + fmt)
    xb = _inputs(rng, T, H) if T else np.zeros((0, H), np.uint16)
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
    P = ep.ep_sf_packs(H, fmt)
    q = poison_(torch.empty((T, H), dtype=torch.uint8, device="cuda"))
    sf = poison_(torch.empty((T, P), dtype=torch.int32, device="cuda"))
    if name == "f32":
        sf = sf.view(torch.float32)
    say("quantize", name, T, H)
    ep.quantize_fp8(x, name, out_q=q, out_sf=sf)
    torch.cuda.synchronize()
    oq, osf = oracle.quantize_fp8(xb, fmt)
    np.testing.assert_array_equal(u8(q), oq)
    np.testing.assert_array_equal(_sf_np(sf), osf)


@pytest.mark.parametrize("name,fmt", FORMATS)
@pytest.mark.parametrize("zp", [False, True])
def test_dispatch_quant_matches_oracle(name, fmt, zp):
    rng = np.random.default_rng(100 + fmt * 2 + zp)
    T, K, E, A, H = 400, 8, 48, 16, 2176            # 17 blocks: a partial UE8M0 pack
    idx = rng.integers(-1, E, size=(T, K))
    cap = T * K + (A - 1) * E + A
    xb = _inputs(rng, T, H)
    w = rng.random((T, K), dtype=np.float32)
    h, rc, _, _ = gpu_layout(idx, E, A, cap)
    P = ep.ep_sf_packs(H, fmt)
    tma = ep.ep_tma_aligned_rows(cap)
    out_x = poison_(torch.empty((cap, H), dtype=torch.uint8, device="cuda"))
    store = poison_(torch.empty((P, tma), dtype=torch.int32, device="cuda"))
    osf = store.view(torch.float32) if name == "f32" else store
    out_w = poison_(torch.empty(cap, dtype=torch.float32, device="cuda"))
    say("dispatch quant", name, zp)
    h.dispatch_quant(torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda(), name,
                     topk_weights=torch.from_numpy(w).cuda(), zero_padding=zp, out_x=out_x,
                     out_sf=osf[:, :cap].t(), out_w=out_w)
    torch.cuda.synchronize()
    lay = oracle.layout(idx, E, A, cap)
    o_x = np.full((cap, H), POISON, np.uint8)
    o_store = np.full((P, tma), np.uint32(0xA5A5A5A5), np.uint32)
    o_w = np.full(cap, np.frombuffer(bytes([POISON] * 4), np.float32)[0], np.float32)
    oracle.dispatch_quant(xb, lay, cap, fmt, weights=w, zero_padding=zp, out_x=o_x,
                          out_sf=o_store, out_sf_strides=(1, tma), out_w=o_w)
    np.testing.assert_array_equal(u8(out_x), o_x)
    np.testing.assert_array_equal(_sf_np(store), o_store)
    np.testing.assert_array_equal(out_w.cpu().numpy().view(np.uint32), o_w.view(np.uint32))


def test_dispatch_quant_prefill_full_size():
    """The prefill workload's routing with bf16 rows 4096 x 7168, fp32 scales,
    whole expanded buffer bit-exact; UE8M0 on sampled tokens."""
    cfg = W.CONFIGS["prefill"]
    idx, w = W.routing(cfg)
    cap = ep.ep_capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment)
    x = W.payload_bf16(cfg.tokens, cfg.hidden, cfg.seed, 3)
    h, rc, _, _ = gpu_layout(idx, cfg.experts, cfg.alignment, cap)
    out_x = poison_(torch.empty((cap, cfg.hidden), dtype=torch.uint8, device="cuda"))
    out_sf = poison_(torch.empty((cap, cfg.hidden // 128), dtype=torch.float32, device="cuda"))
    say("dispatch quant prefill f32")
    h.dispatch_quant(x.cuda(), "f32", out_x=out_x, out_sf=out_sf)
    torch.cuda.synchronize()
    lay = oracle.layout(idx, cfg.experts, cfg.alignment, cap)
    o_x = np.full((cap, cfg.hidden), POISON, np.uint8)
    o_sf = np.full((cap, cfg.hidden // 128), np.uint32(0xA5A5A5A5), np.uint32)
    oracle.dispatch_quant(u16(x), lay, cap, oracle.SF_F32, out_x=o_x, out_sf=o_sf)
    np.testing.assert_array_equal(u8(out_x), o_x)
    np.testing.assert_array_equal(_sf_np(out_sf), o_sf)
    say("dispatch quant prefill ue8m0 sampled")
    q8, s8, _ = h.dispatch_quant(x.cuda(), "ue8m0")
    torch.cuda.synchronize()
    toks = np.random.default_rng(3).choice(cfg.tokens, 256, replace=False)
    oq, osf = oracle.quantize_fp8(u16(x)[toks], oracle.SF_UE8M0)
    q8n, s8n = u8(q8), _sf_np(s8)
    for n, t in enumerate(toks):
        for r in lay.dst[t][lay.dst[t] >= 0]:
            np.testing.assert_array_equal(q8n[r], oq[n])
            np.testing.assert_array_equal(s8n[r], osf[n])


def test_dispatch_quant_after_capacity_error_writes_nothing():
    idx = np.array([[0, 1], [1, 2], [2, 0]])
    h, rc, _, _ = gpu_layout(idx, 3, 4, 11)
    assert rc["status"] == ep.EP_ERR_CAPACITY
    x = torch.ones((3, 256), dtype=torch.bfloat16, device="cuda")
    out = poison_(torch.empty((11, 256), dtype=torch.uint8, device="cuda"))
    sf = poison_(torch.empty((11, 2), dtype=torch.float32, device="cuda"))
    say("dispatch quant after capacity error")
    h.dispatch_quant(x, "f32", zero_padding=True, out_x=out, out_sf=sf)
    torch.cuda.synchronize()
    assert np.all(u8(out) == POISON) and np.all(u8(sf) == POISON)
