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
