"""The oracle's all-cores leg (OpenMP over tokens in dispatch and the
combines) gives the same bytes as its plain sequential loops: every token
writes only its own slot rows and output row.  CPU only."""
import os

import numpy as np
import pytest
import torch

import ep_workloads as W
import oracle


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _run(cfg, tokens, threads):
    oracle.set_threads(threads)
    try:
        idx, w = W.routing(cfg)
        idx, w = np.ascontiguousarray(idx[:tokens]), np.ascontiguousarray(w[:tokens])
        T, K, E, A, H = tokens, cfg.topk, cfg.experts, cfg.alignment, cfg.hidden
        cap = oracle.capacity_bound(T, K, E, A)
        lay = oracle.layout(idx, E, A, cap)
        x = W.payload_bf16(T, H, cfg.seed, 3, "cpu")
        xb = _bits(x).view(np.uint8).reshape(T, 2 * H)
        sf = np.random.default_rng(cfg.seed).random((T, H // 128), dtype=np.float32)
        out_x, out_sf, out_w = oracle.dispatch(xb, lay, cap, sf=sf, weights=w, want_w=True,
                                               zero_padding=True, num_sf_packs=H // 128)
        y = _bits(W.payload_bf16(cap, H, cfg.seed, 4, "cpu"))
        bias = _bits(W.payload_bf16(E, H, cfg.seed, 5, "cpu", std=0.02))
        b0 = _bits(W.payload_bf16(T, H, cfg.seed + 7, 3, "cpu"))
        out = oracle.combine(y, idx, lay.dst, w, bias)
        out_tb = oracle.combine_token_bias(y, idx, lay.dst, w, bias, b0, b0)
        return out_x, out_sf, out_w, out, out_tb
    finally:
        oracle.set_threads(1)


@pytest.mark.parametrize("name,tokens", [("prefill", 1024), ("skewed", 2048), ("tiny", 64)])
def test_threads_give_the_sequential_bytes(name, tokens):
    cfg = W.CONFIGS[name]
    one = _run(cfg, tokens, 1)
    many = _run(cfg, tokens, max(2, min(8, len(os.sched_getaffinity(0)))))
    for a, b in zip(one, many):
        assert a.shape == b.shape and a.dtype == b.dtype
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
