"""Seeded synthetic inputs for MoE routing layout, dispatch and combine.

This module draws inputs only.  It holds no step of the layout, dispatch or
combine computation, so both the HIP path and the CPU oracle can be fed from it
without sharing any of the method's arithmetic.

Workloads follow the DeepSeek-V3/R1 routing settings that the DeepEP README
("Performance" section) benchmarks with: 4096 tokens per batch, hidden 7168,
top-4 groups, top-8 experts, FP8 dispatch and BF16 combine for training and
prefill, and 128 tokens per batch for decode.  No trained router is available,
so router logits are N(0,1) draws.

Random streams: one numpy ``SeedSequence(seed).spawn(6)``, consumed in the
fixed order [routing, empty-mask, weight-logits, x, y, bias].  Dense payloads
(x, y, bias) are drawn with a torch ``Generator`` seeded from the matching
child sequence, on the device the caller asks for, so that multi-GB inputs can
be drawn directly in device memory.  The same (seed, device) always yields the
same tensors.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

__all__ = ["Config", "CONFIGS", "Workload", "make", "routing",
           "payload_bf16", "payload_fp8"]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    tokens: int
    hidden: int
    experts: int
    topk: int
    alignment: int
    x_dtype: str            # "bf16" or "fp8"
    zero_padding: bool
    routing: str            # "uniform", "grouped", "zipf"
    empty_prob: float       # probability that a slot is -1
    weights: str            # "softmax" or "sigmoid_norm"
    bias: bool
    capacity: str           # "exact" (psum[E] after layout) or "bound"
    seed: int

    @property
    def fp8(self) -> bool:
        return self.x_dtype == "fp8"


CONFIGS = {
    # 64 tokens, hidden 256, 16 experts, top-4 distinct, 10% empty slots,
    # alignment 1, identity expert, no bias.
    "tiny": Config("tiny", 64, 256, 16, 4, 1, "bf16", False, "uniform", 0.1,
                   "softmax", False, "bound", 1001),
    # 128 tokens, hidden 7168 FP8 + 56 fp32 scales, 256 experts top-8,
    # alignment 128 with zero padding.
    "decode": Config("decode", 128, 7168, 256, 8, 128, "fp8", True, "uniform",
                     0.0, "softmax", False, "bound", 1002),
    # 4096 tokens, hidden 7168 FP8, 256 experts in 8 groups, group-limited
    # top-4 groups / top-8 experts, sigmoid-normalised weights, alignment 128.
    "prefill": Config("prefill", 4096, 7168, 256, 8, 128, "fp8", False,
                      "grouped", 0.0, "sigmoid_norm", False, "bound", 1003),
    # 16384 tokens, hidden 4096 bf16, 128 experts with Zipf(1.2) popularity,
    # alignment 64, zero padding, per-expert bias.
    "skewed": Config("skewed", 16384, 4096, 128, 8, 64, "bf16", True, "zipf",
                     0.0, "softmax", True, "bound", 1004),
    # 32768 tokens, hidden 7168 bf16, 256 experts top-8, 20% empty slots,
    # alignment 128, output sized at the worst-case bound; the handle is reused.
    "large": Config("large", 32768, 7168, 256, 8, 128, "bf16", False, "uniform",
                    0.2, "softmax", False, "bound", 1005),
}


# Benchmark-only shape (not a parity configuration of its own: the layout
# tests cover its form at 102401-110000 tokens): prefill routing at 110000
# tokens, 880000 slots, more than 400 layout tiles of 2048 slots, the size
# at which the layout takes its single-pass decoupled-lookback form.
BENCH_CONFIGS = {
    "prefill_110k": Config("prefill_110k", 110000, 7168, 256, 8, 128, "fp8", False,
                           "grouped", 0.0, "sigmoid_norm", False, "bound", 1006),
}


def config(name: str) -> Config:
    """A parity configuration or a benchmark-only shape, by name."""
    return CONFIGS[name] if name in CONFIGS else BENCH_CONFIGS[name]


def _children(seed: int):
    return np.random.SeedSequence(seed).spawn(6)


def _torch_seed(child: np.random.SeedSequence) -> int:
    return int(child.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


# ----------------------------------------------------------------------------
# routing


def _uniform_topk(rng: np.random.Generator, T: int, E: int, K: int) -> np.ndarray:
    """The first K entries of an independent random permutation of E per token."""
    keys = rng.random((T, E))
    return np.argsort(keys, axis=1, kind="stable")[:, :K].astype(np.int64)


def _grouped_topk(rng: np.random.Generator, T: int, E: int, K: int,
                  groups: int = 8, topk_groups: int = 4):
    """Group-limited gating: keep the top groups by group-max logit, then the
    top-K experts inside them, slots sorted by descending logit.  Ties break to
    the lower index (stable sorts on negated keys)."""
    logits = rng.standard_normal((T, E), dtype=np.float32)
    per = E // groups
    gscore = logits.reshape(T, groups, per).max(axis=2)
    gorder = np.argsort(-gscore, axis=1, kind="stable")[:, :topk_groups]
    keep = np.zeros((T, groups), dtype=bool)
    np.put_along_axis(keep, gorder, True, axis=1)
    masked = np.where(np.repeat(keep, per, axis=1), logits, -np.inf)
    idx = np.argsort(-masked, axis=1, kind="stable")[:, :K].astype(np.int64)
    scores = np.take_along_axis(logits, idx, axis=1)
    return idx, scores


def _zipf_topk(rng: np.random.Generator, T: int, E: int, K: int, s: float = 1.2):
    """K distinct experts per token without replacement from popularity
    p_r ~ r^-s over a seeded permutation of ranks (Gumbel-top-k, which equals
    sequential draws without replacement)."""
    ranks = np.arange(1, E + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    perm = rng.permutation(E)                  # expert perm[r] has rank r+1
    logp = np.empty(E)
    logp[perm] = np.log(p)
    g = rng.gumbel(size=(T, E))
    return np.argsort(-(logp[None, :] + g), axis=1, kind="stable")[:, :K].astype(np.int64)


def routing(cfg: Config, seed: Optional[int] = None):
    """Return (topk_idx int64 [T,K], topk_weights float32 [T,K]) as numpy.

    -1 marks an empty slot.  Weights are 0 on empty slots and normalised over
    the valid slots of each token.
    """
    seed = cfg.seed if seed is None else seed
    c_route, c_empty, c_w, _, _, _ = _children(seed)
    rng = np.random.Generator(np.random.PCG64(c_route))
    T, E, K = cfg.tokens, cfg.experts, cfg.topk
    scores = None
    if cfg.routing == "uniform":
        idx = _uniform_topk(rng, T, E, K)
    elif cfg.routing == "grouped":
        idx, scores = _grouped_topk(rng, T, E, K)
    elif cfg.routing == "zipf":
        idx = _zipf_topk(rng, T, E, K)
    else:
        raise ValueError(cfg.routing)
    if cfg.empty_prob > 0:
        erng = np.random.Generator(np.random.PCG64(c_empty))
        empty = erng.random((T, K)) < cfg.empty_prob
        idx = np.where(empty, -1, idx)
    valid = idx >= 0
    wrng = np.random.Generator(np.random.PCG64(c_w))
    if cfg.weights == "sigmoid_norm":
        sig = 1.0 / (1.0 + np.exp(-scores.astype(np.float64)))
        sig = np.where(valid, sig, 0.0)
        w = sig / np.maximum(sig.sum(axis=1, keepdims=True), 1e-300)
    else:
        logits = wrng.standard_normal((T, K))
        logits = np.where(valid, logits, -np.inf)
        m = np.max(logits, axis=1, keepdims=True)
        m = np.where(np.isfinite(m), m, 0.0)
        ex = np.where(valid, np.exp(logits - m), 0.0)
        w = ex / np.maximum(ex.sum(axis=1, keepdims=True), 1e-300)
    return idx, w.astype(np.float32)


# ----------------------------------------------------------------------------
# dense payloads


def _gen(child, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(child))
    return g


def payload_bf16(rows: int, hidden: int, seed: int, stream: int,
                 device="cpu", std: float = 1.0) -> torch.Tensor:
    """bf16 [rows, hidden] from N(0, std^2), float32 draws rounded by torch."""
    child = _children(seed)[stream]
    g = _gen(child, device)
    out = torch.empty((rows, hidden), dtype=torch.bfloat16, device=device)
    chunk = max(1, (1 << 26) // max(hidden, 1))
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        v = torch.randn((r1 - r0, hidden), generator=g, dtype=torch.float32,
                        device=device)
        if std != 1.0:
            v.mul_(std)
        out[r0:r1] = v.to(torch.bfloat16)
    return out


def payload_fp8(rows: int, hidden: int, seed: int, stream: int, device="cpu"):
    """FP8 E4M3FN [rows, hidden] plus fp32 scales [rows, hidden/128].

    Per (row, 128-channel block): s = max(amax, 1e-12) / 448 and
    q = e4m3fn(clamp(x / s, -448, 448)) with torch's round-to-nearest-even
    conversion.  Returned as (uint8 codes, float32 scales).
    """
    assert hidden % 128 == 0
    child = _children(seed)[stream]
    g = _gen(child, device)
    q = torch.empty((rows, hidden), dtype=torch.uint8, device=device)
    sf = torch.empty((rows, hidden // 128), dtype=torch.float32, device=device)
    chunk = max(1, (1 << 24) // hidden)
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        v = torch.randn((r1 - r0, hidden // 128, 128), generator=g,
                        dtype=torch.float32, device=device)
        s = v.abs().amax(dim=2).clamp_min(1e-12) / 448.0
        c = (v / s[:, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
        q[r0:r1] = c.view(torch.uint8).reshape(r1 - r0, hidden)
        sf[r0:r1] = s
    return q, sf


@dataclasses.dataclass
class Workload:
    cfg: Config
    topk_idx: np.ndarray            # int64 [T, K]
    topk_weights: np.ndarray        # float32 [T, K]
    x: Optional[torch.Tensor]       # bf16 [T, H] or uint8 [T, H] (fp8 codes)
    sf: Optional[torch.Tensor]      # float32 [T, H/128] for fp8, else None
    y: Optional[torch.Tensor]       # bf16 [y_rows, H] expert outputs
    bias: Optional[torch.Tensor]    # bf16 [E, H] or None


def make(name_or_cfg, seed: Optional[int] = None, device="cpu",
         y_rows: Optional[int] = None, with_x: bool = True) -> Workload:
    """Draw one workload.  Routing is numpy on the host; payloads are drawn on
    ``device``.  Expert outputs y are drawn only when ``y_rows`` is given (the
    caller sizes them to its expanded-buffer capacity); a row of y is only read
    where the layout placed a routed slot."""
    cfg = config(name_or_cfg) if isinstance(name_or_cfg, str) else name_or_cfg
    seed = cfg.seed if seed is None else seed
    idx, w = routing(cfg, seed)
    x = sf = y = b = None
    if with_x:
        if cfg.fp8:
            x, sf = payload_fp8(cfg.tokens, cfg.hidden, seed, 3, device)
        else:
            x = payload_bf16(cfg.tokens, cfg.hidden, seed, 3, device)
    if y_rows is not None:
        y = payload_bf16(y_rows, cfg.hidden, seed, 4, device)
    if cfg.bias:
        b = payload_bf16(cfg.experts, cfg.hidden, seed, 5, device, std=0.02)
    return Workload(cfg, idx, w, x, sf, y, b)
