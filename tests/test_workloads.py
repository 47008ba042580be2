"""The seeded input generator: deterministic per seed, and each workload has
the structure its recipe states (routing shape, empty-slot rate, weight
normalisation, FP8 block scaling).  CPU only; small token counts where the
full size is not needed."""
import dataclasses

import numpy as np
import pytest
import torch

import ep_workloads as W


def _small(name, tokens):
    return dataclasses.replace(W.CONFIGS[name], tokens=tokens)


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_routing_is_deterministic_per_seed(name):
    cfg = _small(name, min(W.CONFIGS[name].tokens, 512))
    a_idx, a_w = W.routing(cfg)
    b_idx, b_w = W.routing(cfg)
    np.testing.assert_array_equal(a_idx, b_idx)
    np.testing.assert_array_equal(a_w, b_w)
    c_idx, _ = W.routing(cfg, cfg.seed + 1)
    assert not np.array_equal(a_idx, c_idx)


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_routing_shape_ids_and_weights(name):
    cfg = _small(name, min(W.CONFIGS[name].tokens, 2048))
    idx, w = W.routing(cfg)
    assert idx.shape == (cfg.tokens, cfg.topk) and idx.dtype == np.int64
    assert w.shape == idx.shape and w.dtype == np.float32
    assert idx.min() >= -1 and idx.max() < cfg.experts
    for row in idx:                                    # distinct experts per token
        v = row[row >= 0]
        assert len(set(v.tolist())) == len(v)
    valid = idx >= 0
    assert np.all(w[~valid] == 0)
    has = valid.any(axis=1)
    np.testing.assert_allclose(w[has].astype(np.float64).sum(axis=1), 1.0, rtol=1e-6)
    rate = 1 - valid.mean()
    assert abs(rate - cfg.empty_prob) < 0.02


def test_prefill_routing_is_group_limited_and_ordered():
    cfg = _small("prefill", 2048)
    idx, w = W.routing(cfg)
    groups = idx // (cfg.experts // 8)
    assert max(len(set(g.tolist())) for g in groups) <= 4      # top-4 of 8 groups
    assert np.all(np.diff(w, axis=1) <= 0)      # sigmoid-normalised, slots by descending logit


def test_skewed_routing_follows_the_popularity_law():
    cfg = _small("skewed", 8192)
    idx, _ = W.routing(cfg)
    share = np.bincount(idx.ravel(), minlength=cfg.experts) / cfg.tokens
    # rank-1 popularity 0.27 with 8 draws without replacement: the hottest
    # expert is in most tokens, the coldest in few
    assert share.max() > 0.8 and share.min() < 0.1
    assert np.count_nonzero(share) == cfg.experts


def test_payloads_are_deterministic_and_fp8_scaled_per_block():
    a = W.payload_bf16(64, 256, 7, 3)
    b = W.payload_bf16(64, 256, 7, 3)
    assert torch.equal(a, b) and a.dtype == torch.bfloat16
    assert abs(float(a.float().std()) - 1.0) < 0.05
    q, sf = W.payload_fp8(96, 1024, 9, 3)
    q2, sf2 = W.payload_fp8(96, 1024, 9, 3)
    assert torch.equal(q, q2) and torch.equal(sf, sf2)
    codes = q.numpy()
    assert not np.any((codes & 0x7F) == 0x7F)               # no NaN codes
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    blk = np.abs(dec).reshape(96, 8, 128).max(axis=2)
    np.testing.assert_array_equal(blk, 448.0)               # amax maps to 448 in every block
    assert sf.shape == (96, 8) and np.all(sf.numpy() > 0)
