"""Bound calls (Handle.bind_layout / bind_dispatch / bind_combine) on the GPU:
bound once, called with new routing and payloads copied into the bound
tensors, every result against the oracle; and a layout with another token
count makes the bound dispatch and combine refuse to run."""
import numpy as np
import pytest
import torch

import combine_ep_layout_08_amd as ep
import oracle
from tests.gpu_util import needs_gpu, say, u16

pytestmark = [pytest.mark.gpu, needs_gpu]

K, E, A, H = 8, 64, 16, 512


def _routing(rng, T):
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    idx = np.where(rng.random((T, K)) < 0.15, -1, idx)
    return idx, rng.random((T, K), dtype=np.float32)


@pytest.mark.parametrize("T", [200, 3000])     # one-launch layout, count + place
def test_bound_calls_follow_new_inputs(T):
    rng = np.random.default_rng(T)
    h = ep.Handle(T, K, E, A)
    cap = h.capacity
    idx_s = torch.zeros((T, K), dtype=torch.int64, device="cuda")
    w_s = torch.zeros((T, K), dtype=torch.float32, device="cuda")
    x_s = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    y_s = torch.zeros((cap, H), dtype=torch.bfloat16, device="cuda")
    idx_s.copy_(torch.from_numpy(_routing(rng, T)[0]))
    layout = h.bind_layout(idx_s)
    layout()
    dispatch = h.bind_dispatch(x_s)
    combine = h.bind_combine(y_s, topk_weights=w_s)
    for rep in range(4):
        idx, w = _routing(rng, T)
        x = torch.randn((T, H), generator=torch.Generator().manual_seed(rep)).to(torch.bfloat16)
        y = torch.randn((cap, H), generator=torch.Generator().manual_seed(50 + rep)).to(
            torch.bfloat16)
        idx_s.copy_(torch.from_numpy(idx))
        w_s.copy_(torch.from_numpy(w))
        x_s.copy_(x)
        y_s.copy_(y)
        say("bound calls", T, rep)
        layout()
        out_x, _, _ = dispatch()
        out = combine()
        torch.cuda.synchronize()
        lay = oracle.layout(idx, E, A, cap)
        n = lay.num_expanded
        routed = np.nonzero(lay.src_meta[:n] >= 0)[0]
        ox, _, _ = oracle.dispatch(u16(x).view(np.uint8), lay, cap)
        np.testing.assert_array_equal(u16(out_x)[routed], ox[routed].view(np.uint16))
        np.testing.assert_array_equal(u16(out), oracle.combine(u16(y), idx, lay.dst, w))
    h.read_counts()


def test_bound_calls_refuse_another_token_count():
    rng = np.random.default_rng(7)
    T = 300
    h = ep.Handle(T, K, E, A)
    idx = torch.from_numpy(_routing(rng, T)[0]).cuda()
    h.layout(idx)
    dispatch = h.bind_dispatch(torch.zeros((T, H), dtype=torch.bfloat16, device="cuda"))
    combine = h.bind_combine(torch.zeros((h.capacity, H), dtype=torch.bfloat16, device="cuda"))
    say("bound calls, token count changed")
    h.layout(idx[:T - 50])                       # a layout of fewer tokens on the same handle
    for call in (dispatch, combine):
        with pytest.raises(ValueError, match="bound for 300 tokens"):
            call()
    h.layout(idx)                                # back to the bound count: runs again
    dispatch()
    combine()
    torch.cuda.synchronize()
    h.read_counts()
