"""Capture-safety and stream independence.

The pages' CUDA-graph and async-stream notes (DeepEP notes ch.8 s8.2, the vLLM
PR digest on graph-safe joins) require that the path can run inside a graph
and on any stream.  Here layout + dispatch + combine are captured once in a
HIP graph and replayed with new routing and payloads copied into the captured
inputs, with eager work between replays; every replay is checked against the
oracle.  A second test runs two handles on two streams at once."""
import numpy as np
import pytest
import torch

import combine_ep_layout_08_amd as ep
import oracle
from tests.gpu_util import needs_gpu, say, u16

pytestmark = [pytest.mark.gpu, needs_gpu]

T, K, E, A, H = 1500, 8, 64, 16, 1024


def _routing(rng):
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    idx = np.where(rng.random((T, K)) < 0.15, -1, idx)
    w = rng.random((T, K), dtype=np.float32)
    return idx, w


def _check(idx, w, x, y, out_x, out, cap):
    lay = oracle.layout(idx, E, A, cap)
    n = lay.num_expanded
    ox, _, _ = oracle.dispatch(u16(x).view(np.uint8), lay, cap)
    routed = np.nonzero(lay.src_meta[:n] >= 0)[0]      # gap rows are unspecified
    np.testing.assert_array_equal(u16(out_x)[routed], ox[routed].view(np.uint16))
    exp = oracle.combine(u16(y), idx, lay.dst, w)
    np.testing.assert_array_equal(u16(out), exp)


def test_graph_capture_and_replay():
    rng = np.random.default_rng(0)
    h = ep.Handle(T, K, E, A)
    cap = h.capacity
    idx_s = torch.zeros((T, K), dtype=torch.int64, device="cuda")
    w_s = torch.zeros((T, K), dtype=torch.float32, device="cuda")
    x_s = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    y_s = torch.zeros((cap, H), dtype=torch.bfloat16, device="cuda")
    out_x = torch.zeros((cap, H), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    idx0, w0 = _routing(rng)
    idx_s.copy_(torch.from_numpy(idx0))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                      # warm-up outside capture
        h.layout(idx_s)
        h.dispatch(x_s, out_x=out_x)
        h.combine(y_s, topk_weights=w_s, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("graph capture")
    with torch.cuda.graph(g):
        h.layout(idx_s)
        h.dispatch(x_s, out_x=out_x)
        h.combine(y_s, topk_weights=w_s, out=out)
    other = ep.Handle(T, K, E, A)
    for rep in range(5):
        idx, w = _routing(rng)
        x = torch.randn((T, H), generator=torch.Generator().manual_seed(rep)).to(torch.bfloat16)
        y = torch.randn((cap, H), generator=torch.Generator().manual_seed(100 + rep)).to(
            torch.bfloat16)
        idx_s.copy_(torch.from_numpy(idx))
        w_s.copy_(torch.from_numpy(w))
        x_s.copy_(x)
        y_s.copy_(y)
        say("graph replay", rep)
        g.replay()
        other.layout(torch.from_numpy(_routing(rng)[0]).cuda())     # eager work between
        torch.cuda.synchronize()
        _check(idx, w, x, y, out_x, out, cap)


def test_two_handles_on_two_streams():
    rng = np.random.default_rng(1)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    handles = [ep.Handle(T, K, E, A), ep.Handle(T, K, E, A)]
    for rep in range(4):
        jobs = []
        keep = []                      # device inputs stay alive until the streams finish
        for s, h in zip(streams, handles):
            idx, w = _routing(rng)
            x = torch.randn((T, H), generator=torch.Generator().manual_seed(rep)).to(torch.bfloat16)
            y = torch.randn((h.capacity, H)).to(torch.bfloat16)
            xd, yd = x.cuda(), y.cuda()
            idx_d, w_d = torch.from_numpy(idx).cuda(), torch.from_numpy(w).cuda()
            out_x = torch.zeros((h.capacity, H), dtype=torch.bfloat16, device="cuda")
            out = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                h.layout(idx_d)
                h.dispatch(xd, out_x=out_x)
                h.combine(yd, topk_weights=w_d, out=out)
            jobs.append((idx, w, x, y, out_x, out, h.capacity))
            keep.append((xd, yd, idx_d, w_d))
        say("two streams", rep)
        torch.cuda.synchronize()
        for j in jobs:
            _check(*j)
