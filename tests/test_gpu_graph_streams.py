"""Capture-safety and stream independence.

The pages' CUDA-graph and async-stream notes (DeepEP notes ch.8 s8.2, the vLLM
PR digest on graph-safe joins) require that the path can run inside a graph
and on any stream.  Here layout + dispatch + combine are captured once in a
HIP graph and replayed with new routing and payloads copied into the captured
inputs, with eager work between replays; every replay is checked against the
oracle.  The same is done for the quantising dispatch, the combine backward
and the rank-layout calls.  A last test runs two handles on two streams at
once."""
import numpy as np
import pytest
import torch

import combine_ep_layout_08_amd as ep
import oracle
from tests.gpu_util import needs_gpu, say, u16

pytestmark = [pytest.mark.gpu, needs_gpu]

T, K, E, A, H = 1500, 8, 64, 16, 1024


def _routing(rng, t=T):
    idx = np.stack([rng.permutation(E)[:K] for _ in range(t)]).astype(np.int64)
    idx = np.where(rng.random((t, K)) < 0.15, -1, idx)
    w = rng.random((t, K), dtype=np.float32)
    return idx, w


def _check(idx, w, x, y, out_x, out, cap):
    lay = oracle.layout(idx, E, A, cap)
    n = lay.num_expanded
    ox, _, _ = oracle.dispatch(u16(x).view(np.uint8), lay, cap)
    routed = np.nonzero(lay.src_meta[:n] >= 0)[0]      # gap rows are unspecified
    np.testing.assert_array_equal(u16(out_x)[routed], ox[routed].view(np.uint16))
    exp = oracle.combine(u16(y), idx, lay.dst, w)
    np.testing.assert_array_equal(u16(out), exp)


@pytest.mark.parametrize("T", [T, 200])     # count + place, and the one-launch layout
def test_graph_capture_and_replay(T):
    rng = np.random.default_rng(0)
    h = ep.Handle(T, K, E, A)
    cap = h.capacity
    idx_s = torch.zeros((T, K), dtype=torch.int64, device="cuda")
    w_s = torch.zeros((T, K), dtype=torch.float32, device="cuda")
    x_s = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    y_s = torch.zeros((cap, H), dtype=torch.bfloat16, device="cuda")
    out_x = torch.zeros((cap, H), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    idx0, w0 = _routing(rng, T)
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
    say("graph capture", T)
    with torch.cuda.graph(g):
        h.layout(idx_s)
        h.dispatch(x_s, out_x=out_x)
        h.combine(y_s, topk_weights=w_s, out=out)
    other = ep.Handle(T, K, E, A)
    for rep in range(5):
        idx, w = _routing(rng, T)
        x = torch.randn((T, H), generator=torch.Generator().manual_seed(rep)).to(torch.bfloat16)
        y = torch.randn((cap, H), generator=torch.Generator().manual_seed(100 + rep)).to(
            torch.bfloat16)
        idx_s.copy_(torch.from_numpy(idx))
        w_s.copy_(torch.from_numpy(w))
        x_s.copy_(x)
        y_s.copy_(y)
        say("graph replay", rep)
        g.replay()
        other.layout(torch.from_numpy(_routing(rng, T)[0]).cuda())     # eager work between
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


def test_graph_capture_of_the_other_calls():
    """The quantising dispatch, the backward pair and the rank-layout calls
    captured after a layout in one graph, replayed with new routing and rows
    (eager work between replays); every replay checked against the oracle."""
    rng = np.random.default_rng(3)
    T2, K2, E2, A2, H2 = 600, 4, 32, 8, 512
    h = ep.Handle(T2, K2, E2, A2)
    cap = h.capacity
    idx_s = torch.zeros((T2, K2), dtype=torch.int64, device="cuda")
    w_s = torch.zeros((T2, K2), dtype=torch.float32, device="cuda")
    x_s = torch.zeros((T2, H2), dtype=torch.bfloat16, device="cuda")
    y_s = torch.zeros((cap, H2), dtype=torch.bfloat16, device="cuda")
    g_s = torch.zeros((T2, H2), dtype=torch.bfloat16, device="cuda")
    qx = torch.zeros((cap, H2), dtype=torch.uint8, device="cuda")
    qsf = torch.zeros((cap, H2 // 128), dtype=torch.float32, device="cuda")
    gy = torch.zeros((cap, H2), dtype=torch.bfloat16, device="cuda")
    rx = torch.zeros((T2, H2), dtype=torch.bfloat16, device="cuda")
    ri = torch.zeros((T2, K2), dtype=torch.int64, device="cuda")
    rw = torch.zeros((T2, K2), dtype=torch.float32, device="cuda")
    rout = torch.zeros((T2, H2), dtype=torch.bfloat16, device="cuda")

    def calls():
        h.layout(idx_s)
        h.dispatch_quant(x_s, "f32", out_x=qx, out_sf=qsf)
        h.combine_backward(g_s, topk_weights=w_s, y=y_s, grad_y=gy)
        h.dispatch_rank(x_s, topk_weights=w_s, out_x=rx, out_topk_idx=ri, out_topk_weights=rw)
        h.combine_rank(rx, bias_0=g_s, out=rout)

    def route():
        idx = np.stack([rng.permutation(E2)[:K2] for _ in range(T2)]).astype(np.int64)
        return np.where(rng.random((T2, K2)) < 0.2, -1, idx)

    idx_s.copy_(torch.from_numpy(route()))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("graph capture other calls")
    with torch.cuda.graph(g):
        calls()
    other = ep.Handle(T2, K2, E2, A2)
    for rep in range(3):
        idx = route()
        w = rng.random((T2, K2), dtype=np.float32)
        gen = torch.Generator().manual_seed(rep)
        x = torch.randn((T2, H2), generator=gen).to(torch.bfloat16)
        y = torch.randn((cap, H2), generator=gen).to(torch.bfloat16)
        gr = torch.randn((T2, H2), generator=gen).to(torch.bfloat16)
        for dst_t, src_t in ((idx_s, torch.from_numpy(idx)), (w_s, torch.from_numpy(w)),
                             (x_s, x), (y_s, y), (g_s, gr)):
            dst_t.copy_(src_t)
        say("graph replay other calls", rep)
        g.replay()
        other.layout(torch.from_numpy(route()).cuda())          # eager work between
        torch.cuda.synchronize()
        lay = oracle.layout(idx, E2, A2, cap)
        n = lay.num_expanded
        routed = np.nonzero(lay.src_meta[:n] >= 0)[0]
        oq, osf, _ = oracle.dispatch_quant(u16(x), lay, cap, oracle.SF_F32)
        np.testing.assert_array_equal(qx.cpu().numpy()[routed], oq[routed])
        np.testing.assert_array_equal(qsf.cpu().numpy().view(np.uint32)[routed], osf[routed])
        ogy = np.zeros((cap, H2), np.uint16)
        ogy, _, _ = oracle.combine_backward(u16(gr), lay, idx, w, u16(y), None, capacity=cap,
                                            want_grad_w=False, grad_y=ogy)
        np.testing.assert_array_equal(u16(gy)[routed], ogy[routed])
        row, _, nr = oracle.rank_layout(idx, E2)
        ox, _, oi, ow = oracle.dispatch_rank(u16(x).view(np.uint8), idx, E2, row, T2, weights=w)
        np.testing.assert_array_equal(u16(rx)[:nr], ox[:nr].view(np.uint16))
        np.testing.assert_array_equal(ri.cpu().numpy()[:nr], oi[:nr])
        np.testing.assert_array_equal(rw.cpu().numpy()[:nr], ow[:nr])
        np.testing.assert_array_equal(u16(rout), oracle.combine_rank(u16(rx), row, u16(gr)))


def test_binding_passes_the_current_stream():
    """The binding hands the library the raw handle of the current stream,
    the same value torch reports for it, on the default stream and inside a
    stream context."""
    assert ep._stream() == torch.cuda.current_stream().cuda_stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert ep._stream() == s.cuda_stream == torch.cuda.current_stream().cuda_stream
