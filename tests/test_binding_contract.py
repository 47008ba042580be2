"""Hermetic contract tests of the Python binding (no GPU, no library): a fake
C library records every call, host tensors stand in for device tensors, and
the tests check the argument plumbing - pointers, element strides, scale-pack
counts, the column-major TMA stride, argument order, the stream, status
codes turned into exceptions, and that the handle keeps its topk_idx."""
import numpy as np
import pytest
import torch

import combine_ep_layout_08_amd as ep

STREAM = 0xABC


class FakeLib:
    def __init__(self, status=0):
        self.calls = []
        self.status = status

    def __getattr__(self, name):
        def call(*args):
            self.calls.append((name, args))
            if name == "ep_capacity_bound":
                T, K, E, A = args
                return (T * min(K, E) + (A - 1) * E + A - 1) // A * A
            if name == "ep_workspace_bytes":
                return 1 << 16
            if name == "ep_tma_aligned_rows":
                return (args[0] + 3) // 4 * 4
            if name == "ep_sf_packs":
                H, fmt = args
                return H // 128 if fmt == 0 else (H // 128 + 3) // 4
            if name == "ep_status_str":
                return b"fake status"
            return self.status
        return call

    def last(self, name):
        return [a for n, a in self.calls if n == name][-1]


@pytest.fixture
def fake(monkeypatch):
    lib = FakeLib()
    monkeypatch.setattr(ep, "lib", lambda: lib)
    monkeypatch.setattr(ep, "_stream", lambda: STREAM)

    def host_ok(t, name):
        ep._need(t.is_contiguous(), f"{name} must be contiguous")
    monkeypatch.setattr(ep, "_dev", host_ok)
    monkeypatch.setattr(ep, "_dev_strided", lambda t, name: None)
    return lib


def _handle(fake, T=16, K=4, E=8, A=4):
    h = ep.Handle(T, K, E, A, device="cpu")
    h.h.num_tokens, h.h.num_topk, h.h.num_experts, h.h.max_tokens = T, K, E, T
    return h


def test_handle_init_and_layout_keep_their_inputs(fake):
    h = _handle(fake)
    args = fake.last("ep_handle_init")
    assert args[1:6] == (16, 4, 8, 4, h.capacity)
    assert args[6] == h.workspace.data_ptr() and args[7] == 1 << 16 and args[8] == STREAM
    idx = torch.zeros((16, 4), dtype=torch.int32)
    h.layout(idx)
    la = fake.last("ep_layout")
    assert la[1] == idx.data_ptr() and la[2] == ep.EP_I32 and la[3] == 16 and la[5] == STREAM
    assert h.topk_idx is idx                          # borrowed: kept alive


def test_dispatch_plumbs_scale_packs_and_strides(fake):
    h = _handle(fake)
    T, H = 16, 1024
    x = torch.zeros((T, H), dtype=torch.uint8)
    sf_cols = torch.zeros((H // 128, T), dtype=torch.float32)
    sf = sf_cols.t()                                   # column-major source scales
    out_x, out_sf, _ = h.dispatch(x, sf=sf, col_major_sf=True)
    a = fake.last("ep_dispatch")
    assert a[2] == ep.EP_FP8_E4M3 and a[3] == H
    assert a[4] == sf.data_ptr() and (a[5], a[6]) == (1, T) and a[7] == H // 128
    tma = (h.capacity + 3) // 4 * 4
    assert (a[11], a[12]) == (1, tma) and out_sf.stride() == (1, tma)
    assert out_sf.shape == (h.capacity, H // 128) and a[10] == out_sf.data_ptr()
    assert a[14] == 0 and a[15] == STREAM
    packs = torch.zeros((T, 2), dtype=torch.int32)     # UE8M0 exponents, 4 per pack
    h.dispatch(x, sf=packs, zero_padding=True)
    a = fake.last("ep_dispatch")
    assert a[7] == 2 and (a[11], a[12]) == (2, 1) and a[14] == 1
    with pytest.raises(ValueError):
        h.dispatch(x, sf=torch.zeros((T, 3), dtype=torch.float32))   # fp32 must be [T, H/128]
    with pytest.raises(ValueError):
        h.dispatch(torch.zeros((T, 64), dtype=torch.bfloat16), sf=packs)   # scales with bf16


def test_combine_argument_order(fake):
    h = _handle(fake)
    T, H = 16, 64
    y = torch.zeros((h.capacity, H), dtype=torch.bfloat16)
    w = torch.zeros((T, 4), dtype=torch.float32)
    b0 = torch.zeros((T, H), dtype=torch.bfloat16)
    b1 = torch.ones((T, H), dtype=torch.bfloat16)
    out = h.combine(y, topk_weights=w, bias_0=b0, bias_1=b1)
    a = fake.last("ep_combine")
    assert a[1] == y.data_ptr() and a[2] == ep.EP_BF16 and a[3] == H and a[4] == w.data_ptr()
    assert a[5] is None and a[6] == b0.data_ptr() and a[7] == b1.data_ptr()
    assert a[8] == out.data_ptr() and a[9] == STREAM


def test_quantiser_formats_and_outputs(fake):
    x = torch.zeros((8, 640), dtype=torch.bfloat16)
    q, sf = ep.quantize_fp8(x, "ue8m0")
    a = fake.last("ep_quantize_fp8")
    assert a[1:4] == (8, 640, ep.EP_SF_UE8M0) and a[4] == q.data_ptr() and a[5] == sf.data_ptr()
    assert sf.dtype == torch.int32 and sf.shape == (8, 2) and (a[6], a[7]) == (2, 1)
    q, sf = ep.quantize_fp8(x, "f32", col_major_sf=True)
    a = fake.last("ep_quantize_fp8")
    assert sf.dtype == torch.float32 and sf.shape == (8, 5) and (a[6], a[7]) == (1, 8)
    with pytest.raises(ValueError):
        ep.quantize_fp8(x, "e5m2")


def test_error_status_raises(fake):
    h = _handle(fake)
    fake.status = ep.EP_ERR_SHAPE
    with pytest.raises(ep.EpError, match="fake status"):
        h.combine(torch.zeros((h.capacity, 64), dtype=torch.bfloat16))


def test_bound_calls_pass_what_the_direct_calls_pass(fake, monkeypatch):
    """bind_layout / bind_dispatch / bind_combine marshal once; every call
    hands the C entry point the same arguments as the direct method, with
    the stream read at call time."""
    h = _handle(fake)
    T, K, H = 16, 4, 256
    idx = torch.zeros((T, K), dtype=torch.int64)
    x = torch.zeros((T, H), dtype=torch.bfloat16)
    w = torch.zeros((T, K), dtype=torch.float32)
    y = torch.zeros((h.capacity, H), dtype=torch.bfloat16)
    out_x = torch.zeros((h.capacity, H), dtype=torch.bfloat16)
    out = torch.zeros((T, H), dtype=torch.bfloat16)
    direct = []
    h.layout(idx)
    direct.append(fake.last("ep_layout"))
    h.dispatch(x, topk_weights=w, out_x=out_x, zero_padding=True)
    direct.append(fake.last("ep_dispatch"))
    h.combine(y, topk_weights=w, out=out)
    direct.append(fake.last("ep_combine"))
    bl = h.bind_layout(idx)
    bd = h.bind_dispatch(x, topk_weights=w, out_x=out_x, zero_padding=True)
    bc = h.bind_combine(y, topk_weights=w, out=out)
    n_before = len(fake.calls)
    assert bl() is h and h.topk_idx is idx
    assert bd()[0] is out_x and bc() is out
    bound = [a for _, a in fake.calls[n_before:]]
    assert [n for n, _ in fake.calls[n_before:]] == ["ep_layout", "ep_dispatch", "ep_combine"]
    for d, b in zip(direct, bound):
        assert d[1:] == b[1:]
    monkeypatch.setattr(ep, "_stream", lambda: STREAM + 1)
    bc()
    assert fake.last("ep_combine")[-1] == STREAM + 1


def test_bound_call_refuses_a_changed_token_count(fake):
    """A later layout with another token count makes a bound dispatch or
    combine refuse to run (its tensors were checked against the old count)."""
    h = _handle(fake)
    x = torch.zeros((16, 128), dtype=torch.bfloat16)
    y = torch.zeros((h.capacity, 128), dtype=torch.bfloat16)
    bd, bc = h.bind_dispatch(x), h.bind_combine(y)
    n_before = len(fake.calls)
    h.h.num_tokens = 12                               # what ep_layout does for 12 tokens
    for call in (bd, bc):
        with pytest.raises(ValueError, match="bound for 16 tokens"):
            call()
    assert len(fake.calls) == n_before                # nothing reached the library
    h.h.num_tokens = 16
    bd()
    assert fake.calls[-1][0] == "ep_dispatch"


def test_bound_call_raises_on_status(fake):
    h = _handle(fake)
    bc = h.bind_combine(torch.zeros((h.capacity, 64), dtype=torch.bfloat16))
    fake.status = ep.EP_ERR_NOT_LAID_OUT
    with pytest.raises(ep.EpError):
        bc()
