"""The profiling hook ep_time_next_call stamps events on exactly one call's
kernels, and the stamped interval is positive and within the host-measured
time of a synchronised call."""
import time

import pytest
import torch

import combine_ep_layout_08_amd as ep
from tests.gpu_util import needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]


def test_time_next_call_stamps_one_call():
    T, K, E, H = 2048, 8, 64, 1024
    idx = torch.randint(0, E, (T, K), device="cuda")
    x = torch.randn((T, H), device="cuda").to(torch.bfloat16)
    h = ep.Handle(T, K, E, 16)
    y = torch.randn((h.capacity, H), device="cuda").to(torch.bfloat16)
    for name, call in (("layout", lambda: h.layout(idx)),
                       ("dispatch", lambda: h.dispatch(x)),
                       ("combine", lambda: h.combine(y))):
        say("timing hook", name)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ep.time_next_call(s, e)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        call()
        torch.cuda.synchronize()
        host_ms = (time.perf_counter() - t0) * 1e3
        ms = s.elapsed_time(e)
        assert 0 < ms <= host_ms + 0.05, (name, ms, host_ms)
        # the hook is consumed: a second call leaves the events as they were
        call()
        torch.cuda.synchronize()
        assert s.elapsed_time(e) == ms
