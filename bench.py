"""Benchmark: MoE routing layout + dispatch + combine on one MI355X.

One step is one pass of the whole hot path over one batch: ep_layout on
topk_idx, ep_dispatch of the FP8 token rows (+ fp32 scales) into the
expert-expanded layout, ep_combine of bf16 expert outputs back to token order
with fp32 weights.  Default workload: prefill, 4096 tokens x hidden 7168,
256 experts in 8 groups (group-limited top-4 groups, top-8 experts),
expert_alignment 128, buffers sized at the worst-case bound (65280 rows).
Inputs are seeded synthetic data, resident in HBM before timing starts.

Prints one JSON line.  ``value`` is the whole step's algorithmic HBM
throughput (GB/s) over back-to-back steps.  Per-call figures (``kernels``)
follow the cache-cold protocol: every timed call runs right after a 1 GiB
read that leaves L2 and the 256 MB MALL full of unrelated clean lines, and
is timed by HIP events attached to its own kernel dispatches
(ep_time_next_call); median, p10, p90 and mean over the calls.  Back-to-back
per-call figures are the secondary ones (``kernels_back_to_back``).  Beside
them: the calls' time including the write-back of what they leave dirty in
the MALL, bandwidth ceilings measured with plain kernels of the same access
patterns (libep_ceilings.so), the roofline of dispatch and combine, and the
CPU oracle's throughput on the host's cores as a baseline.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, AMD published peak
MALL_BYTES = 256 << 20          # MI355X last-level cache (Infinity Cache)
FLUSH_BYTES = 1 << 30           # the cache flush: a 1 GiB read
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "hbm_counters.json")
CSRC = os.path.join(ROOT, "combine_ep_layout_08_amd", "csrc")
CEILINGS_LIB = os.path.join(ROOT, "combine_ep_layout_08_amd", "libep_ceilings.so")
# Sources whose change makes a kernel's committed HBM counters stale: the
# kernel's file, the shared header, and the C ABI that chooses its launch
# (grid, which work units run, which outputs are written).
KERNEL_SOURCES = {"combine": ["ep_combine.hip", "ep_internal.h", "ep_api.cpp"],
                  "dispatch": ["ep_dispatch.hip", "ep_internal.h", "ep_api.cpp"],
                  "layout": ["ep_layout.hip", "ep_internal.h", "ep_api.cpp"]}
PHASES = ("steps", "cold", "writeback", "ceilings", "graph", "backward", "rank", "quant")


def parse(argv=None):
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="prefill", help="workload name (default prefill)")
    p.add_argument("--calls", type=int, default=50,
                   help="timed calls per entry point in the cache-cold protocol "
                        "(after 5 untimed ones)")
    p.add_argument("--phases", default=",".join(PHASES),
                   help="comma-separated phases to run, of: " + ", ".join(PHASES))
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the oracle timing (for profiler runs)")
    p.add_argument("--cpu-seconds", type=float, default=6.0,
                   help="minimum oracle time per CPU-baseline leg (1 thread, all cores)")
    p.add_argument("--cpu-row-tokens", type=int, default=512,
                   help="tokens of the CPU-oracle sample for the calls beyond the step")
    p.add_argument("--reps", type=int, default=30,
                   help="cache-cold calls per entry point in the backward, rank and "
                        "quantiser phases")
    p.add_argument("--graph-steps", type=int, default=200,
                   help="replays of one step captured in a HIP graph")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (profiler calibration)")
    a = p.parse_args(argv)
    a.phases = [x for x in a.phases.split(",") if x]
    bad = [x for x in a.phases if x not in PHASES]
    if bad:
        p.error(f"unknown phases {bad}")
    return a


def algorithmic_bytes(cfg, V: int, G: int, expanded: int, idx_bytes: int = 8) -> dict:
    """Bytes the method must move per call (read each input once, write each
    output once).  V = routed slots, G = alignment-gap rows."""
    T, K, H, E = cfg.tokens, cfg.topk, cfg.hidden, cfg.experts
    R = H if cfg.fp8 else 2 * H                 # row bytes of x
    S = 4 * (H // 128) if cfg.fp8 else 0        # scale bytes per row
    dispatch = T * (R + S) + V * (R + S) + 4 * T * K
    if cfg.zero_padding:
        dispatch += G * (R + S)
    combine = V * 2 * H + T * 2 * H + 4 * T * K + 4 * T * K
    if cfg.bias:
        combine += 2 * E * H + idx_bytes * T * K
    layout = idx_bytes * T * K + 4 * T * K + 4 * expanded + 4 * (2 * E + 1)
    return {"layout": layout, "dispatch": dispatch, "combine": combine}


def written_bytes(cfg, V: int, G: int) -> dict:
    """Bytes each call writes (the part that can sit dirty in the MALL)."""
    T, H = cfg.tokens, cfg.hidden
    R = H if cfg.fp8 else 2 * H
    S = 4 * (H // 128) if cfg.fp8 else 0
    return {"dispatch": (V + (G if cfg.zero_padding else 0)) * (R + S), "combine": T * 2 * H}


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_record(kernel: str, workload: str):
    """The committed rocprofv3 record of `kernel` at `workload`, or None."""
    if not os.path.exists(PROFILE_COUNTERS):
        return None
    with open(PROFILE_COUNTERS) as f:
        return json.load(f).get("workloads", {}).get(workload, {}).get(kernel)


def measured_traffic(kernel: str, workload: str = "prefill"):
    """(HBM bytes per launch from the committed FETCH_SIZE + WRITE_SIZE
    counters, calibrated on a plain copy; stale flag).  The bytes are None
    when no record exists or when the record was taken on another version of
    the kernel's sources (stale = True then, and bench.py warns)."""
    rec = counter_record(kernel, workload)
    if not rec:
        return None, False
    if rec.get("source_sha256_16") != kernel_source_hash(kernel):
        return None, True
    return rec.get("hbm_bytes_per_launch"), False


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads() -> int:
    """Host cores this process may use: its affinity mask, capped by
    OMP_NUM_THREADS when that is set (the GPU machine's share of the host)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


# ---------------------------------------------------------------- ceilings library

class Ceilings:
    """ctypes binding of libep_ceilings.so (bandwidth-ceiling kernels)."""

    def __init__(self, torch):
        if not os.path.exists(CEILINGS_LIB):
            raise RuntimeError(f"{CEILINGS_LIB} is missing: build it with "
                               "`python -m combine_ep_layout_08_amd.build`")
        self.torch = torch
        lib = ctypes.CDLL(CEILINGS_LIB)
        P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        sig = {"epc_read_sink_words": (I64, [SZ, I32, I32]),
               "epc_read": (ctypes.c_int, [P, SZ, P, I32, I32, I32, P, P, P]),
               "epc_write": (ctypes.c_int, [P, SZ, ctypes.c_uint32, I32, I32, I32, P, P, P]),
               "epc_copy": (ctypes.c_int, [P, P, SZ, I32, I32, I32, P, P, P]),
               "epc_row_store": (ctypes.c_int, [P, I64, I64, P, I64, I32, I32, P, P, P]),
               "epc_gather": (ctypes.c_int, [P, P, I64, I64, P, I64, I32, P, P, P]),
               "epc_empty": (ctypes.c_int, [I32, I32, P, P, P])}
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        self.lib = lib
        self.sink = torch.empty(int(lib.epc_read_sink_words(FLUSH_BYTES, 1, 0)) + 64,
                                dtype=torch.int32, device="cuda")
        self.flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")

    @staticmethod
    def _stream():
        import combine_ep_layout_08_amd as ep
        return ep._stream()

    @staticmethod
    def _ev(e):
        if e is None:
            return None
        if e.cuda_event == 0:
            e.record()
        return e.cuda_event

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed ({rc})")

    # Tunables of the sequential kernels: (vectors per thread, blocks,
    # non-temporal); FLUSH_TUNE reads with the most requests in flight.
    FLUSH_TUNE = (4, 0, 0)

    def read(self, t, nbytes=None, start=None, stop=None, tune=FLUSH_TUNE):
        n = t.numel() * t.element_size() if nbytes is None else nbytes
        self._ok(self.lib.epc_read(t.data_ptr(), n, self.sink.data_ptr(), *tune, self._stream(),
                                   self._ev(start), self._ev(stop)), "epc_read")

    def flush(self):
        """Leave L2 and the MALL full of clean lines of an unrelated buffer."""
        self.read(self.flush_buf)

    def write(self, t, nbytes, start=None, stop=None, tune=FLUSH_TUNE):
        self._ok(self.lib.epc_write(t.data_ptr(), nbytes, 7, *tune, self._stream(),
                                    self._ev(start), self._ev(stop)), "epc_write")

    def copy(self, dst, src, nbytes, start=None, stop=None, tune=FLUSH_TUNE):
        self._ok(self.lib.epc_copy(dst.data_ptr(), src.data_ptr(), nbytes, *tune, self._stream(),
                                   self._ev(start), self._ev(stop)), "epc_copy")

    def row_store(self, dst, rows, row_bytes, slot_row, tokens, K, start=None, stop=None,
                  nontemporal=False):
        self._ok(self.lib.epc_row_store(dst.data_ptr(), rows, row_bytes, slot_row.data_ptr(),
                                        tokens, K, 1 if nontemporal else 0, self._stream(),
                                        self._ev(start), self._ev(stop)), "epc_row_store")

    def empty(self, blocks, threads, start=None, stop=None):
        self._ok(self.lib.epc_empty(blocks, threads, self._stream(), self._ev(start),
                                    self._ev(stop)), "epc_empty")

    def gather(self, out, inp, rows, row_bytes, slot_row, tokens, K, start=None, stop=None):
        self._ok(self.lib.epc_gather(out.data_ptr(), inp.data_ptr(), rows, row_bytes,
                                     slot_row.data_ptr(), tokens, K, self._stream(),
                                     self._ev(start), self._ev(stop)), "epc_gather")


# ---------------------------------------------------------------- timing protocols

def _stats(us):
    import numpy as np
    return {"us_median": round(statistics.median(us), 2),
            "us_p10": round(float(np.percentile(us, 10)), 2),
            "us_p90": round(float(np.percentile(us, 90)), 2),
            "us_mean": round(statistics.mean(us), 2), "calls": len(us)}


def _rate(nbytes, us):
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"GBps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}


def events(torch, n):
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for a, b in ev:                 # created (first record) outside any timed region
        a.record()
        b.record()
    torch.cuda.synchronize()
    return ev


def time_cold(torch, ep, ceil, fn, calls, warm=5):
    """Cache-cold per-call protocol: `warm` untimed calls, then `calls` calls,
    each right after the 1 GiB flush (outside its events), each timed by
    events attached to its own kernels.  Returns the list of µs."""
    for _ in range(warm):
        ceil.flush()
        fn()
    ev = events(torch, calls)
    for e0, e1 in ev:
        ceil.flush()
        ep.time_next_call(e0, e1)
        fn()
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]


def time_back_to_back(torch, ep, fn, calls):
    """The same call repeated with nothing between: µs per call."""
    fn()
    ev = events(torch, calls)
    for e0, e1 in ev:
        ep.time_next_call(e0, e1)
        fn()
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]


def time_with_writeback(torch, ep, ceil, fn, calls, probe):
    """The call's time including the write-back of the lines it leaves dirty
    in the MALL: after a flush, the interval from the call's first kernel to
    the end of a fixed 1 GiB read (`probe`, which evicts those lines), minus
    the same read timed alone after a flush; medians over `calls` pairs taken
    in turn."""
    with_call, alone = [], []
    ev = events(torch, 2 * calls)
    for i in range(calls):
        e0, e1 = ev[2 * i]
        ceil.flush()
        ep.ep_time_next_call(e0.cuda_event, None)     # stamps the call's first kernel
        fn()
        ceil.read(probe, stop=e1)
        f0, f1 = ev[2 * i + 1]
        ceil.flush()
        ceil.read(probe, start=f0, stop=f1)
    torch.cuda.synchronize()
    for i in range(calls):
        e0, e1 = ev[2 * i]
        f0, f1 = ev[2 * i + 1]
        with_call.append(e0.elapsed_time(e1) * 1e3)
        alone.append(f0.elapsed_time(f1) * 1e3)
    a, b = statistics.median(with_call), statistics.median(alone)
    return {"call_plus_read_us_median": round(a, 2), "read_alone_us_median": round(b, 2),
            "us_with_writeback": round(a - b, 2)}


def time_ceiling(torch, ceil, fn, calls):
    """A ceiling kernel under the cache-cold protocol (fn takes start, stop)."""
    fn(None, None)
    ev = events(torch, calls)
    for e0, e1 in ev:
        ceil.flush()
        fn(e0, e1)
    torch.cuda.synchronize()
    return statistics.median(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)


def time_calls(torch, ep, ceil, calls, nbytes, reps, probe=None):
    """Cache-cold median/p10/p90 per call, the back-to-back mean and, with a
    1 GiB `probe`, the time including the write-back of what the call leaves
    dirty in the MALL (time_with_writeback)."""
    out = {}
    for name, fn in calls.items():
        cold = _stats(time_cold(torch, ep, ceil, fn, reps))
        warm = statistics.mean(time_back_to_back(torch, ep, fn, reps))
        out[name] = {**cold, "bytes": nbytes[name], **_rate(nbytes[name], cold["us_median"]),
                     "back_to_back_us_mean": round(warm, 2),
                     "back_to_back_GBps": _rate(nbytes[name], warm)["GBps"]}
        if probe is not None:
            wb = time_with_writeback(torch, ep, ceil, fn, max(10, reps // 2), probe)
            out[name]["with_writeback_us"] = wb["us_with_writeback"]
            out[name]["with_writeback_GBps"] = _rate(nbytes[name], wb["us_with_writeback"])["GBps"]
    return out


# ---------------------------------------------------------------- CPU oracle

def cpu_baseline(cfg, wl, y_host, min_seconds: float, threads: int):
    """The CPU oracle as it stands on the same workload: layout (single
    threaded) + dispatch + combine (OpenMP over tokens with `threads`) of the
    whole batch, repeated until ``min_seconds`` have passed; median step."""
    import numpy as np
    import oracle
    import torch
    cap = oracle.capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment)
    x_bytes = wl.x.contiguous().view(torch.uint8).cpu().numpy()
    sf = wl.sf.cpu().numpy() if wl.sf is not None else None
    out_x = np.empty((cap, x_bytes.shape[1]), np.uint8)
    out_sf = np.empty((cap, sf.shape[1]), np.float32) if sf is not None else None
    times = []
    oracle.set_threads(threads)
    try:
        t_end = time.perf_counter() + min_seconds
        while True:
            t0 = time.perf_counter()
            lay = oracle.layout(wl.topk_idx, cfg.experts, cfg.alignment, cap)
            oracle.dispatch(x_bytes, lay, cap, sf=sf, zero_padding=cfg.zero_padding,
                            out_x=out_x, out_sf=out_sf)
            oracle.combine(y_host, wl.topk_idx, lay.dst, wl.topk_weights)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() >= t_end and len(times) >= 3:
                break
    finally:
        oracle.set_threads(1)
    return statistics.median(times), len(times)


def _oracle_rank_quant(oracle, x_bits, idx, E, row, w):
    """The quantising rank dispatch as the oracle states it: quantise (fp32
    scales), then dispatch codes and scales into the rank layout."""
    q, sf = oracle.quantize_fp8(x_bits, oracle.SF_F32)
    return oracle.dispatch_rank(q, idx, E, row, idx.shape[0], sf=sf, weights=w,
                                num_sf_packs=sf.shape[1])


def cpu_oracle_rows(cfg, wl, tokens: int):
    """The CPU oracle (single thread, as it stands) on the first `tokens`
    tokens of the workload for every call beyond layout + dispatch +
    combine: GB/s of each call's algorithmic bytes at that sample size
    (median over repetitions filling 0.25 s, at least one).  Expert rows are
    zeros; the rows the quantiser and the backward read are N(0,1) bf16, so
    the quantiser's search does its real work (timing only)."""
    import numpy as np
    import oracle
    import torch
    import ep_workloads as W
    T, K, E, A, H = min(tokens, cfg.tokens), cfg.topk, cfg.experts, cfg.alignment, cfg.hidden
    idx = np.ascontiguousarray(wl.topk_idx[:T])
    w = np.ascontiguousarray(wl.topk_weights[:T])
    cap = oracle.capacity_bound(T, K, E, A)
    lay = oracle.layout(idx, E, A, cap)
    V = int((lay.dst >= 0).sum())
    row, _, nrecv = oracle.rank_layout(idx, E)
    y = np.zeros((cap, H), np.uint16)

    def bits(t):
        return t.view(torch.int16).numpy().view(np.uint16)

    g = bits(W.payload_bf16(T, H, cfg.seed + 1, 3, "cpu"))
    b = np.zeros((T, H), np.uint16)
    gwr = np.zeros(cap, np.float32)
    xq = bits(W.payload_bf16(T, H, cfg.seed + 5, 3, "cpu"))
    R, S = (H, 4 * (H // 128)) if cfg.fp8 else (2 * H, 0)
    x_bytes = np.zeros((T, R), np.uint8)
    sf = np.zeros((T, H // 128), np.float32) if cfg.fp8 else None
    P = {"f32": H // 128, "ue8m0": (H // 128 + 3) // 4}
    calls = {
        "combine_backward": (lambda: oracle.combine_backward(g, lay, idx, w, y, None, capacity=cap),
                             T * 2 * H + 2 * V * 2 * H + 12 * T * K),
        "dispatch_backward": (lambda: oracle.dispatch_backward(y, idx, lay.dst, gwr),
                              V * 2 * H + T * 2 * H + 16 * T * K),
        "dispatch_rank": (lambda: oracle.dispatch_rank(x_bytes, idx, E, row, T, sf=sf, weights=w),
                          T * (R + S) + nrecv * (R + S) + T * K * 12 + nrecv * K * 12 + 4 * T),
        "combine_rank": (lambda: oracle.combine_rank(g, row, b, b), nrecv * 2 * H + 3 * T * 2 * H + 4 * T),
        "combine_token_biases": (lambda: oracle.combine_token_bias(y, idx, lay.dst, w, None, b, b),
                                 V * 2 * H + 3 * T * 2 * H + 8 * T * K),
        "quantize_f32": (lambda: oracle.quantize_fp8(xq, oracle.SF_F32),
                         T * 2 * H + T * H + 4 * T * P["f32"]),
        "quantize_ue8m0": (lambda: oracle.quantize_fp8(xq, oracle.SF_UE8M0),
                           T * 2 * H + T * H + 4 * T * P["ue8m0"]),
        "dispatch_quant_f32": (lambda: oracle.dispatch_quant(xq, lay, cap, oracle.SF_F32),
                               T * 2 * H + V * (H + 4 * P["f32"]) + 4 * T * K),
        "dispatch_quant_ue8m0": (lambda: oracle.dispatch_quant(xq, lay, cap, oracle.SF_UE8M0),
                                 T * 2 * H + V * (H + 4 * P["ue8m0"]) + 4 * T * K),
        "dispatch_rank_quant_f32": (lambda: _oracle_rank_quant(oracle, xq, idx, E, row, w),
                                    T * 2 * H + nrecv * (H + 4 * P["f32"]) + 12 * T * K
                                    + 12 * nrecv * K + 4 * T),
    }
    out = {}
    for name, (fn, nb) in calls.items():
        times = []
        t_end = time.perf_counter() + 0.25            # repeat short calls; median
        while not times or time.perf_counter() < t_end:
            t0 = time.perf_counter()
            fn()
            times.append(time.perf_counter() - t0)
        dt = statistics.median(times)
        out[name] = {"GBps": round(nb / dt / 1e9, 3), "seconds": round(dt, 4), "tokens": T,
                     "repetitions": len(times), "cores": 1}
    return out


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


# ---------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path: the data-parallel share per GPU is the one-GPU workload.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration()
        return

    import combine_ep_layout_08_amd as ep
    import ep_workloads as W

    phases = set(args.phases)
    cfg = W.config(args.config)
    cap = ep.ep_capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment)
    wl = W.make(cfg, device="cuda", y_rows=cap)
    idx = torch.from_numpy(wl.topk_idx).cuda()
    w = torch.from_numpy(wl.topk_weights).cuda()
    h = ep.Handle(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment, cap)
    out_x = torch.empty((cap, cfg.hidden), dtype=wl.x.dtype, device="cuda")
    out_sf = (torch.empty((cap, cfg.hidden // 128), dtype=torch.float32, device="cuda")
              if cfg.fp8 else None)
    out = torch.empty((cfg.tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    ceil = Ceilings(torch)

    # The step's three calls, validated and marshalled once (bound calls:
    # the same entry points and kernels, about 3 us of host time per call
    # instead of 5-6, so small batches are not bound by the Python side).
    h.layout(idx)
    layout_call = h.bind_layout(idx)
    dispatch_call = h.bind_dispatch(wl.x, sf=wl.sf, zero_padding=cfg.zero_padding,
                                    out_x=out_x, out_sf=out_sf)
    combine_call = h.bind_combine(wl.y, topk_weights=w, bias=wl.bias, out=out)
    calls = {"layout": layout_call, "dispatch": dispatch_call, "combine": combine_call}
    # The uncached dispatch in one call (layout + copy; same outputs),
    # timed beside the step's calls in the cache-cold protocol.
    fused_call = h.bind_layout_dispatch(idx, wl.x, sf=wl.sf, zero_padding=cfg.zero_padding,
                                        out_x=out_x, out_sf=out_sf)
    # Both with streaming (non-temporal) row stores: the rows go on to HBM
    # during the call instead of staying dirty in the MALL.
    streaming_calls = {
        "dispatch_streaming": h.bind_dispatch(wl.x, sf=wl.sf, zero_padding=cfg.zero_padding,
                                              out_x=out_x, out_sf=out_sf, streaming=True),
        "layout_dispatch_streaming": h.bind_layout_dispatch(
            idx, wl.x, sf=wl.sf, zero_padding=cfg.zero_padding, out_x=out_x, out_sf=out_sf,
            streaming=True)}

    def step():
        layout_call()
        dispatch_call()
        combine_call()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    rc = h.read_counts()                        # raises on any device error
    V = int((wl.topk_idx >= 0).sum())
    G = int(rc["num_expanded"]) - V
    nbytes = algorithmic_bytes(cfg, V, G, int(rc["num_expanded"]))
    total_bytes = sum(nbytes.values())

    # Timed region: exactly `steps` steps back to back, synchronised on both
    # sides, nothing but the calls on the stream.
    ms_per_step = None
    kernels_b2b = None
    if "steps" in phases:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
        # Back-to-back per-call figures: `steps` more steps with each call's
        # kernels stamped by events attached to their dispatches (the stamps
        # cost GPU time of their own, ≈ 5 µs per call, so they stay out of
        # the timed region above).
        evs = [events(torch, 3) for _ in range(args.steps)]
        per = {k: [] for k in calls}
        for e3 in evs:
            for (e0, e1), (name, fn) in zip(e3, calls.items()):
                ep.time_next_call(e0, e1)
                fn()
        torch.cuda.synchronize()
        for e3 in evs:
            for (e0, e1), name in zip(e3, calls):
                per[name].append(e0.elapsed_time(e1) * 1e3)
        kernels_b2b = {k: {**_stats(v), **_rate(nbytes[k], statistics.mean(v))}
                       for k, v in per.items()}

    # Headline per-call figures: the cache-cold protocol.
    kernels = None
    if "cold" in phases:
        kernels = {}
        nbytes_all = dict(nbytes, layout_dispatch=nbytes["layout"] + nbytes["dispatch"],
                          dispatch_streaming=nbytes["dispatch"],
                          layout_dispatch_streaming=nbytes["layout"] + nbytes["dispatch"])
        for name, fn in {**calls, "layout_dispatch": fused_call, **streaming_calls}.items():
            st = _stats(time_cold(torch, ep, ceil, fn, args.calls))
            nb = nbytes_all[name]
            kernels[name] = {**st, "bytes": nb, **_rate(nb, st["us_median"]),
                             "mean_GBps": _rate(nb, st["us_mean"])["GBps"]}
            if name in ("dispatch", "combine"):
                traffic, stale = measured_traffic(name, cfg.name)
                kernels[name]["traffic"] = traffic
                if stale:
                    kernels[name]["traffic_stale"] = True
                    print(f"bench.py: committed HBM counters of {name} at {cfg.name} were taken "
                          "on other kernel sources; traffic reported as null", file=sys.stderr)
        h.read_counts()

    # Write-back: what the call leaves dirty in the MALL, evicted by a fixed
    # 1 GiB read; the difference to the read alone is the call's time with
    # its write-back.
    writeback = None
    if "writeback" in phases:
        probe = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
        wbytes = written_bytes(cfg, V, G)
        writeback = {"protocol": "flush; call + 1 GiB read, minus the 1 GiB read alone; "
                                 "medians", "mall_bytes": MALL_BYTES}
        wcalls = {**calls, "dispatch_streaming": streaming_calls["dispatch_streaming"]}
        for name in ("dispatch", "dispatch_streaming", "combine"):
            base = "dispatch" if name == "dispatch_streaming" else name
            r = time_with_writeback(torch, ep, ceil, wcalls[name], max(10, args.calls // 2),
                                    probe)
            r.update(_rate(nbytes[base], r["us_with_writeback"]))
            r["written_bytes"] = wbytes[base]
            r["writes_fit_mall"] = wbytes[base] < MALL_BYTES
            writeback[name] = r
        del probe
        h.read_counts()

    # Ceilings: plain kernels of the same access patterns, cache-cold.
    ceilings = None
    if "ceilings" in phases:
        # Sizes: the sequential write and copy move 4 GiB and 2 + 2 GiB, so
        # the 256 MB MALL, which can keep the last written lines dirty past
        # the kernel's end, absorbs at most ~6 % of their writes; the write
        # of the dispatch's own output bytes fits the MALL and shows what
        # absorption alone gives.
        n = 20
        big = 4 * FLUSH_BYTES
        a = torch.empty(big // 4, dtype=torch.int32, device="cuda")
        b = torch.empty(big // 8, dtype=torch.int32, device="cuda")
        a.fill_(3)
        K, H = cfg.topk, cfg.hidden
        R = H if cfg.fp8 else 2 * H
        wd = written_bytes(cfg, V, G)["dispatch"]
        wd16 = min(FLUSH_BYTES, (wd + 15) // 16 * 16)
        contig = torch.arange(cfg.tokens * K, dtype=torch.int32, device="cuda")
        y_rows = wl.y.shape[0]
        # The sequential ceilings keep the fastest of a few launch settings
        # (vectors per thread, grid, non-temporal).
        tunes = [(1, 0, 0), (2, 0, 0), (4, 0, 0), (8, 0, 0), (16, 0, 0), (4, 2048, 0),
                 (4, 8192, 0), (8, 4096, 0), (1, 0, 1), (4, 0, 1), (16, 0, 1)]
        seq = {"read_1GiB": lambda t: (lambda s, e: ceil.read(a, FLUSH_BYTES, s, e, tune=t)),
               "write_4GiB": lambda t: (lambda s, e: ceil.write(a, big, s, e, tune=t)),
               "copy_2GiB": lambda t: (lambda s, e: ceil.copy(b, a, big // 2, s, e, tune=t)),
               "write_dispatch_bytes": lambda t: (lambda s, e: ceil.write(a, wd16, s, e, tune=t))}
        ceil_us, ceil_tune = {}, {}
        for name, mk in seq.items():
            best = min(((time_ceiling(torch, ceil, mk(t), n), t) for t in tunes))
            ceil_us[name], ceil_tune[name] = best
        ceil_us.update({
            "row_store_dispatch_rows_streaming": time_ceiling(
                torch, ceil, lambda s, e: ceil.row_store(out_x, cap, R, h.dst_slot, cfg.tokens, K,
                                                         s, e, nontemporal=True), n),
            "row_store_dispatch_rows": time_ceiling(
                torch, ceil, lambda s, e: ceil.row_store(out_x, cap, R, h.dst_slot, cfg.tokens, K,
                                                         s, e), n),
            "gather_combine_rows": time_ceiling(
                torch, ceil, lambda s, e: ceil.gather(out, wl.y, y_rows, 2 * H, h.dst_slot,
                                                      cfg.tokens, K, s, e), n),
        })
        # The floor of a timed launch: an empty grid of one block and one of
        # the combine's grid size (one 256-thread block per 4 KB of output).
        comb_blocks = max(1, (cfg.tokens * (2 * H // 16) + 255) // 256)
        ceil_us["empty_1_block"] = time_ceiling(torch, ceil,
                                                lambda s, e: ceil.empty(1, 256, s, e), n)
        ceil_us["empty_combine_grid"] = time_ceiling(
            torch, ceil, lambda s, e: ceil.empty(comb_blocks, 256, s, e), n)
        if y_rows >= cfg.tokens * K:
            ceil_us["gather_contiguous_rows"] = time_ceiling(
                torch, ceil, lambda s, e: ceil.gather(out, wl.y, y_rows, 2 * H, contig,
                                                      cfg.tokens, K, s, e), n)
        moved = {"read_1GiB": FLUSH_BYTES, "write_4GiB": big, "copy_2GiB": big,
                 "write_dispatch_bytes": wd16,
                 "row_store_dispatch_rows": V * R,
                 "row_store_dispatch_rows_streaming": V * R,
                 "gather_combine_rows": V * 2 * H + cfg.tokens * 2 * H,
                 "gather_contiguous_rows": cfg.tokens * K * 2 * H + cfg.tokens * 2 * H,
                 "empty_1_block": 0, "empty_combine_grid": 0}
        ceilings = {k: {"us_median": round(v, 2), "bytes": moved[k],
                        **(_rate(moved[k], v) if moved[k] else {})}
                    for k, v in ceil_us.items()}
        ceilings["empty_combine_grid"]["blocks"] = comb_blocks
        for k, t in ceil_tune.items():
            ceilings[k]["tune"] = {"vec_per_thread": t[0], "blocks": t[1], "nontemporal": t[2]}
        ceilings["note"] = ("cache-cold medians of plain kernels (libep_ceilings.so): sequential "
                            "read, sequential write, 1:1 copy (best of 11 launch settings each), "
                            "a sequential write of the dispatch's output bytes (fits the MALL), "
                            "the dispatch's row stores alone (same rows, no loads; ordinary "
                            "and non-temporal stores), the "
                            "combine's row loads and output stores alone (same rows, XOR "
                            "instead of arithmetic), and the same with contiguous rows")
        del a, b, contig
        h.read_counts()
        if kernels:
            for name, ck in (("dispatch", "row_store_dispatch_rows"),
                             ("dispatch_streaming", "row_store_dispatch_rows_streaming"),
                             ("combine", "gather_combine_rows")):
                if name not in kernels:
                    continue
                cu = ceilings[ck]["us_median"]
                kernels[name]["ceiling"] = {"kernel": ck, "us": cu,
                                            "frac_of_ceiling": round(cu / kernels[name]["us_median"], 4)}

    # Graph replay: the step captured once in a HIP graph and replayed back
    # to back; the replayed output must equal the eager one bit for bit.
    graph = None
    if "graph" in phases and args.graph_steps > 0:
        step()
        torch.cuda.synchronize()
        out_eager = out.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg):
            step()
        cg.replay()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for _ in range(args.graph_steps):
            cg.replay()
        torch.cuda.synchronize()
        g_ms = (time.perf_counter() - t2) * 1e3 / args.graph_steps
        h.read_counts()
        if not torch.equal(out.view(torch.int16), out_eager.view(torch.int16)):
            raise RuntimeError("graph replay gave a different combine output")
        graph = {"steps": args.graph_steps, "ms_per_step": round(g_ms, 4),
                 "GBps": round(total_bytes / (g_ms * 1e-3) / 1e9, 1)}
        del cg

    T, K, H = cfg.tokens, cfg.topk, cfg.hidden
    # The 1 GiB read that evicts what a call leaves dirty, for the with-write-
    # back figures of the other calls.
    probe = (torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
             if {"backward", "rank", "quant"} & set(phases) else None)
    # Backward pair on the same layout.
    backward = None
    if "backward" in phases:
        g = W.payload_bf16(T, H, cfg.seed + 1, 3, "cuda")
        grad_y = torch.empty((cap, H), dtype=torch.bfloat16, device="cuda")
        gw_rows = torch.randn(cap, device="cuda")
        bb = {"combine_backward": T * 2 * H + V * 2 * H + V * 2 * H + 8 * T * K + 4 * T * K,
              "dispatch_backward": V * 2 * H + T * 2 * H + 4 * T * K + 8 * T * K + 4 * T * K}
        bcalls = {"combine_backward": lambda: h.combine_backward(
                      g, topk_weights=w, y=wl.y, grad_y=grad_y, want_grad_weights=True),
                  "dispatch_backward": lambda: h.dispatch_backward(
                      wl.y, grad_out_w=gw_rows, want_grad_weights=True)}
        backward = time_calls(torch, ep, ceil, bcalls, bb, args.reps, probe)
        del g, grad_y, gw_rows

    # Rank (non-expanded) layout and per-token biases, on the same layout.
    rank = None
    if "rank" in phases:
        nrecv = int(rc["num_recv_tokens"])
        R = H if cfg.fp8 else 2 * H
        S = 4 * (H // 128) if cfg.fp8 else 0
        rx = torch.empty((T, H), dtype=wl.x.dtype, device="cuda")
        rsf = torch.empty((T, H // 128), dtype=torch.float32, device="cuda") if cfg.fp8 else None
        ri = torch.empty((T, K), dtype=torch.int64, device="cuda")
        rw = torch.empty((T, K), dtype=torch.float32, device="cuda")
        xr = W.payload_bf16(T, H, cfg.seed + 2, 3, "cuda")
        b0 = W.payload_bf16(T, H, cfg.seed + 3, 3, "cuda")
        b1 = W.payload_bf16(T, H, cfg.seed + 4, 3, "cuda")
        rb = {"dispatch_rank": T * (R + S) + nrecv * (R + S) + T * K * 12 + nrecv * K * 12 + 4 * T,
              "combine_rank": nrecv * 2 * H + 3 * T * 2 * H + 4 * T,
              "combine_token_biases": nbytes["combine"] + 2 * T * 2 * H}
        rcalls = {"dispatch_rank": lambda: h.dispatch_rank(
                      wl.x, sf=wl.sf, topk_weights=w, out_x=rx, out_sf=rsf, out_topk_idx=ri,
                      out_topk_weights=rw),
                  "combine_rank": lambda: h.combine_rank(xr, bias_0=b0, bias_1=b1, out=out),
                  "combine_token_biases": lambda: h.combine(wl.y, topk_weights=w, bias=wl.bias,
                                                            out=out, bias_0=b0, bias_1=b1)}
        rank = time_calls(torch, ep, ceil, rcalls, rb, args.reps, probe)
        del rx, rsf, ri, rw, xr, b0, b1

    # FP8 quantiser on its own and fused with dispatch: bf16 rows of the
    # same workload, on the same layout, fp32 and packed UE8M0 scales.
    quant = None
    if "quant" in phases and H % 128 == 0:
        xq = W.payload_bf16(T, H, cfg.seed + 5, 3, "cuda")
        qx = torch.empty((cap, H), dtype=torch.uint8, device="cuda")
        qt = torch.empty((T, H), dtype=torch.uint8, device="cuda")
        P = {f: ep.ep_sf_packs(H, c) for f, c in (("f32", ep.EP_SF_F32),
                                                    ("ue8m0", ep.EP_SF_UE8M0))}
        sfs = {f: torch.empty((cap, P[f]), dtype=torch.float32 if f == "f32" else torch.int32,
                              device="cuda") for f in P}
        sft = {f: torch.empty((T, P[f]), dtype=torch.float32 if f == "f32" else torch.int32,
                              device="cuda") for f in P}
        nrq = int(rc["num_recv_tokens"])
        rqx = torch.empty((T, H), dtype=torch.uint8, device="cuda")
        rqsf = torch.empty((T, P["f32"]), dtype=torch.float32, device="cuda")
        rqi = torch.empty((T, K), dtype=torch.int64, device="cuda")
        rqw = torch.empty((T, K), dtype=torch.float32, device="cuda")
        qb = {"quantize_f32": T * 2 * H + T * H + 4 * T * P["f32"],
              "quantize_ue8m0": T * 2 * H + T * H + 4 * T * P["ue8m0"],
              "dispatch_quant_f32": T * 2 * H + V * (H + 4 * P["f32"]) + 4 * T * K,
              "dispatch_quant_ue8m0": T * 2 * H + V * (H + 4 * P["ue8m0"]) + 4 * T * K,
              "dispatch_rank_quant_f32": T * 2 * H + nrq * (H + 4 * P["f32"]) + 12 * T * K
                                         + 12 * nrq * K + 4 * T}
        qcalls = {"quantize_f32": lambda: ep.quantize_fp8(xq, "f32", out_q=qt, out_sf=sft["f32"]),
                  "quantize_ue8m0": lambda: ep.quantize_fp8(xq, "ue8m0", out_q=qt,
                                                            out_sf=sft["ue8m0"]),
                  "dispatch_quant_f32": lambda: h.dispatch_quant(xq, "f32", out_x=qx,
                                                                 out_sf=sfs["f32"]),
                  "dispatch_quant_ue8m0": lambda: h.dispatch_quant(xq, "ue8m0", out_x=qx,
                                                                   out_sf=sfs["ue8m0"]),
                  "dispatch_rank_quant_f32": lambda: h.dispatch_rank_quant(
                      xq, "f32", topk_weights=w, out_x=rqx, out_sf=rqsf, out_topk_idx=rqi,
                      out_topk_weights=rqw)}
        quant = time_calls(torch, ep, ceil, qcalls, qb, args.reps, probe)
        del xq, qx, qt, sfs, sft, rqx, rqsf, rqi, rqw
    del probe
    h.read_counts()

    # Roofline of dispatch and combine (combine is the dominant kernel: the
    # most bytes per step): algorithmic bytes over the cache-cold mean
    # duration (rocprofv3's average over the same launches, with
    # `--phases cold`, must agree), with the back-to-back figures beside.
    roofline = None
    if kernels:
        def roof(name):
            k = kernels[name]
            ach = nbytes[name] / (k["us_mean"] * 1e-6) / 1e9
            r = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
                 "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                 "traffic": k.get("traffic"), "kernel": name,
                 "bytes_per_launch": nbytes[name], "timing": "cache-cold mean",
                 "frac_median": k["frac_hbm_peak"]}
            if kernels_b2b:
                r["frac_back_to_back"] = kernels_b2b[name]["frac_hbm_peak"]
            if writeback and name in writeback:
                r["frac_with_writeback"] = writeback[name]["frac_hbm_peak"]
            if "ceiling" in k:
                r["frac_of_ceiling"] = k["ceiling"]["frac_of_ceiling"]
            return r
        roofline = roof("combine")
        roofline["per_kernel"] = {"dispatch": roof("dispatch"), "combine": roof("combine")}
        if "dispatch_streaming" in kernels:
            k = kernels["dispatch_streaming"]
            st = {"frac": round(k["mean_GBps"] / HBM_PEAK_GBPS, 4),
                  "frac_median": k["frac_hbm_peak"], "timing": "cache-cold mean"}
            if writeback and "dispatch_streaming" in writeback:
                st["frac_with_writeback"] = writeback["dispatch_streaming"]["frac_hbm_peak"]
            if "ceiling" in k:
                st["frac_of_ceiling"] = k["ceiling"]["frac_of_ceiling"]
            roofline["per_kernel"]["dispatch"]["streaming_stores"] = st

    cpu = None
    cpu_rows = None
    if not args.no_cpu_baseline:
        y_host = wl.y.view(torch.int16).cpu().numpy().view(np.uint16)
        wl_host = W.Workload(cfg, wl.topk_idx, wl.topk_weights, wl.x.cpu(),
                             None if wl.sf is None else wl.sf.cpu(), None, None)
        n_thr = cpu_threads()
        med1, reps1 = cpu_baseline(cfg, wl_host, y_host, args.cpu_seconds, 1)
        medn, repsn = cpu_baseline(cfg, wl_host, y_host, args.cpu_seconds, n_thr)
        cpu = {"value": round(total_bytes / medn / 1e9, 3), "unit": "GB/s", "cores": n_thr,
               "kind": "oracle",
               "sample": f"whole {cfg.name} batch ({cfg.tokens} tokens): layout (1 thread) + "
                         f"dispatch + combine (OpenMP over tokens, {n_thr} threads), {repsn} "
                         f"repetitions, median {medn:.3f} s per step",
               "ms_per_step": round(medn * 1e3, 1),
               "single_thread": {"value": round(total_bytes / med1 / 1e9, 3), "cores": 1,
                                 "ms_per_step": round(med1 * 1e3, 1), "repetitions": reps1},
               "cpu_model": cpu_model()}
        cpu_rows = cpu_oracle_rows(cfg, wl_host, args.cpu_row_tokens)

    value = (total_bytes / (ms_per_step * 1e-3) / 1e9) if ms_per_step else None
    head = kernels or kernels_b2b or {}
    dc_us = (head["dispatch"]["us_median"] + head["combine"]["us_median"]) if head else None
    line = {
        "metric": "dispatch+combine µs/call and HBM GB/s (% of peak) at 4096×7168 top-8",
        "value": round(value, 1) if value else None,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4) if ms_per_step else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.tokens} tokens x hidden {cfg.hidden}, "
                               f"{cfg.experts} experts, top-{cfg.topk}, "
                               f"{'FP8 e4m3 + fp32 scales' if cfg.fp8 else 'bf16'} dispatch, "
                               f"bf16 combine with fp32 weights, alignment {cfg.alignment}",
                   "tokens": cfg.tokens, "hidden": cfg.hidden, "experts": cfg.experts,
                   "topk": cfg.topk, "expert_alignment": cfg.alignment, "capacity": cap,
                   "zero_padding": cfg.zero_padding, "routed_slots": V, "gap_rows": G,
                   "seed": cfg.seed},
        "timing": {"value": "back-to-back steps, wall clock",
                   "kernels": "cache-cold: 1 GiB read before every call, outside its events; "
                              f"{args.calls} calls after 5 untimed; events on the call's kernels",
                   "kernels_back_to_back": "steps back to back, events on each call's kernels"},
        "dispatch_plus_combine_us": round(dc_us, 2) if dc_us else None,
        "dispatch_plus_combine_GBps": (round((nbytes["dispatch"] + nbytes["combine"]) /
                                             (dc_us * 1e-6) / 1e9, 1) if dc_us else None),
        "uncached_dispatch_us": (head["layout_dispatch"]["us_median"] if "layout_dispatch" in head
                                 else None),
        "layout_plus_dispatch_us": (round(head["layout"]["us_median"] +
                                          head["dispatch"]["us_median"], 2) if head else None),
        "kernels": kernels,
        "kernels_back_to_back": kernels_b2b,
        "writeback": writeback,
        "ceilings": ceilings,
        "graph_replay": graph,
        "backward": backward,
        "rank_and_token_bias": rank,
        "quantize": quant,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cpu_oracle_other_calls": cpu_rows,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
