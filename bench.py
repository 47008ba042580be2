"""Benchmark: MoE routing layout + dispatch + combine on one MI355X.

One step is one pass of the whole hot path over one batch: ep_layout on
topk_idx, ep_dispatch of the FP8 token rows (+ fp32 scales) into the
expert-expanded layout, ep_combine of bf16 expert outputs back to token order
with fp32 weights.  Default workload: prefill, 4096 tokens x hidden 7168,
256 experts in 8 groups (group-limited top-4 groups, top-8 experts),
expert_alignment 128, buffers sized at the worst-case bound (65280 rows).
Inputs are seeded synthetic data, resident in HBM before timing starts.

Prints one JSON line.  ``value`` is whole-step algorithmic HBM throughput
(GB/s); per-kernel microseconds, GB/s and fractions of the 8 TB/s HBM peak
are reported beside it, with the roofline of the dominant kernel (combine)
and the CPU oracle's throughput on the host as a baseline.  Per-call times
come from HIP events that the library attaches to the calls' own kernel
dispatches (ep_time_next_call), on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, AMD published peak
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "prefill_hbm_counters.json")
CSRC = os.path.join(ROOT, "combine_ep_layout_08_amd", "csrc")
KERNEL_SOURCES = {"combine": ["ep_combine.hip", "ep_internal.h"],
                  "dispatch": ["ep_dispatch.hip", "ep_internal.h"]}


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="prefill", help="workload name (default prefill)")
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the oracle timing (for profiler runs)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum oracle time for the CPU baseline")
    p.add_argument("--cold-reps", type=int, default=30,
                   help="calls per kernel in the cold-cache phase after the timed steps (0 = skip)")
    p.add_argument("--backward-reps", type=int, default=30,
                   help="calls of each backward entry point after the timed steps (0 = skip)")
    p.add_argument("--rank-reps", type=int, default=30,
                   help="calls of the rank-layout and per-token-bias entry points (0 = skip)")
    p.add_argument("--cpu-row-tokens", type=int, default=512,
                   help="tokens of the CPU-oracle sample for the calls beyond the step")
    p.add_argument("--quant-reps", type=int, default=30,
                   help="calls timed for the FP8 quantiser phase (0 skips it)")
    p.add_argument("--graph-steps", type=int, default=200,
                   help="replays of one step captured in a HIP graph, timed after the "
                        "eager steps (0 = skip)")
    p.add_argument("--flush", action="store_true",
                   help="read a 1 GiB scratch buffer before every call (outside the per-call "
                        "events) so each kernel starts with cold L2 and MALL")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (profiler calibration)")
    return p.parse_args()


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


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counters
    (FETCH_SIZE + WRITE_SIZE, calibrated on a plain copy), if they were taken
    on the kernel's current source; else None."""
    if not os.path.exists(PROFILE_COUNTERS):
        return None
    with open(PROFILE_COUNTERS) as f:
        k = json.load(f).get("kernels", {}).get(kernel)
    if not k or k.get("source_sha256_16") != kernel_source_hash(kernel):
        return None
    return k.get("hbm_bytes_per_launch")


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


def ceilings(torch, nbytes=1 << 30, reps=5):
    """Measured device ceilings: 1 GiB device-to-device copy and fill (torch
    kernels)."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(3)
    b.copy_(a)
    torch.cuda.synchronize()
    out = {}
    for name, fn, moved in (("copy", lambda: b.copy_(a), 2 * nbytes),
                            ("fill", lambda: b.fill_(7), nbytes)):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        out[name + "_GBps"] = round(moved / ms / 1e6, 1)
    del a, b
    return out


def cpu_baseline(cfg, wl, y_host, min_seconds: float):
    """Time the CPU oracle (single thread, as it stands) on the same workload:
    full layout + dispatch + combine of the whole batch, repeated until
    ``min_seconds`` have passed; median step time."""
    import numpy as np
    import oracle
    import torch
    cap = oracle.capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment)
    x_bytes = wl.x.contiguous().view(torch.uint8).cpu().numpy()
    sf = wl.sf.cpu().numpy() if wl.sf is not None else None
    out_x = np.empty((cap, x_bytes.shape[1]), np.uint8)
    out_sf = np.empty((cap, sf.shape[1]), np.float32) if sf is not None else None
    times = []
    lay = None
    t_end = time.perf_counter() + min_seconds
    while True:
        t0 = time.perf_counter()
        lay = oracle.layout(wl.topk_idx, cfg.experts, cfg.alignment, cap)
        oracle.dispatch(x_bytes, lay, cap, sf=sf, zero_padding=cfg.zero_padding,
                        out_x=out_x, out_sf=out_sf)
        oracle.combine(y_host, wl.topk_idx, lay.dst, wl.topk_weights)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() >= t_end and len(times) >= 1:
            break
    return statistics.median(times), len(times), lay


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
    import torch
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


def time_calls(calls, nbytes, reps, flush=None):
    """Each call once untimed, then `reps` calls whose kernel intervals are
    stamped by ep_time_next_call; mean µs, GB/s of the algorithmic bytes.
    With `flush` (a 1 GiB device tensor), `reps` more calls each run right
    after a full read of it (outside the stamped interval), so inputs that
    would fit the 256 MB MALL between repeated calls come from HBM: the
    cold_* figures."""
    import torch
    import combine_ep_layout_08_amd as ep

    def run(fn, cold):
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(reps)]
        for e0, e1 in pairs:
            e0.record()
            e1.record()
        for e0, e1 in pairs:
            if cold:
                flush.sum()
            ep.time_next_call(e0, e1)
            fn()
        torch.cuda.synchronize()
        return statistics.mean(e0.elapsed_time(e1) * 1e3 for e0, e1 in pairs)

    out = {}
    for name, fn in calls.items():
        fn()
        us = run(fn, False)
        gbps = nbytes[name] / (us * 1e-6) / 1e9
        out[name] = {"us_mean": round(us, 2), "bytes": nbytes[name], "GBps": round(gbps, 1),
                     "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
        if flush is not None:
            cus = run(fn, True)
            cg = nbytes[name] / (cus * 1e-6) / 1e9
            out[name].update({"cold_us_mean": round(cus, 2), "cold_GBps": round(cg, 1),
                              "cold_frac_hbm_peak": round(cg / HBM_PEAK_GBPS, 4)})
    return out


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

    cfg = W.CONFIGS[args.config]
    cap = ep.ep_capacity_bound(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment)
    wl = W.make(cfg, device="cuda", y_rows=cap)
    idx = torch.from_numpy(wl.topk_idx).cuda()
    w = torch.from_numpy(wl.topk_weights).cuda()
    h = ep.Handle(cfg.tokens, cfg.topk, cfg.experts, cfg.alignment, cap)
    out_x = torch.empty((cap, cfg.hidden), dtype=wl.x.dtype, device="cuda")
    out_sf = (torch.empty((cap, cfg.hidden // 128), dtype=torch.float32, device="cuda")
              if cfg.fp8 else None)
    out = torch.empty((cfg.tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda")

    # Cache flush by reading 1 GiB (four times the 256 MB MALL): the caches
    # end up full of clean lines, so the next kernel pays no write-back.
    scratch = (torch.ones(1 << 28, dtype=torch.int32, device="cuda") if args.flush else None)

    def flush():
        if scratch is not None:
            scratch.sum()

    # The step's three calls, validated and marshalled once (bound calls:
    # the same entry points and kernels, about 3 us of host time per call
    # instead of 5-6, so small batches are not bound by the Python side).
    h.layout(idx)
    layout_call = h.bind_layout(idx)
    dispatch_call = h.bind_dispatch(wl.x, sf=wl.sf, zero_padding=cfg.zero_padding,
                                    out_x=out_x, out_sf=out_sf)
    combine_call = h.bind_combine(wl.y, topk_weights=w, bias=wl.bias, out=out)

    def step(ev=None):
        # ev: six events; each pair is stamped on the kernels of one call.
        flush()
        if ev is not None:
            ep.time_next_call(ev[0], ev[1])
        layout_call()
        flush()
        if ev is not None:
            ep.time_next_call(ev[2], ev[3])
        dispatch_call()
        flush()
        if ev is not None:
            ep.time_next_call(ev[4], ev[5])
        combine_call()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    rc = h.read_counts()                        # raises on any device error
    V = int((wl.topk_idx >= 0).sum())
    G = int(rc["num_expanded"]) - V
    nbytes = algorithmic_bytes(cfg, V, G, int(rc["num_expanded"]))

    # Timed region: exactly `steps` steps, synchronised on both sides, with
    # nothing but the calls themselves on the stream.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # Kernel durations: `steps` more steps, each call's kernels stamped by
    # events attached to their dispatches (ep_time_next_call).  The stamps
    # cost GPU time of their own (measured ≈ 5 µs per call), so they stay out
    # of the timed region above; the events are created (first record)
    # before this region starts.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for e6 in evs:
        for e in e6:
            e.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms_per_step_stamped = (time.perf_counter() - t1) * 1e3 / args.steps
    per = {"layout": [], "dispatch": [], "combine": []}
    for e in evs:
        per["layout"].append(e[0].elapsed_time(e[1]) * 1e3)
        per["dispatch"].append(e[2].elapsed_time(e[3]) * 1e3)
        per["combine"].append(e[4].elapsed_time(e[5]) * 1e3)
    step_gpu_ms = sum(e[0].elapsed_time(e[5]) for e in evs) / args.steps
    kernels = {}
    for k, v in per.items():
        us = statistics.mean(v)
        gbps = nbytes[k] / (us * 1e-6) / 1e9
        kernels[k] = {"us_mean": round(us, 2), "us_median": round(statistics.median(v), 2),
                      "us_p10": round(float(np.percentile(v, 10)), 2),
                      "us_p90": round(float(np.percentile(v, 90)), 2),
                      "bytes": nbytes[k], "GBps": round(gbps, 1),
                      "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
        if k in KERNEL_SOURCES:
            kernels[k]["traffic"] = measured_traffic(k)
    # Graph replay (after the timed region): the step's three calls captured
    # once in a HIP graph (torch.cuda.CUDAGraph; the library launches on the
    # capturing stream and allocates nothing) and replayed back to back, so
    # the host's per-call launch cost drops out; the replayed output must equal
    # the eager one bit for bit.
    graph = None
    if args.graph_steps > 0 and not args.flush:
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
        h.read_counts()                         # raises on any device error
        if not torch.equal(out.view(torch.int16), out_eager.view(torch.int16)):
            raise RuntimeError("graph replay gave a different combine output")
        graph = {"steps": args.graph_steps, "ms_per_step": round(g_ms, 4),
                 "GBps": round(sum(nbytes.values()) / (g_ms * 1e-3) / 1e9, 1)}
        del cg

    # Cold-cache phase (after the timed region): each call runs right after a
    # 1 GiB read that leaves L2 and the MALL full of unrelated clean lines, so
    # its inputs come from HBM; timed by the events on its own kernels.
    kernels_cold = None
    big = None
    if args.cold_reps > 0:
        big = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
        calls = {"layout": lambda: h.layout(idx),
                 "dispatch": lambda: h.dispatch(wl.x, sf=wl.sf, zero_padding=cfg.zero_padding,
                                                out_x=out_x, out_sf=out_sf),
                 "combine": lambda: h.combine(wl.y, topk_weights=w, bias=wl.bias, out=out)}
        kernels_cold = {}
        for name, fn in calls.items():
            pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                     for _ in range(args.cold_reps)]
            for e0, e1 in pairs:
                e0.record()
                e1.record()
            for e0, e1 in pairs:
                big.sum()
                ep.time_next_call(e0, e1)
                fn()
            torch.cuda.synchronize()
            us = statistics.mean(e0.elapsed_time(e1) * 1e3 for e0, e1 in pairs)
            gbps = nbytes[name] / (us * 1e-6) / 1e9
            kernels_cold[name] = {"us_mean": round(us, 2), "GBps": round(gbps, 1),
                                  "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}

    # Backward pair on the same layout (a separate phase after the timed
    # steps): combine backward with row and weight gradients, dispatch
    # backward with the row combine and the weight gather.
    backward = None
    if args.backward_reps > 0:
        T, K, H = cfg.tokens, cfg.topk, cfg.hidden
        g = W.payload_bf16(T, H, cfg.seed + 1, 3, "cuda")
        grad_y = torch.empty((cap, H), dtype=torch.bfloat16, device="cuda")
        gw_rows = torch.randn(cap, device="cuda")
        bb = {"combine_backward": T * 2 * H + V * 2 * H + V * 2 * H + 8 * T * K + 4 * T * K,
              "dispatch_backward": V * 2 * H + T * 2 * H + 4 * T * K + 8 * T * K + 4 * T * K}
        bcalls = {"combine_backward": lambda: h.combine_backward(
                      g, topk_weights=w, y=wl.y, grad_y=grad_y, want_grad_weights=True),
                  "dispatch_backward": lambda: h.dispatch_backward(
                      wl.y, grad_out_w=gw_rows, want_grad_weights=True)}
        backward = time_calls(bcalls, bb, args.backward_reps, big)

    # Rank (non-expanded) layout and per-token biases, on the same layout.
    rank = None
    if args.rank_reps > 0:
        T, K, H = cfg.tokens, cfg.topk, cfg.hidden
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
        rank = time_calls(rcalls, rb, args.rank_reps, big)
        del rx, rsf, ri, rw, xr, b0, b1

    # FP8 quantiser on its own and fused with dispatch: bf16 rows of the
    # same workload, on the same layout, fp32 and packed UE8M0 scales.
    quant = None
    if args.quant_reps > 0 and cfg.hidden % 128 == 0:
        T, K, H = cfg.tokens, cfg.topk, cfg.hidden
        xq = W.payload_bf16(T, H, cfg.seed + 5, 3, "cuda")
        qx = torch.empty((cap, H), dtype=torch.uint8, device="cuda")
        qt = torch.empty((T, H), dtype=torch.uint8, device="cuda")
        sfs = {f: torch.empty((cap, ep.ep_sf_packs(H, c)),
                              dtype=torch.float32 if f == "f32" else torch.int32, device="cuda")
               for f, c in (("f32", ep.EP_SF_F32), ("ue8m0", ep.EP_SF_UE8M0))}
        P = {f: ep.ep_sf_packs(H, c) for f, c in (("f32", ep.EP_SF_F32),
                                                    ("ue8m0", ep.EP_SF_UE8M0))}
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
        quant = time_calls(qcalls, qb, args.quant_reps, big)
        del xq, qx, qt, sfs, sft, rqx, rqsf, rqi, rqw
    del big

    total_bytes = sum(nbytes.values())
    if args.flush:
        # The wall time also holds the cache flushes; use the calls' own time.
        ms_per_step = sum(kernels[k]["us_mean"] for k in kernels) / 1e3
    value = total_bytes / (ms_per_step * 1e-3) / 1e9
    dc_us = kernels["dispatch"]["us_mean"] + kernels["combine"]["us_mean"]
    comb = kernels["combine"]
    roofline = {"bound": "hbm", "achieved": comb["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(comb["GBps"] / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic("combine"), "kernel": "combine",
                "bytes_per_launch": nbytes["combine"]}
    if kernels_cold:
        roofline["achieved_cold_cache"] = kernels_cold["combine"]["GBps"]
        roofline["frac_cold_cache"] = kernels_cold["combine"]["frac_hbm_peak"]
    ceil = ceilings(torch)

    cpu = None
    cpu_rows = None
    if not args.no_cpu_baseline:
        y_host = wl.y.view(torch.int16).cpu().numpy().view(np.uint16)
        wl_host = W.Workload(cfg, wl.topk_idx, wl.topk_weights, wl.x.cpu(),
                             None if wl.sf is None else wl.sf.cpu(), None, None)
        med, reps, _ = cpu_baseline(cfg, wl_host, y_host, args.cpu_seconds)
        cpu = {"value": round(total_bytes / med / 1e9, 3), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"whole {cfg.name} batch ({cfg.tokens} tokens): layout + dispatch + "
                         f"combine, {reps} repetitions, median {med:.3f} s per step, "
                         "single-threaded C oracle",
               "ms_per_step": round(med * 1e3, 1)}
        cpu_rows = cpu_oracle_rows(cfg, wl_host, args.cpu_row_tokens)

    line = {
        "metric": "dispatch+combine µs/call and HBM GB/s (% of peak) at 4096×7168 top-8",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
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
        "dispatch_plus_combine_us": round(dc_us, 2),
        "dispatch_plus_combine_GBps": round((nbytes["dispatch"] + nbytes["combine"]) /
                                            (dc_us * 1e-6) / 1e9, 1),
        "step_gpu_ms_stamped": round(step_gpu_ms, 4),
        "ms_per_step_stamped": round(ms_per_step_stamped, 4),
        "graph_replay": graph,
        "cache_flush_between_calls": bool(args.flush),
        "kernels": kernels,
        "kernels_cold_cache": kernels_cold,
        "backward": backward,
        "rank_and_token_bias": rank,
        "quantize": quant,
        "roofline": roofline,
        "ceilings": ceil,
        "cpu_baseline": cpu,
        "cpu_oracle_other_calls": cpu_rows,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
