"""Host-side logic of bench.py (CPU only): the algorithmic byte counts the
roofline divides by, the staleness rule for the committed HBM counters, the
one-GPU guard, and that the profiler commands it records are ones bench.py
accepts."""
from __future__ import annotations

import json
import os
import shlex
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import ep_workloads as W  # noqa: E402


def test_prefill_bytes_closed_form():
    """Prefill: 4096 tokens of 7168 FP8 bytes + 56 fp32 scales, top-8, every
    slot routed (V = 32768), no zero padding.  Dispatch reads each token row
    and its scales once, writes them once per slot and reads the slot index;
    combine reads each routed bf16 row once, writes each token row once and
    reads the slot index and the weights."""
    cfg = W.CONFIGS["prefill"]
    b = bench.algorithmic_bytes(cfg, V=32768, G=14976, expanded=47744)
    row = 7168 + 56 * 4
    assert b["dispatch"] == 4096 * row + 32768 * row + 4 * 32768 == 272_629_760
    assert b["combine"] == 32768 * 14336 + 4096 * 14336 + 8 * 32768 == 528_744_448
    # ids (int64) read, slot rows written, source metadata of every expanded
    # row, counts and psum
    assert b["layout"] == 8 * 32768 + 4 * 32768 + 4 * 47744 + 4 * (2 * 256 + 1)


def test_zero_padding_and_bias_terms():
    """Zero padding adds the gap rows' bytes to dispatch; an expert bias adds
    the bias table once and the ids combine reads to find each slot's expert."""
    cfg = W.CONFIGS["skewed"]          # bf16 rows of 4096, zero padding, bias
    V, G = 131072, 4160
    b = bench.algorithmic_bytes(cfg, V=V, G=G, expanded=V + G)
    row = 2 * 4096
    assert b["dispatch"] == 16384 * row + V * row + 4 * 16384 * 8 + G * row
    assert b["combine"] == (V * row + 16384 * row + 8 * 16384 * 8
                            + 2 * 128 * 4096 + 8 * 16384 * 8)


def test_traffic_only_for_current_source(tmp_path, monkeypatch):
    """roofline.traffic comes from the committed counters only while the
    kernel's source hash equals the one recorded with them."""
    with open(bench.PROFILE_COUNTERS) as f:
        counters = json.load(f)["kernels"]
    for kernel in bench.KERNEL_SOURCES:
        rec = counters[kernel]
        current = rec["source_sha256_16"] == bench.kernel_source_hash(kernel)
        want = rec["hbm_bytes_per_launch"] if current else None
        assert bench.measured_traffic(kernel) == want
        # within 2 % of the algorithmic bytes: no row crosses HBM twice
        assert abs(rec["hbm_bytes_per_launch"] / rec["algorithmic_bytes"] - 1) < 0.02
    # an edit to a combine-only source makes combine's counters stale and
    # leaves dispatch's as they were
    edited = bench.KERNEL_SOURCES["combine"][0]
    assert edited not in bench.KERNEL_SOURCES["dispatch"]
    csrc = tmp_path / "csrc"
    shutil.copytree(bench.CSRC, csrc)
    with open(csrc / edited, "a") as f:
        f.write("\n// edited\n")
    dispatch_before = bench.measured_traffic("dispatch")
    monkeypatch.setattr(bench, "CSRC", str(csrc))
    assert bench.measured_traffic("combine") is None
    assert bench.measured_traffic("dispatch") == dispatch_before


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_recorded_profiler_commands_parse():
    """Every command recorded beside the counters runs bench.py with flags it
    accepts (so the summaries can be regenerated from committed files)."""
    with open(bench.PROFILE_COUNTERS) as f:
        commands = json.load(f)["commands"]
    for cmd in commands.values():
        argv = shlex.split(cmd)
        assert argv[0] == "rocprofv3"
        prog = argv[argv.index("--") + 1:]
        assert prog[:3] == ["python", "-u", "bench.py"]
        monkey_argv = ["bench.py", *prog[3:]]
        old = sys.argv
        try:
            sys.argv = monkey_argv
            args = bench.parse()
        finally:
            sys.argv = old
        assert args.gpus == 1


@pytest.mark.parametrize("name", sorted(W.CONFIGS))
def test_every_workload_has_byte_counts(name):
    cfg = W.CONFIGS[name]
    b = bench.algorithmic_bytes(cfg, V=cfg.tokens * cfg.topk, G=0,
                                expanded=cfg.tokens * cfg.topk)
    assert all(v > 0 for v in b.values())
