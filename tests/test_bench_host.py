"""Host-side logic of bench.py (CPU only): the algorithmic byte counts the
roofline divides by, the staleness rule for the committed HBM counters, the
one-GPU guard, the phase selection, and that the profiler commands it records
are ones bench.py accepts."""
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


def _write_counters(path, records):
    with open(path, "w") as f:
        json.dump({"workloads": records, "commands": {}}, f)


def test_traffic_only_for_current_source(tmp_path, monkeypatch):
    """roofline.traffic comes from the committed counters only while the
    kernel's sources (its file, the shared header and the C ABI that picks
    its launch) hash to the value recorded with them; otherwise it is null
    and flagged stale."""
    path = tmp_path / "hbm_counters.json"
    cur = {k: bench.kernel_source_hash(k) for k in bench.KERNEL_SOURCES}
    _write_counters(path, {"prefill": {
        "combine": {"hbm_bytes_per_launch": 123, "source_sha256_16": cur["combine"]},
        "dispatch": {"hbm_bytes_per_launch": 456, "source_sha256_16": "0" * 16}}})
    monkeypatch.setattr(bench, "PROFILE_COUNTERS", str(path))
    assert bench.measured_traffic("combine", "prefill") == (123, False)
    assert bench.measured_traffic("dispatch", "prefill") == (None, True)
    assert bench.measured_traffic("combine", "decode") == (None, False)
    # an edit to a combine-only source makes combine's counters stale and
    # leaves dispatch's hash as it was; an edit to the C ABI touches both
    orig = bench.CSRC
    for edited, hit, kept in (("ep_combine.hip", "combine", "dispatch"),
                              ("ep_api.cpp", "dispatch", None)):
        csrc = tmp_path / f"csrc_{edited}"
        shutil.copytree(orig, csrc)
        with open(csrc / edited, "a") as f:
            f.write("\n// edited\n")
        monkeypatch.setattr(bench, "CSRC", str(csrc))
        assert bench.kernel_source_hash(hit) != cur[hit]
        if kept:
            assert bench.kernel_source_hash(kept) == cur[kept]
        else:
            assert bench.kernel_source_hash("combine") != cur["combine"]
        monkeypatch.setattr(bench, "CSRC", orig)


def test_committed_counters_near_algorithmic_bytes():
    """Every committed counter record of a call that moves at least 100 MB
    lies within 2 % of its algorithmic bytes (no row crosses HBM twice),
    allowing the dispatch one extra read of its token's scale packs per
    routed row (the packs are copied in expanded-row order, each row reading
    its source token's packs)."""
    if not os.path.exists(bench.PROFILE_COUNTERS):
        pytest.skip("no committed counters")
    with open(bench.PROFILE_COUNTERS) as f:
        data = json.load(f)
    n = 0
    for wl, kernels in data["workloads"].items():
        cfg = W.config(wl)
        idx, _ = W.routing(cfg)
        V = int((idx >= 0).sum())
        S = 4 * (cfg.hidden // 128) if cfg.fp8 else 0
        for name, rec in kernels.items():
            alg = rec.get("algorithmic_bytes")
            if not alg or alg < 100e6:
                continue
            extra = V * S if name == "dispatch" else 0
            got = rec["hbm_bytes_per_launch"]
            assert 0.98 * alg <= got <= 1.02 * (alg + extra), (wl, name, got / alg)
            n += 1
    assert n >= 8


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_recorded_profiler_commands_parse():
    """Every command recorded beside the counters runs bench.py with flags it
    accepts (so the summaries can be regenerated from committed files)."""
    if not os.path.exists(bench.PROFILE_COUNTERS):
        pytest.skip("no committed counters")
    with open(bench.PROFILE_COUNTERS) as f:
        commands = json.load(f)["commands"]
    assert commands
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


def test_phases_are_checked():
    assert bench.parse(["--phases", "cold,steps"]).phases == ["cold", "steps"]
    with pytest.raises(SystemExit):
        bench.parse(["--phases", "cold,nonsense"])


@pytest.mark.parametrize("name", sorted(W.CONFIGS) + sorted(W.BENCH_CONFIGS))
def test_every_workload_has_byte_counts(name):
    cfg = W.config(name)
    b = bench.algorithmic_bytes(cfg, V=cfg.tokens * cfg.topk, G=0,
                                expanded=cfg.tokens * cfg.topk)
    assert all(v > 0 for v in b.values())
