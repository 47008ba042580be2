"""The library from plain C, with no torch and no Python in the path.

``tests/abi_client.c`` calls ep_handle_init, ep_layout, ep_dispatch,
ep_combine and ep_handle_read_counts through ``include/ep.h`` with its own
hipMalloc'd buffers and a non-blocking stream it creates.  On the CPU it is
built with gcc as a program and as a shared object against ``libep.so``
(every call it makes resolves) and its argument checks run.  On the GPU the
shared object's ``ep_client_run`` is called in-process (no child process is
started from the GPU-initialised test runner) on seeded inputs written to
files, and every output it writes is compared with the oracle, bit-exact:
layout (counts, psum, slot rows, source metadata), the zero-padded dispatch
with weights (untouched rows keep the client's 0xA5 fill) and the combine
with weights and an expert bias."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import bruteforce as BF

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "abi_client.c")
LIB_DIR = os.path.join(ROOT, "combine_ep_layout_08_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(out: str, shared: bool) -> str:
    if not os.path.exists(os.path.join(LIB_DIR, "libep.so")):
        pytest.skip("libep.so is not built")
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-o", out, "-L", LIB_DIR, "-l:libep.so", "-L", os.path.join(ROCM, "lib"),
           "-lamdhip64", "-Wl,-rpath," + LIB_DIR, "-Wl,--no-undefined"]
    if shared:
        cmd[1:1] = ["-shared", "-fPIC"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    return out


def test_c_client_builds_and_checks_its_arguments(tmp_path):
    exe = _build(str(tmp_path / "abi_client"), shared=False)
    _build(str(tmp_path / "libabi_client.so"), shared=True)
    usage = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert usage.returncode == 2 and "usage" in usage.stderr
    bad = subprocess.run([exe, str(tmp_path), "4", "0", "4", "1", "8"], capture_output=True,
                         text=True, timeout=60)
    assert bad.returncode == 2 and "bad sizes" in bad.stderr


def _bf16(rng, shape, scale=1.0):
    return BF.f32_to_bf16_bits_torch((rng.standard_normal(shape) * scale).astype(np.float32))


@pytest.mark.gpu
def test_c_client_matches_oracle(tmp_path):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X GPU")
    import combine_ep_layout_08_amd  # noqa: F401  (libep.so first, bound to torch's HIP runtime)
    so = _build(str(tmp_path / "libabi_client.so"), shared=True)
    T, K, E, A, H = 777, 6, 40, 16, 1032          # ragged rows: 129 vectors of 16 bytes
    rng = np.random.default_rng(2024)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    idx[rng.random((T, K)) < 0.2] = -1
    idx[5] = -1                                    # a token with no valid slot
    cap = oracle.capacity_bound(T, K, E, A)
    x = _bf16(rng, (T, H))
    w = rng.random((T, K), dtype=np.float32)
    y = _bf16(rng, (cap, H))
    bias = _bf16(rng, (E, H), 0.02)
    d = tmp_path / "io"
    d.mkdir()
    for name, arr in (("topk_idx", idx), ("x", x), ("w", w), ("y", y), ("bias", bias)):
        np.ascontiguousarray(arr).tofile(str(d / f"{name}.bin"))
    client = ctypes.CDLL(so)
    client.ep_client_run.restype = ctypes.c_int
    client.ep_client_run.argtypes = [ctypes.c_char_p] + [ctypes.c_int32] * 5
    print("[case] C client", T, K, E, A, H, flush=True)
    assert client.ep_client_run(str(d).encode(), T, K, E, A, H) == 0

    lay = oracle.layout(idx, E, A, cap)
    n = lay.num_expanded
    num_expanded, num_recv, bits, invalid = map(int, (d / "scalars.txt").read_text().split())
    assert (num_expanded, num_recv, bits, invalid) == (n, lay.num_recv_tokens, 0, 0)
    np.testing.assert_array_equal(np.fromfile(str(d / "counts.bin"), np.int32), lay.counts)
    np.testing.assert_array_equal(np.fromfile(str(d / "psum.bin"), np.int32), lay.psum)
    np.testing.assert_array_equal(np.fromfile(str(d / "dst.bin"), np.int32),
                                  lay.dst.reshape(-1))
    np.testing.assert_array_equal(np.fromfile(str(d / "src_meta.bin"), np.int32),
                                  lay.src_meta[:n])
    o_x = np.full((cap, 2 * H), 0xA5, np.uint8)
    o_w = np.full(cap, np.frombuffer(bytes([0xA5] * 4), np.float32)[0], np.float32)
    oracle.dispatch(x.view(np.uint8).reshape(T, 2 * H), lay, cap, weights=w, zero_padding=True,
                    out_x=o_x, out_w=o_w)
    np.testing.assert_array_equal(np.fromfile(str(d / "out_x.bin"), np.uint8).reshape(cap, -1),
                                  o_x)
    np.testing.assert_array_equal(np.fromfile(str(d / "out_w.bin"), np.uint32),
                                  o_w.view(np.uint32))
    exp = oracle.combine(y, idx, lay.dst, w, bias)
    np.testing.assert_array_equal(np.fromfile(str(d / "out.bin"), np.uint16).reshape(T, H), exp)
