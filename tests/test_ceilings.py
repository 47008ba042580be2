"""The benchmark's bandwidth-ceiling kernels (libep_ceilings.so): every
function include/ep_ceilings.h declares is exported and refuses invalid
arguments before any launch (CPU), and on the GPU each kernel moves exactly
the bytes it claims (the read's fold, the write's value, the copy, the
dispatch-pattern row stores and the combine-pattern gather)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep_ceilings.h")


@pytest.fixture(scope="module")
def ceil():
    import bench
    if not os.path.exists(bench.CEILINGS_LIB):
        from combine_ep_layout_08_amd import build
        build.build_ceilings()
    return ctypes.CDLL(bench.CEILINGS_LIB)


def declared():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(epc_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported(ceil):
    names = declared()
    assert names == ["epc_copy", "epc_empty", "epc_gather", "epc_read", "epc_read_sink_words",
                     "epc_row_store", "epc_write"]
    for n in names:
        assert hasattr(ceil, n), n


def test_invalid_arguments_launch_nothing(ceil):
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    ceil.epc_read.argtypes = [P, SZ, P, I32, I32, I32, P, P, P]
    ceil.epc_write.argtypes = [P, SZ, ctypes.c_uint32, I32, I32, I32, P, P, P]
    ceil.epc_copy.argtypes = [P, P, SZ, I32, I32, I32, P, P, P]
    ceil.epc_row_store.argtypes = [P, I64, I64, P, I64, I32, I32, P, P, P]
    ceil.epc_gather.argtypes = [P, P, I64, I64, P, I64, I32, P, P, P]
    ceil.epc_read_sink_words.restype = I64
    ceil.epc_read_sink_words.argtypes = [SZ, I32, I32]
    ceil.epc_empty.argtypes = [I32, I32, P, P, P]
    assert ceil.epc_empty(0, 64, None, None, None) == -1
    assert ceil.epc_empty(1, 2048, None, None, None) == -1
    A = 0x300000
    assert ceil.epc_read(A, 17, A, 4, 0, 0, None, None, None) == -1     # not a multiple of 16
    assert ceil.epc_read(A + 4, 32, A, 4, 0, 0, None, None, None) == -1  # misaligned
    assert ceil.epc_read(A, 32, A, 3, 0, 0, None, None, None) == -1     # vectors per thread
    assert ceil.epc_read(A, 32, A, 4, -1, 0, None, None, None) == -1    # grid
    assert ceil.epc_read(A, 0, A, 4, 0, 0, None, None, None) == 0       # nothing to do
    assert ceil.epc_write(None, 32, 0, 4, 0, 0, None, None, None) == -1
    assert ceil.epc_copy(A, A + 8, 32, 4, 0, 0, None, None, None) == -1
    assert ceil.epc_row_store(A, 10, 100, A, 4, 8, 0, None, None, None) == -1   # row bytes % 16
    assert ceil.epc_row_store(A, 10, 128, A, 4, 0, 1, None, None, None) == -1   # K < 1
    assert ceil.epc_row_store(A, 10, 128, A, 4, 65, 0, None, None, None) == -1  # K > 64
    assert ceil.epc_gather(A, A, 10, 128, None, 4, 8, None, None, None) == -1
    assert ceil.epc_gather(A, A, -1, 128, A, 4, 8, None, None, None) == -1
    # a block covers 4096 * vec_per_thread bytes per round; one word per wave
    assert ceil.epc_read_sink_words(1 << 30, 16, 0) == (1 << 30) // 65536 * 4
    assert ceil.epc_read_sink_words(1 << 30, 4, 2048) == 2048 * 4
    assert ceil.epc_read_sink_words(16, 1, 0) == 4
    assert ceil.epc_read_sink_words(16, 5, 0) == -1


@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")
def test_ceiling_kernels_move_what_they_claim():
    import bench
    c = bench.Ceilings(torch)
    n = (3 << 20) + 48                              # not a whole number of blocks
    src = torch.randint(0, 2**31 - 1, (n // 4,), dtype=torch.int32, device="cuda")
    want = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
    for tune in [(1, 0, 0), (4, 0, 0), (16, 0, 1), (4, 7, 0), (8, 300, 1)]:
        c.sink.zero_()
        c.read(src, tune=tune)
        torch.cuda.synchronize()
        words = int(c.lib.epc_read_sink_words(n, tune[0], tune[1]))
        got = np.bitwise_xor.reduce(c.sink[:words].cpu().numpy().view(np.uint32))
        assert got == want, tune
        dst = torch.zeros_like(src)
        c.write(dst, n - 16, tune=tune)
        torch.cuda.synchronize()
        assert (dst[:-4] == 7).all() and (dst[-4:] == 0).all(), tune
        c.copy(dst, src, n, tune=tune)
        torch.cuda.synchronize()
        assert torch.equal(dst, src), tune
    # dispatch-pattern row stores: 5 tokens, K 3, rows of 2064 bytes (ragged
    # last pass); -1 and out-of-range rows skipped
    T, K, rows, rb = 5, 3, 12, 2064
    slot_row = torch.tensor([0, 4, -1, 7, 1, 11, 12, 2, 3, -1, -1, 5, 6, 9, 8], dtype=torch.int32,
                            device="cuda")
    for nt in (False, True):
        out = torch.full((rows, rb // 4), -5, dtype=torch.int32, device="cuda")
        c.row_store(out, rows, rb, slot_row, T, K, nontemporal=nt)
        torch.cuda.synchronize()
        o = out.cpu().numpy().reshape(rows, rb // 16, 4)
        for t in range(T):
            for k in range(K):
                r = int(slot_row[t * K + k])
                if 0 <= r < rows:
                    assert (o[r] == np.array([t, 1, 2, 3])).all()
        assert (o[10] == -5).all()                  # no slot maps to row 10
    # combine-pattern gather: out[t] = XOR of its slot rows
    inp = torch.randint(0, 2**31 - 1, (rows, rb // 4), dtype=torch.int32, device="cuda")
    g = torch.empty((T, rb // 4), dtype=torch.int32, device="cuda")
    c.gather(g, inp, rows, rb, slot_row, T, K)
    torch.cuda.synchronize()
    x = inp.cpu().numpy()
    for t in range(T):
        want = np.zeros(rb // 4, np.int32)
        for k in range(K):
            r = int(slot_row[t * K + k])
            if 0 <= r < rows:
                want ^= x[r]
        assert (g[t].cpu().numpy() == want).all()
