"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
(via the binding) and bring results to the host in the oracle's formats."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import combine_ep_layout_08_amd as ep
import oracle

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")

POISON = 0xA5


def say(*msg):
    """Name the case before a GPU step (unbuffered, so it survives a crash)."""
    print("[case]", *msg, file=sys.stderr, flush=True)


def u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.uint8).cpu().numpy()


def poison_(t: torch.Tensor) -> torch.Tensor:
    t.view(torch.uint8).fill_(POISON)
    return t


def gpu_layout(idx: np.ndarray, E: int, A: int, capacity: int, idx_dtype=torch.int64,
               max_tokens=None, handle=None):
    """Layout on the GPU.  Returns (handle, read_counts dict, dst, src_meta)."""
    T, K = idx.shape
    t_idx = torch.from_numpy(np.ascontiguousarray(idx)).to(idx_dtype).cuda()
    h = handle or ep.Handle(max_tokens if max_tokens is not None else T, K, E, A, capacity)
    h.layout(t_idx)
    rc = h.read_counts(check=False)
    dst = h.dst_slot.cpu().numpy().copy()
    src = h.src_meta.cpu().numpy().copy()
    rc["recv_row"] = h.recv_row.cpu().numpy().copy()
    rc["recv_src"] = h.recv_src.cpu().numpy().copy()[:max(rc["num_recv_tokens"], 0)]
    return h, rc, dst, src


def assert_rank_equal(rc, idx, E):
    """Rank-layout rows of the GPU layout against the oracle's."""
    row, src, n = oracle.rank_layout(idx, E)
    np.testing.assert_array_equal(rc["recv_row"], row)
    np.testing.assert_array_equal(rc["recv_src"], src)
    assert rc["num_recv_tokens"] == n


def assert_layout_equal(rc, dst, src, lay: oracle.Layout):
    """Bit-exact comparison of everything the layout defines."""
    assert rc["num_expanded"] == lay.num_expanded
    assert rc["invalid_count"] == lay.invalid_count
    if lay.status == oracle.ERR_CAPACITY:
        assert rc["status"] == ep.EP_ERR_CAPACITY
        assert rc["error_bits"] & ep.EP_ERRBIT_CAPACITY
        np.testing.assert_array_equal(rc["counts"], lay.counts)
        return
    assert lay.status == 0
    np.testing.assert_array_equal(rc["counts"], lay.counts)
    np.testing.assert_array_equal(rc["psum"], lay.psum)
    np.testing.assert_array_equal(dst, lay.dst)
    n = lay.num_expanded
    np.testing.assert_array_equal(src[:n], lay.src_meta[:n])
    assert rc["num_recv_tokens"] == lay.num_recv_tokens
    want = ep.EP_ERR_INVALID_ID if lay.invalid_count else ep.EP_OK
    assert rc["status"] == want


def assert_rows_equal(got: np.ndarray, exp: np.ndarray, what: str):
    """Bit-exact comparison of two [rows, cols] arrays that, on a mismatch,
    names the rows that differ, how many elements each, and whether a wrong
    row equals the expected row of another index (stale or misplaced data)."""
    if np.array_equal(got, exp):
        return
    bad = np.nonzero((got != exp).any(axis=1))[0]
    lines = [f"{what}: {len(bad)} of {got.shape[0]} rows differ"]
    keys = {exp[r].tobytes(): r for r in range(exp.shape[0])}
    for r in bad[:12]:
        n = int((got[r] != exp[r]).sum())
        other = keys.get(got[r].tobytes())
        lines.append(f"  row {r}: {n} elements differ" +
                     (f"; equals expected row {other}" if other is not None else ""))
    raise AssertionError("\n".join(lines))
