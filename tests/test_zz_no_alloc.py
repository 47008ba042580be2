"""ep_layout_noalloc, the layout whose scans keep their scratch (tile ticket,
call epoch, per-tile status words) in the library's static device array
instead of the handle's workspace, against ep_layout on the same ids through
the C ABI: every output bit-exact.  Calls in a row on one handle take the
decoupled-lookback form, then the count + place form, then the one-launch
form, each on a smaller batch than the one before, so a status word left in
the shared array by an earlier call would show up as a wrong row.  A batch
whose status words exceed the array is refused before any launch."""
import numpy as np
import pytest
import torch

import combine_ep_layout_08_amd as ep
from tests.gpu_util import needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]


def _ids(T, K, E, seed):
    """Uniform experts (a token may repeat one), 10 % empty slots, a few ids
    outside [-1, E) (counted and flagged, like empty ones)."""
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, E, size=(T, K), dtype=np.int64)
    idx[rng.random((T, K)) < 0.10] = -1
    idx[rng.random((T, K)) < 0.001] = E + 7
    idx[0, 0] = E + 7
    return idx


def _outputs(h, stats):
    rc = h.read_counts(check=False)
    n, r = rc["num_expanded"], max(rc["num_recv_tokens"], 0)
    return {
        "status": rc["status"], "error_bits": rc["error_bits"],
        "num_expanded": n, "num_recv_tokens": rc["num_recv_tokens"],
        "invalid_count": rc["invalid_count"],
        "counts": rc["counts"].copy(), "psum": rc["psum"].copy(),
        "dst": h.dst_slot.cpu().numpy().copy(),
        "src_meta": h.src_meta.cpu().numpy()[:n].copy(),
        "recv_row": h.recv_row.cpu().numpy().copy(),
        "recv_src": h.recv_src.cpu().numpy()[:r].copy(),
        "stats": stats.cpu().numpy().copy(),
    }


def _assert_same(got, want, what):
    for k in want:
        np.testing.assert_array_equal(np.asarray(got[k]), np.asarray(want[k]),
                                      err_msg=f"{what}: {k}")


def test_noalloc_layout_matches_layout_on_shrinking_batches():
    K, E, A = 8, 256, 128
    T_max = 110000                    # 880000 slots: more than 400 long tiles
    cap = ep.ep_capacity_bound(T_max, K, E, A)
    ref = ep.Handle(T_max, K, E, A, cap)
    h = ep.Handle(T_max, K, E, A, cap)
    # Poison the rows the layout defines, so nothing is left from init.
    h.dst_slot.fill_(-77)
    h.src_meta.fill_(-77)
    stats_ref = torch.zeros(E, dtype=torch.int32, device="cuda")
    stats = torch.zeros(E, dtype=torch.int32, device="cuda")
    for n, T in enumerate([T_max, 4096, 100]):   # lookback, count + place, one launch
        idx = torch.from_numpy(_ids(T, K, E, seed=900 + n)).cuda()
        say("noalloc layout", T, K, E, A)
        ref.layout(idx, cumulative_stats=stats_ref)
        h.layout_noalloc(idx, cumulative_stats=stats)
        torch.cuda.synchronize()
        want = _outputs(ref, stats_ref)
        got = _outputs(h, stats)
        assert want["status"] == ep.EP_ERR_INVALID_ID and want["num_expanded"] > 0
        _assert_same(got, want, f"T={T}")


def test_noalloc_layout_two_handles_alternate():
    """Two handles take turns on the shared array (ordered on one stream):
    each call must see only its own status words."""
    K, E, A = 8, 64, 16
    T_max = 110000
    cap = T_max * K + (A - 1) * E
    hs = [ep.Handle(T_max, K, E, A, cap) for _ in range(2)]
    refs = [ep.Handle(T_max, K, E, A, cap) for _ in range(2)]
    stats = torch.zeros(E, dtype=torch.int32, device="cuda")
    # lookback, lookback, count + place, count + place
    for n, T in enumerate([T_max, 104000, 9000, 8000]):
        i = n % 2
        idx = torch.from_numpy(_ids(T, K, E, seed=700 + n)).cuda()
        say("noalloc alternate", i, T, K, E, A)
        refs[i].layout(idx)
        hs[i].layout_noalloc(idx)
        torch.cuda.synchronize()
        _assert_same(_outputs(hs[i], stats), _outputs(refs[i], stats), f"handle {i} T={T}")


def test_noalloc_layout_refuses_batches_beyond_the_array():
    """E = 1024 at K = 8: 1026 status words per tile, so 127 long tiles fit in
    the 1 MiB array; 33000 tokens need 129 and are refused with nothing
    launched (the handle keeps its previous layout)."""
    K, E, A = 8, 1024, 1
    T = 33000
    h = ep.Handle(T, K, E, A, T * K)
    small = torch.from_numpy(_ids(3000, K, E, seed=5)).cuda()
    h.layout_noalloc(small)
    torch.cuda.synchronize()
    before = _outputs(h, torch.zeros(1))
    big = torch.from_numpy(_ids(T, K, E, seed=6)).cuda()
    say("noalloc refused", T, K, E)
    with pytest.raises(ep.EpError) as err:
        h.layout_noalloc(big)
    assert err.value.status == ep.EP_ERR_WORKSPACE
    torch.cuda.synchronize()
    _assert_same(_outputs(h, torch.zeros(1)), before, "after a refused call")
    # the workspace form takes the same batch
    h.layout(big)
    assert h.read_counts(check=False)["num_expanded"] > 0
