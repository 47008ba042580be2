"""MI355X (gfx950) MoE routing layout, dispatch copy and combine.

A thin ctypes binding of the C ABI declared in ``include/ep.h`` and built into
``libep.so`` next to this file (``python -m combine_ep_layout_08_amd.build``).
Every step of the computation runs in the library's HIP kernels; this module
only marshals arguments.  PyTorch supplies device memory and the current
stream.  There is no fallback: without the built library, every entry point
raises.

Low-level functions carry the C names (``ep_layout``, ``ep_dispatch``, ...)
and take raw pointers.  :class:`Handle` wraps them for torch tensors.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch  # noqa: F401  (loaded first so libep.so binds torch's HIP runtime)

__all__ = [
    "EP_OK", "EP_ERR_NULL", "EP_ERR_SHAPE", "EP_ERR_DTYPE", "EP_ERR_UNSUPPORTED",
    "EP_ERR_MISALIGNED", "EP_ERR_WORKSPACE", "EP_ERR_NOT_LAID_OUT", "EP_ERR_CAPACITY",
    "EP_ERR_INVALID_ID", "EP_ERR_HIP", "EP_ERR_TIMEOUT", "EP_BF16", "EP_FP8_E4M3", "EP_F32", "EP_I32",
    "EP_I64", "EpError", "ep_handle", "lib", "Handle", "BoundCall", "ep_capacity_bound",
    "ep_workspace_bytes", "ep_handle_init", "ep_layout", "ep_layout_noalloc", "ep_layout_dispatch",
    "ep_handle_read_counts",
    "ep_handle_import", "ep_dispatch", "ep_combine", "ep_status_str", "ep_handle_sizeof",
    "ep_time_next_call", "time_next_call", "ep_combine_backward", "ep_dispatch_backward",
    "ep_dispatch_rank", "ep_dispatch_rank_quant", "ep_combine_rank", "ep_tma_aligned_rows",
    "ep_sf_packs",
    "ep_quantize_fp8", "ep_dispatch_quant", "EP_SF_F32", "EP_SF_UE8M0", "quantize_fp8",
]

LIB_PATH = os.environ.get("EP_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libep.so")

(EP_OK, EP_ERR_NULL, EP_ERR_SHAPE, EP_ERR_DTYPE, EP_ERR_UNSUPPORTED, EP_ERR_MISALIGNED,
 EP_ERR_WORKSPACE, EP_ERR_NOT_LAID_OUT, EP_ERR_CAPACITY, EP_ERR_INVALID_ID,
 EP_ERR_HIP, EP_ERR_TIMEOUT) = range(12)
EP_BF16, EP_FP8_E4M3, EP_F32, EP_I32, EP_I64 = range(5)
EP_DISPATCH_ZERO_PADDING, EP_DISPATCH_STREAMING = 1, 2
EP_SF_F32, EP_SF_UE8M0 = 0, 1
_SF_FORMATS = {"f32": EP_SF_F32, "ue8m0": EP_SF_UE8M0}
EP_ERRBIT_CAPACITY = 1
EP_ERRBIT_INVALID_ID = 2
EP_ERRBIT_SCAN_TIMEOUT = 4
# Indices into the handle's device scalars (Handle.scalars), as in ep.h.
EP_SCALAR_NUM_RECV_TOKENS, EP_SCALAR_ERROR_BITS, EP_SCALAR_INVALID_COUNT = 0, 1, 2
EP_SCALAR_NUM_EXPANDED = 5


class ep_handle(ctypes.Structure):
    """Mirror of ``struct ep_handle`` (checked against ep_handle_sizeof)."""
    _fields_ = [
        ("max_tokens", ctypes.c_int32),
        ("num_tokens", ctypes.c_int32),
        ("num_topk", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("expert_alignment", ctypes.c_int32),
        ("laid_out", ctypes.c_int32),
        ("capacity", ctypes.c_int64),
        ("counts", ctypes.c_void_p),
        ("psum", ctypes.c_void_p),
        ("dst_slot", ctypes.c_void_p),
        ("src_meta", ctypes.c_void_p),
        ("scalars", ctypes.c_void_p),
        ("tile_status", ctypes.c_void_p),
        ("topk_idx", ctypes.c_void_p),
        ("topk_idx_dtype", ctypes.c_int32),
        ("status_tiles", ctypes.c_int32),
        ("recv_row", ctypes.c_void_p),
        ("recv_src", ctypes.c_void_p),
    ]


class EpError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {ep_status_str(status)}" if what else ep_status_str(status))


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_HP = ctypes.POINTER(ep_handle)

_SIGNATURES = {
    "ep_handle_sizeof": (ctypes.c_size_t, []),
    "ep_capacity_bound": (_I64, [_I32, _I32, _I32, _I32]),
    "ep_workspace_bytes": (ctypes.c_size_t, [_I32, _I32, _I32, _I32, _I64]),
    "ep_handle_init": (ctypes.c_int, [_HP, _I32, _I32, _I32, _I32, _I64, _P, ctypes.c_size_t, _P]),
    "ep_layout": (ctypes.c_int, [_HP, _P, ctypes.c_int, _I32, _P, _P]),
    "ep_layout_noalloc": (ctypes.c_int, [_HP, _P, ctypes.c_int, _I32, _P, _P]),
    "ep_handle_read_counts": (ctypes.c_int, [_HP, _P, _P, _P, _P, _P, _P, _P]),
    "ep_handle_import": (ctypes.c_int, [_HP, _P, ctypes.c_int, _I32, _P, _P, _P, _P, _I32, _P]),
    "ep_dispatch": (ctypes.c_int, [_HP, _P, ctypes.c_int, _I32, _P, _I64, _I64, _I32, _P, _P,
                                   _P, _I64, _I64, _P, _I32, _P]),
    "ep_layout_dispatch": (ctypes.c_int, [_HP, _P, ctypes.c_int, _I32, _P,
                                          _P, ctypes.c_int, _I32, _P, _I64, _I64, _I32, _P, _P,
                                          _P, _I64, _I64, _P, _I32, _P]),
    "ep_tma_aligned_rows": (_I64, [_I64]),
    "ep_sf_packs": (_I32, [_I32, ctypes.c_int]),
    "ep_quantize_fp8": (ctypes.c_int, [_P, _I32, _I32, ctypes.c_int, _P, _P, _I64, _I64, _P]),
    "ep_dispatch_quant": (ctypes.c_int, [_HP, _P, _I32, ctypes.c_int, _P, _P, _P, _I64, _I64,
                                         _P, _I32, _P]),
    "ep_combine": (ctypes.c_int, [_HP, _P, ctypes.c_int, _I32, _P, _P, _P, _P, _P, _P]),
    "ep_dispatch_rank": (ctypes.c_int, [_HP, _P, ctypes.c_int, _I32, _P, _I64, _I64, _I32, _P,
                                        _P, _P, _I64, _I64, _P, _P, _P]),
    "ep_dispatch_rank_quant": (ctypes.c_int, [_HP, _P, _I32, ctypes.c_int, _P, _P, _P, _I64,
                                              _I64, _P, _P, _P]),
    "ep_combine_rank": (ctypes.c_int, [_HP, _P, _I32, _P, _P, _P, _P]),
    "ep_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "ep_time_next_call": (ctypes.c_int, [_P, _P]),
    "ep_combine_backward": (ctypes.c_int, [_HP, _P, _I32, _P, _P, _P, _P, _P, _P, _P]),
    "ep_dispatch_backward": (ctypes.c_int, [_HP, _P, _I32, _P, _P, _P, _P]),
}

_lib = None


def lib():
    """The loaded ``libep.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m combine_ep_layout_08_amd.build` (there is no fallback path)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        if handle.ep_handle_sizeof() != ctypes.sizeof(ep_handle):
            raise RuntimeError("ep_handle layout mismatch between libep.so and the binding")
        _lib = handle
    return _lib


# ---------------------------------------------------------------- C-named calls

def ep_handle_sizeof() -> int:
    return int(lib().ep_handle_sizeof())


def ep_capacity_bound(num_tokens: int, num_topk: int, num_experts: int,
                      expert_alignment: int) -> int:
    return int(lib().ep_capacity_bound(num_tokens, num_topk, num_experts, expert_alignment))


def ep_workspace_bytes(max_tokens: int, num_topk: int, num_experts: int,
                       expert_alignment: int, capacity: int) -> int:
    return int(lib().ep_workspace_bytes(max_tokens, num_topk, num_experts,
                                        expert_alignment, capacity))


def ep_handle_init(h: ep_handle, max_tokens, num_topk, num_experts, expert_alignment,
                   capacity, workspace_ptr, ws_bytes, stream) -> int:
    return lib().ep_handle_init(ctypes.byref(h), max_tokens, num_topk, num_experts,
                                expert_alignment, capacity, workspace_ptr, ws_bytes, stream)


def ep_layout(h: ep_handle, topk_idx_ptr, idx_dtype, num_tokens, stats_ptr, stream) -> int:
    return lib().ep_layout(ctypes.byref(h), topk_idx_ptr, idx_dtype, num_tokens, stats_ptr,
                           stream)


def ep_layout_noalloc(h: ep_handle, topk_idx_ptr, idx_dtype, num_tokens, stats_ptr,
                      stream) -> int:
    return lib().ep_layout_noalloc(ctypes.byref(h), topk_idx_ptr, idx_dtype, num_tokens,
                                   stats_ptr, stream)


def ep_handle_read_counts(h: ep_handle, counts_ptr, psum_ptr, num_expanded_ptr,
                          num_recv_ptr, error_bits_ptr, invalid_ptr, stream) -> int:
    return lib().ep_handle_read_counts(ctypes.byref(h), counts_ptr, psum_ptr,
                                       num_expanded_ptr, num_recv_ptr, error_bits_ptr,
                                       invalid_ptr, stream)


def ep_handle_import(h: ep_handle, topk_idx_ptr, idx_dtype, num_tokens, counts_ptr, psum_ptr,
                     dst_ptr, src_meta_ptr, num_recv_tokens, stream) -> int:
    return lib().ep_handle_import(ctypes.byref(h), topk_idx_ptr, idx_dtype, num_tokens,
                                  counts_ptr, psum_ptr, dst_ptr, src_meta_ptr,
                                  num_recv_tokens, stream)


def ep_dispatch(h: ep_handle, x_ptr, x_dtype, hidden, sf_ptr, sf_ts, sf_hs, num_sf_packs,
                w_ptr, out_x_ptr, out_sf_ptr, out_ts, out_hs, out_w_ptr, flags,
                stream) -> int:
    return lib().ep_dispatch(ctypes.byref(h), x_ptr, x_dtype, hidden, sf_ptr, sf_ts, sf_hs,
                             num_sf_packs, w_ptr, out_x_ptr, out_sf_ptr, out_ts, out_hs,
                             out_w_ptr, flags, stream)


def ep_tma_aligned_rows(rows: int) -> int:
    return int(lib().ep_tma_aligned_rows(rows))


def ep_sf_packs(hidden: int, fmt: int) -> int:
    return int(lib().ep_sf_packs(hidden, fmt))


def ep_quantize_fp8(x_ptr, num_tokens, hidden, fmt, out_q_ptr, out_sf_ptr, out_ts, out_hs,
                    stream) -> int:
    return lib().ep_quantize_fp8(x_ptr, num_tokens, hidden, fmt, out_q_ptr, out_sf_ptr, out_ts,
                                 out_hs, stream)


def ep_dispatch_quant(h: ep_handle, x_ptr, hidden, fmt, w_ptr, out_x_ptr, out_sf_ptr, out_ts,
                      out_hs, out_w_ptr, zero_padding, stream) -> int:
    return lib().ep_dispatch_quant(ctypes.byref(h), x_ptr, hidden, fmt, w_ptr, out_x_ptr,
                                   out_sf_ptr, out_ts, out_hs, out_w_ptr, zero_padding, stream)


def ep_combine(h: ep_handle, y_ptr, y_dtype, hidden, w_ptr, bias_ptr, bias0_ptr, bias1_ptr,
               out_ptr, stream) -> int:
    return lib().ep_combine(ctypes.byref(h), y_ptr, y_dtype, hidden, w_ptr, bias_ptr, bias0_ptr,
                            bias1_ptr, out_ptr, stream)


def ep_dispatch_rank(h: ep_handle, x_ptr, x_dtype, hidden, sf_ptr, sf_ts, sf_hs,
                     num_sf_packs, w_ptr, out_x_ptr, out_sf_ptr, out_ts, out_hs, out_idx_ptr,
                     out_w_ptr, stream) -> int:
    return lib().ep_dispatch_rank(ctypes.byref(h), x_ptr, x_dtype, hidden, sf_ptr, sf_ts, sf_hs,
                                  num_sf_packs, w_ptr, out_x_ptr, out_sf_ptr, out_ts, out_hs,
                                  out_idx_ptr, out_w_ptr, stream)


def ep_dispatch_rank_quant(h: ep_handle, x_ptr, hidden, fmt, w_ptr, out_x_ptr, out_sf_ptr,
                           out_ts, out_hs, out_idx_ptr, out_w_ptr, stream) -> int:
    return lib().ep_dispatch_rank_quant(ctypes.byref(h), x_ptr, hidden, fmt, w_ptr, out_x_ptr,
                                        out_sf_ptr, out_ts, out_hs, out_idx_ptr, out_w_ptr,
                                        stream)


def ep_combine_rank(h: ep_handle, x_ptr, hidden, bias0_ptr, bias1_ptr, out_ptr, stream) -> int:
    return lib().ep_combine_rank(ctypes.byref(h), x_ptr, hidden, bias0_ptr, bias1_ptr, out_ptr,
                                 stream)


def ep_combine_backward(h: ep_handle, grad_out_ptr, hidden, w_ptr, y_ptr, bias_ptr, grad_y_ptr,
                        grad_w_ptr, grad_bias_ptr, stream) -> int:
    return lib().ep_combine_backward(ctypes.byref(h), grad_out_ptr, hidden, w_ptr, y_ptr,
                                     bias_ptr, grad_y_ptr, grad_w_ptr, grad_bias_ptr, stream)


def ep_dispatch_backward(h: ep_handle, grad_out_x_ptr, hidden, grad_out_w_ptr, grad_x_ptr,
                         grad_w_ptr, stream) -> int:
    return lib().ep_dispatch_backward(ctypes.byref(h), grad_out_x_ptr, hidden, grad_out_w_ptr,
                                      grad_x_ptr, grad_w_ptr, stream)


def ep_status_str(status: int) -> str:
    return lib().ep_status_str(status).decode()


def ep_time_next_call(start_event, stop_event) -> int:
    """Attach raw HIP events (handles) to the next layout/dispatch/combine."""
    return lib().ep_time_next_call(start_event, stop_event)


def time_next_call(start: "torch.cuda.Event", stop: "torch.cuda.Event") -> None:
    """Stamp two torch events with the first kernel start and last kernel end
    of the next layout/dispatch/combine call on this thread."""
    for e in (start, stop):
        if e.cuda_event == 0:           # torch creates events lazily on first record
            e.record()
    _check(ep_time_next_call(start.cuda_event, stop.cuda_event), "ep_time_next_call")


# ---------------------------------------------------------------- torch wrapper

def _stream() -> int:
    """Raw handle of the current device's current stream: the value of
    torch.cuda.current_stream().cuda_stream, read without building a Stream
    object (0.3 us instead of 2.8 us per call on MI355X)."""
    return torch._C._cuda_getCurrentRawStream(torch.cuda.current_device())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _check(status: int, what: str):
    if status != EP_OK:
        raise EpError(status, what)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _dev(t: torch.Tensor, name: str):
    _need(t.is_cuda, f"{name} must be a device tensor")
    _need(t.is_contiguous(), f"{name} must be contiguous")


def _dev_strided(t: torch.Tensor, name: str):
    """Scale tensors may have any non-negative strides (the kernels take them)."""
    _need(t.is_cuda, f"{name} must be a device tensor")
    _need(t.dim() == 2 and min(t.stride()) >= 0, f"{name} must be a 2-D strided view")


class BoundCall:
    """One entry point with its arguments validated and marshalled once.

    Calling it enqueues the same call on the current stream (read at every
    call) and returns what the direct method returns.  It keeps the tensors it
    was bound to alive: their contents may change between calls (new routing,
    new payloads), their storage and shapes may not.  A direct method spends
    about 5-6 us of host time per call on validation and marshalling, a bound
    call about 3 us (the C entry point and the launch), which lets small
    batches run at the GPU's pace.

    Dispatch and combine calls are bound for the handle's token count at bind
    time (their tensors were checked against it) and refuse to run once a
    later layout has changed it, as the direct methods would."""
    __slots__ = ("_fn", "_args", "_what", "_result", "_keep", "_h", "_tokens")

    def __init__(self, fn, args, what, result, keep, h=None):
        self._fn, self._args, self._what = fn, args, what
        self._result, self._keep = result, keep
        self._h = h
        self._tokens = None if h is None else h.num_tokens

    def __call__(self):
        if self._h is not None and self._h.num_tokens != self._tokens:
            raise ValueError(f"{self._what}: bound for {self._tokens} tokens, but the handle's "
                             f"layout now has {self._h.num_tokens}")
        status = self._fn(*self._args, _stream())
        if status != EP_OK:
            raise EpError(status, self._what)
        return self._result


_SF_DTYPES = (torch.float32, torch.int32)


def _scale_packs(sf, T, H, rows, out_sf, col_major, device):
    """Check FP8 scale packs and allocate their output.  sf: fp32 [T, H/128]
    (one scale per 128 channels) or int32 [T, P] (P packs of four UE8M0
    exponent bytes), any strides.  Returns (packs, sf strides, out_sf, out
    strides); a column-major out_sf has token stride 1 and pack stride
    ep_tma_aligned_rows(rows)."""
    _need(sf is not None, "FP8 dispatch needs scale factors")
    _dev_strided(sf, "sf")
    _need(sf.dtype in _SF_DTYPES and sf.dim() == 2 and sf.shape[0] == T,
          "sf must be fp32 [T, H/128] or int32 packs [T, P]")
    packs = sf.shape[1]
    _need(sf.dtype == torch.int32 or packs == H // 128, "fp32 sf must be [T, H/128]")
    if out_sf is None:
        if col_major:
            store = torch.empty((packs, ep_tma_aligned_rows(rows)), dtype=sf.dtype, device=device)
            out_sf = store[:, :rows].t()
        else:
            out_sf = torch.empty((rows, packs), dtype=sf.dtype, device=device)
    _dev_strided(out_sf, "out_sf")
    _need(out_sf.dtype == sf.dtype and tuple(out_sf.shape) == (rows, packs),
          f"out_sf must be [{rows}, {packs}] of sf's dtype")
    return packs, sf.stride(), out_sf, out_sf.stride()


def _sf_format(scale_format) -> int:
    fmt = _SF_FORMATS.get(scale_format, scale_format)
    _need(fmt in (EP_SF_F32, EP_SF_UE8M0), "scale_format must be 'f32' or 'ue8m0'")
    return fmt


def _quant_sf_out(out_sf, rows, packs, fmt, col_major, device):
    dt = torch.float32 if fmt == EP_SF_F32 else torch.int32
    if out_sf is None:
        if col_major:
            out_sf = torch.empty((packs, ep_tma_aligned_rows(rows)), dtype=dt,
                                 device=device)[:, :rows].t()
        else:
            out_sf = torch.empty((rows, packs), dtype=dt, device=device)
    _dev_strided(out_sf, "out_sf")
    _need(out_sf.dtype == dt and tuple(out_sf.shape) == (rows, packs),
          f"out_sf must be [{rows}, {packs}] {dt}")
    return out_sf


def quantize_fp8(x: torch.Tensor, scale_format="f32", out_q=None, out_sf=None,
                 col_major_sf: bool = False):
    """bf16 [T, H] -> (E4M3FN codes uint8 [T, H], scales): fp32 [T, H/128]
    for 'f32', int32 packs [T, ceil(H/512)] of UE8M0 exponents for 'ue8m0'."""
    _dev(x, "x")
    _need(x.dtype == torch.bfloat16 and x.dim() == 2, "x must be bf16 [T, H]")
    T, H = x.shape
    fmt = _sf_format(scale_format)
    packs = ep_sf_packs(H, fmt)
    _need(packs > 0, "hidden must be a positive multiple of 128")
    if out_q is None:
        out_q = torch.empty((T, H), dtype=torch.uint8, device=x.device)
    _dev(out_q, "out_q")
    _need(out_q.dtype in (torch.uint8, torch.float8_e4m3fn) and tuple(out_q.shape) == (T, H),
          "out_q must be FP8 codes [T, H]")
    out_sf = _quant_sf_out(out_sf, T, packs, fmt, col_major_sf, x.device)
    ts, hs = out_sf.stride()
    _check(ep_quantize_fp8(_ptr(x), T, H, fmt, _ptr(out_q), _ptr(out_sf), ts, hs, _stream()),
           "ep_quantize_fp8")
    return out_q, out_sf


class Handle:
    """Routing state in a torch-allocated workspace, with layout, dispatch and
    combine on torch tensors.  ``capacity`` defaults to the worst-case bound,
    so no count needs to be read back before dispatch."""

    def __init__(self, max_tokens: int, num_topk: int, num_experts: int,
                 expert_alignment: int = 1, capacity: Optional[int] = None,
                 device="cuda"):
        if capacity is None:
            capacity = ep_capacity_bound(max_tokens, num_topk, num_experts, expert_alignment)
            _need(capacity >= 0, "invalid sizes")
        nbytes = ep_workspace_bytes(max_tokens, num_topk, num_experts, expert_alignment,
                                    capacity)
        _need(nbytes > 0, "sizes outside the library's limits")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.h = ep_handle()
        _check(ep_handle_init(self.h, max_tokens, num_topk, num_experts, expert_alignment,
                              capacity, self.workspace.data_ptr(), nbytes, _stream()),
               "ep_handle_init")
        self.capacity = capacity
        self.topk_idx = None      # kept alive: the handle borrows it

    # -- views of the handle's device arrays
    def _view(self, ptr: int, n: int) -> torch.Tensor:
        off = ptr - self.workspace.data_ptr()
        return self.workspace[off:off + 4 * n].view(torch.int32)

    @property
    def num_tokens(self) -> int:
        return self.h.num_tokens

    @property
    def counts(self) -> torch.Tensor:
        return self._view(self.h.counts, self.h.num_experts)

    @property
    def psum(self) -> torch.Tensor:
        return self._view(self.h.psum, self.h.num_experts + 1)

    @property
    def dst_slot(self) -> torch.Tensor:
        return self._view(self.h.dst_slot, self.h.num_tokens * self.h.num_topk).view(
            self.h.num_tokens, self.h.num_topk)

    @property
    def src_meta(self) -> torch.Tensor:
        return self._view(self.h.src_meta, self.capacity)

    @property
    def scalars(self) -> torch.Tensor:
        return self._view(self.h.scalars, 8)

    @property
    def recv_row(self) -> torch.Tensor:
        return self._view(self.h.recv_row, self.h.num_tokens)

    @property
    def recv_src(self) -> torch.Tensor:
        return self._view(self.h.recv_src, self.h.max_tokens)

    def _layout_call(self, topk_idx, cumulative_stats, noalloc=False):
        _dev(topk_idx, "topk_idx")
        _need(topk_idx.dim() == 2 and topk_idx.shape[1] == self.h.num_topk,
              "topk_idx must be [num_tokens, num_topk]")
        _need(topk_idx.dtype in (torch.int64, torch.int32), "topk_idx must be int64 or int32")
        if cumulative_stats is not None:
            _dev(cumulative_stats, "cumulative_stats")
            _need(cumulative_stats.dtype == torch.int32 and
                  cumulative_stats.numel() == self.h.num_experts,
                  "cumulative_stats must be int32 [num_experts]")
        dt = EP_I64 if topk_idx.dtype == torch.int64 else EP_I32
        fn = lib().ep_layout_noalloc if noalloc else lib().ep_layout
        return fn, (ctypes.byref(self.h), _ptr(topk_idx), dt, topk_idx.shape[0],
                    _ptr(cumulative_stats))

    def layout(self, topk_idx: torch.Tensor,
               cumulative_stats: Optional[torch.Tensor] = None) -> "Handle":
        fn, args = self._layout_call(topk_idx, cumulative_stats)
        _check(fn(*args, _stream()), "ep_layout")
        self.topk_idx = topk_idx
        return self

    def layout_noalloc(self, topk_idx: torch.Tensor,
                       cumulative_stats: Optional[torch.Tensor] = None) -> "Handle":
        """``layout`` through ep_layout_noalloc: the scans' scratch is the
        library's static per-device array, not the handle's workspace (calls
        that overlap on one device race)."""
        fn, args = self._layout_call(topk_idx, cumulative_stats, noalloc=True)
        _check(fn(*args, _stream()), "ep_layout_noalloc")
        self.topk_idx = topk_idx
        return self

    def bind_layout(self, topk_idx: torch.Tensor,
                    cumulative_stats: Optional[torch.Tensor] = None) -> BoundCall:
        """``layout`` bound to these tensors (see BoundCall); the handle
        borrows ``topk_idx`` from now on."""
        fn, args = self._layout_call(topk_idx, cumulative_stats)
        self.topk_idx = topk_idx
        return BoundCall(fn, args, "ep_layout", self, (topk_idx, cumulative_stats))

    def _layout_dispatch_call(self, topk_idx, x, sf, topk_weights, zero_padding, out_x, out_sf,
                              out_w, want_weights, col_major_sf, cumulative_stats, streaming):
        lfn, largs = self._layout_call(topk_idx, cumulative_stats)
        _, dargs, result, keep = self._dispatch_call(
            x, sf, topk_weights, zero_padding, out_x, out_sf, out_w, want_weights, col_major_sf,
            num_tokens=topk_idx.shape[0], streaming=streaming)
        # ep_layout_dispatch takes the layout's arguments, then the dispatch's
        # (the handle appears once)
        args = largs + dargs[1:]
        return lib().ep_layout_dispatch, args, result, keep + (topk_idx, cumulative_stats)

    def layout_dispatch(self, topk_idx: torch.Tensor, x: torch.Tensor,
                        sf: Optional[torch.Tensor] = None,
                        topk_weights: Optional[torch.Tensor] = None, zero_padding: bool = False,
                        out_x: Optional[torch.Tensor] = None, out_sf: Optional[torch.Tensor] = None,
                        out_w: Optional[torch.Tensor] = None, want_weights: bool = False,
                        col_major_sf: bool = False,
                        cumulative_stats: Optional[torch.Tensor] = None,
                        streaming: bool = False):
        """``layout`` then ``dispatch`` in one call (ep_layout_dispatch: the
        same outputs, one host-side check of both argument sets).  Returns
        (out_x, out_sf, out_w)."""
        fn, args, result, _ = self._layout_dispatch_call(
            topk_idx, x, sf, topk_weights, zero_padding, out_x, out_sf, out_w, want_weights,
            col_major_sf, cumulative_stats, streaming)
        _check(fn(*args, _stream()), "ep_layout_dispatch")
        self.topk_idx = topk_idx
        return result

    def bind_layout_dispatch(self, topk_idx: torch.Tensor, x: torch.Tensor,
                             sf: Optional[torch.Tensor] = None,
                             topk_weights: Optional[torch.Tensor] = None,
                             zero_padding: bool = False, out_x: Optional[torch.Tensor] = None,
                             out_sf: Optional[torch.Tensor] = None,
                             out_w: Optional[torch.Tensor] = None, want_weights: bool = False,
                             col_major_sf: bool = False,
                             cumulative_stats: Optional[torch.Tensor] = None,
                             streaming: bool = False) -> "BoundCall":
        """``layout_dispatch`` bound to these tensors (see BoundCall)."""
        fn, args, result, keep = self._layout_dispatch_call(
            topk_idx, x, sf, topk_weights, zero_padding, out_x, out_sf, out_w, want_weights,
            col_major_sf, cumulative_stats, streaming)
        self.topk_idx = topk_idx
        # no token-count check: the call lays the batch out itself
        return BoundCall(fn, args, "ep_layout_dispatch", result, keep)

    def import_layout(self, topk_idx: torch.Tensor, counts, psum, dst_slot, src_meta,
                      num_recv_tokens: int) -> "Handle":
        """Install a host-computed layout (numpy int32 arrays)."""
        import numpy as np
        _dev(topk_idx, "topk_idx")
        c = np.ascontiguousarray(counts, np.int32)
        p = np.ascontiguousarray(psum, np.int32)
        d = np.ascontiguousarray(dst_slot, np.int32)
        s = np.ascontiguousarray(src_meta, np.int32)
        dt = EP_I64 if topk_idx.dtype == torch.int64 else EP_I32
        _check(ep_handle_import(self.h, _ptr(topk_idx), dt, topk_idx.shape[0], c.ctypes.data,
                                p.ctypes.data, d.ctypes.data, s.ctypes.data if s.size else None,
                                num_recv_tokens, _stream()), "ep_handle_import")
        self.topk_idx = topk_idx
        return self

    def read_counts(self, check: bool = True) -> dict:
        """Blocking: wait for the stream and read counts, psum and scalars."""
        import numpy as np
        E = self.h.num_experts
        counts = np.zeros(E, np.int32)
        psum = np.zeros(E + 1, np.int32)
        ne = ctypes.c_int64(0)
        nr = ctypes.c_int32(0)
        eb = ctypes.c_uint32(0)
        inv = ctypes.c_int32(0)
        st = ep_handle_read_counts(self.h, counts.ctypes.data, psum.ctypes.data,
                                   ctypes.addressof(ne), ctypes.addressof(nr),
                                   ctypes.addressof(eb), ctypes.addressof(inv), _stream())
        if check and st not in (EP_OK,):
            raise EpError(st, "ep_handle_read_counts")
        return dict(status=st, counts=counts, psum=psum, num_expanded=ne.value,
                    num_recv_tokens=nr.value, error_bits=eb.value, invalid_count=inv.value)

    def dispatch(self, x: torch.Tensor, sf: Optional[torch.Tensor] = None,
                 topk_weights: Optional[torch.Tensor] = None, zero_padding: bool = False,
                 out_x: Optional[torch.Tensor] = None, out_sf: Optional[torch.Tensor] = None,
                 out_w: Optional[torch.Tensor] = None, want_weights: bool = False,
                 col_major_sf: bool = False, streaming: bool = False):
        """x: bf16 [T, H], or FP8 (float8_e4m3fn or uint8 codes) [T, H] with
        scales ``sf``: fp32 [T, H/128] or int32 packs [T, P] (any strides).
        Returns (out_x, out_sf, out_w); outputs are allocated with
        ``capacity`` rows unless given (out_sf column-major, TMA-aligned, when
        ``col_major_sf``).  ``streaming``: non-temporal stores of the rows
        (EP_DISPATCH_STREAMING)."""
        fn, args, result, _ = self._dispatch_call(x, sf, topk_weights, zero_padding, out_x,
                                                  out_sf, out_w, want_weights, col_major_sf,
                                                  streaming=streaming)
        _check(fn(*args, _stream()), "ep_dispatch")
        return result

    def bind_dispatch(self, x: torch.Tensor, sf: Optional[torch.Tensor] = None,
                      topk_weights: Optional[torch.Tensor] = None, zero_padding: bool = False,
                      out_x: Optional[torch.Tensor] = None, out_sf: Optional[torch.Tensor] = None,
                      out_w: Optional[torch.Tensor] = None, want_weights: bool = False,
                      col_major_sf: bool = False, streaming: bool = False) -> BoundCall:
        """``dispatch`` bound to these tensors (see BoundCall); each call
        returns (out_x, out_sf, out_w)."""
        fn, args, result, keep = self._dispatch_call(x, sf, topk_weights, zero_padding, out_x,
                                                      out_sf, out_w, want_weights, col_major_sf,
                                                      streaming=streaming)
        return BoundCall(fn, args, "ep_dispatch", result, keep, self.h)

    def _dispatch_call(self, x, sf, topk_weights, zero_padding, out_x, out_sf, out_w,
                       want_weights, col_major_sf, num_tokens=None, streaming=False):
        T = self.h.num_tokens if num_tokens is None else num_tokens
        _dev(x, "x")
        _need(x.dim() == 2 and x.shape[0] == T, "x must be [num_tokens, hidden]")
        H = x.shape[1]
        fp8 = x.dtype in (torch.float8_e4m3fn, torch.uint8)
        _need(fp8 or x.dtype == torch.bfloat16, "x must be bf16 or FP8 e4m3")
        cap = self.capacity
        if out_x is None:
            out_x = torch.empty((cap, H), dtype=x.dtype, device=x.device)
        _dev(out_x, "out_x")
        _need(out_x.shape == (cap, H) and out_x.dtype == x.dtype, "out_x must be [capacity, H]")
        packs, (sf_ts, sf_hs), (o_ts, o_hs) = 0, (0, 0), (0, 0)
        if fp8:
            packs, (sf_ts, sf_hs), out_sf, (o_ts, o_hs) = _scale_packs(
                sf, T, H, cap, out_sf, col_major_sf, x.device)
        else:
            _need(sf is None and out_sf is None, "scale factors are for FP8 only")
        if topk_weights is not None:
            _dev(topk_weights, "topk_weights")
            _need(topk_weights.dtype == torch.float32 and
                  tuple(topk_weights.shape) == (T, self.h.num_topk),
                  "topk_weights must be fp32 [T, K]")
        if want_weights and out_w is None:
            out_w = torch.empty(cap, dtype=torch.float32, device=x.device)
        if out_w is not None:
            _dev(out_w, "out_w")
            _need(out_w.dtype == torch.float32 and out_w.numel() == cap, "out_w: fp32 [capacity]")
        args = (ctypes.byref(self.h), _ptr(x), EP_FP8_E4M3 if fp8 else EP_BF16, H, _ptr(sf),
                sf_ts, sf_hs, packs, _ptr(topk_weights), _ptr(out_x), _ptr(out_sf), o_ts, o_hs,
                _ptr(out_w), (EP_DISPATCH_ZERO_PADDING if zero_padding else 0) |
                (EP_DISPATCH_STREAMING if streaming else 0))
        return lib().ep_dispatch, args, (out_x, out_sf, out_w), (x, sf, topk_weights)

    def dispatch_quant(self, x: torch.Tensor, scale_format="f32",
                       topk_weights: Optional[torch.Tensor] = None, zero_padding: bool = False,
                       out_x=None, out_sf=None, out_w=None, want_weights: bool = False,
                       col_major_sf: bool = False):
        """Quantise bf16 x [T, H] to FP8 and dispatch in one pass.  Returns
        (codes uint8 [capacity, H], scales [capacity, packs], out_w)."""
        T = self.h.num_tokens
        _dev(x, "x")
        _need(x.dtype == torch.bfloat16 and x.dim() == 2 and x.shape[0] == T,
              "x must be bf16 [num_tokens, H]")
        H = x.shape[1]
        fmt = _sf_format(scale_format)
        packs = ep_sf_packs(H, fmt)
        _need(packs > 0, "hidden must be a positive multiple of 128")
        cap = self.capacity
        if out_x is None:
            out_x = torch.empty((cap, H), dtype=torch.uint8, device=x.device)
        _dev(out_x, "out_x")
        _need(out_x.dtype in (torch.uint8, torch.float8_e4m3fn) and
              tuple(out_x.shape) == (cap, H), "out_x must be FP8 codes [capacity, H]")
        out_sf = _quant_sf_out(out_sf, cap, packs, fmt, col_major_sf, x.device)
        o_ts, o_hs = out_sf.stride()
        if topk_weights is not None:
            _dev(topk_weights, "topk_weights")
            _need(topk_weights.dtype == torch.float32 and
                  tuple(topk_weights.shape) == (T, self.h.num_topk),
                  "topk_weights must be fp32 [T, K]")
        if want_weights and out_w is None:
            out_w = torch.empty(cap, dtype=torch.float32, device=x.device)
        if out_w is not None:
            _dev(out_w, "out_w")
            _need(out_w.dtype == torch.float32 and out_w.numel() == cap, "out_w: fp32 [capacity]")
        _check(ep_dispatch_quant(self.h, _ptr(x), H, fmt, _ptr(topk_weights), _ptr(out_x),
                                 _ptr(out_sf), o_ts, o_hs, _ptr(out_w),
                                 1 if zero_padding else 0, _stream()), "ep_dispatch_quant")
        return out_x, out_sf, out_w

    def combine(self, y: torch.Tensor, topk_weights: Optional[torch.Tensor] = None,
                bias: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None,
                bias_0: Optional[torch.Tensor] = None,
                bias_1: Optional[torch.Tensor] = None) -> torch.Tensor:
        """y: bf16 [capacity, H] expert outputs; returns bf16 [T, H].  bias is
        the per-expert [E, H] bias; bias_0 / bias_1 are per-token [T, H]
        biases added after the reduction."""
        fn, args, out, _ = self._combine_call(y, topk_weights, bias, out, bias_0, bias_1)
        _check(fn(*args, _stream()), "ep_combine")
        return out

    def bind_combine(self, y: torch.Tensor, topk_weights: Optional[torch.Tensor] = None,
                     bias: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                     bias_0: Optional[torch.Tensor] = None,
                     bias_1: Optional[torch.Tensor] = None) -> BoundCall:
        """``combine`` bound to these tensors (see BoundCall); each call
        returns ``out``."""
        fn, args, out, keep = self._combine_call(y, topk_weights, bias, out, bias_0, bias_1)
        return BoundCall(fn, args, "ep_combine", out, keep, self.h)

    def _combine_call(self, y, topk_weights, bias, out, bias_0, bias_1):
        T = self.h.num_tokens
        _dev(y, "y")
        _need(y.dtype == torch.bfloat16, "combine input must be bf16")
        _need(y.dim() == 2 and y.shape[0] == self.capacity, "y must be [capacity, H]")
        H = y.shape[1]
        if topk_weights is not None:
            _dev(topk_weights, "topk_weights")
            _need(topk_weights.dtype == torch.float32 and
                  tuple(topk_weights.shape) == (T, self.h.num_topk),
                  "topk_weights must be fp32 [T, K]")
        if bias is not None:
            _dev(bias, "bias")
            _need(bias.dtype == torch.bfloat16 and tuple(bias.shape) == (self.h.num_experts, H),
                  "bias must be bf16 [E, H]")
        for name, b in (("bias_0", bias_0), ("bias_1", bias_1)):
            if b is not None:
                _dev(b, name)
                _need(b.dtype == torch.bfloat16 and tuple(b.shape) == (T, H),
                      f"{name} must be bf16 [T, H]")
        if out is None:
            out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
        _dev(out, "out")
        _need(tuple(out.shape) == (T, H) and out.dtype == torch.bfloat16, "out must be bf16 [T, H]")
        args = (ctypes.byref(self.h), _ptr(y), EP_BF16, H, _ptr(topk_weights), _ptr(bias),
                _ptr(bias_0), _ptr(bias_1), _ptr(out))
        return lib().ep_combine, args, out, (y, topk_weights, bias, bias_0, bias_1)


    # ------------------------------------------------------------ backward

    def combine_backward(self, grad_out: torch.Tensor, topk_weights=None, y=None, bias=None,
                         grad_y=None, want_grad_y: bool = True, want_grad_weights: bool = False,
                         want_grad_bias: bool = False):
        """Backward of combine.  grad_out: bf16 [T, H].  Returns
        (grad_y bf16 [capacity, H] or None, grad_topk_weights fp32 [T, K] or
        None, grad_bias fp32 [E, H] or None).  Rows of grad_y without a slot
        are left as they were (uninitialised when allocated here)."""
        T, K, E = self.h.num_tokens, self.h.num_topk, self.h.num_experts
        _dev(grad_out, "grad_out")
        _need(grad_out.dtype == torch.bfloat16 and grad_out.dim() == 2 and
              grad_out.shape[0] == T, "grad_out must be bf16 [T, H]")
        H = grad_out.shape[1]
        if topk_weights is not None:
            _dev(topk_weights, "topk_weights")
            _need(topk_weights.dtype == torch.float32 and tuple(topk_weights.shape) == (T, K),
                  "topk_weights must be fp32 [T, K]")
        if y is not None:
            _dev(y, "y")
            _need(y.dtype == torch.bfloat16 and tuple(y.shape) == (self.capacity, H),
                  "y must be bf16 [capacity, H]")
        if bias is not None:
            _dev(bias, "bias")
            _need(bias.dtype == torch.bfloat16 and tuple(bias.shape) == (E, H),
                  "bias must be bf16 [E, H]")
        if want_grad_y and grad_y is None:
            grad_y = torch.empty((self.capacity, H), dtype=torch.bfloat16, device=grad_out.device)
        if grad_y is not None:
            _dev(grad_y, "grad_y")
            _need(grad_y.dtype == torch.bfloat16 and tuple(grad_y.shape) == (self.capacity, H),
                  "grad_y must be bf16 [capacity, H]")
        gw = torch.empty((T, K), dtype=torch.float32, device=grad_out.device) \
            if want_grad_weights else None
        if gw is not None:
            _need(y is not None, "the weight gradient needs y")
        gb = torch.empty((E, H), dtype=torch.float32, device=grad_out.device) \
            if want_grad_bias else None
        _check(ep_combine_backward(self.h, _ptr(grad_out), H, _ptr(topk_weights), _ptr(y),
                                   _ptr(bias), _ptr(grad_y), _ptr(gw), _ptr(gb), _stream()),
               "ep_combine_backward")
        return grad_y, gw, gb

    def dispatch_backward(self, grad_out_x: torch.Tensor, grad_out_w=None,
                          want_grad_weights: bool = False):
        """Backward of dispatch.  grad_out_x: bf16 [capacity, H].  Returns
        (grad_x bf16 [T, H], grad_topk_weights fp32 [T, K] or None)."""
        T, K = self.h.num_tokens, self.h.num_topk
        _dev(grad_out_x, "grad_out_x")
        _need(grad_out_x.dtype == torch.bfloat16 and grad_out_x.dim() == 2 and
              grad_out_x.shape[0] == self.capacity, "grad_out_x must be bf16 [capacity, H]")
        H = grad_out_x.shape[1]
        if grad_out_w is not None:
            _dev(grad_out_w, "grad_out_w")
            _need(grad_out_w.dtype == torch.float32 and grad_out_w.numel() == self.capacity,
                  "grad_out_w must be fp32 [capacity]")
        gx = torch.empty((T, H), dtype=torch.bfloat16, device=grad_out_x.device)
        gw = torch.empty((T, K), dtype=torch.float32, device=grad_out_x.device) \
            if want_grad_weights else None
        _check(ep_dispatch_backward(self.h, _ptr(grad_out_x), H, _ptr(grad_out_w), _ptr(gx),
                                    _ptr(gw), _stream()), "ep_dispatch_backward")
        return gx, gw


    # ------------------------------------------------------------ rank layout

    def dispatch_rank(self, x: torch.Tensor, sf: Optional[torch.Tensor] = None,
                      topk_weights: Optional[torch.Tensor] = None, out_x=None, out_sf=None,
                      out_topk_idx=None, out_topk_weights=None, col_major_sf: bool = False):
        """Rank (non-expanded) dispatch: one row per received token, in token
        order, with [max_tokens] rows allocated; rows past num_recv_tokens are
        not written.  Returns (out_x, out_sf, out_topk_idx, out_topk_weights)."""
        T, K = self.h.num_tokens, self.h.num_topk
        M = self.h.max_tokens
        _dev(x, "x")
        _need(x.dim() == 2 and x.shape[0] == T, "x must be [num_tokens, hidden]")
        H = x.shape[1]
        fp8 = x.dtype in (torch.float8_e4m3fn, torch.uint8)
        _need(fp8 or x.dtype == torch.bfloat16, "x must be bf16 or FP8 e4m3")
        if out_x is None:
            out_x = torch.empty((M, H), dtype=x.dtype, device=x.device)
        _need(tuple(out_x.shape) == (M, H) and out_x.dtype == x.dtype and out_x.is_cuda,
              "out_x must be [max_tokens, H]")
        packs, (sf_ts, sf_hs), (o_ts, o_hs) = 0, (0, 0), (0, 0)
        if fp8:
            packs, (sf_ts, sf_hs), out_sf, (o_ts, o_hs) = _scale_packs(
                sf, T, H, M, out_sf, col_major_sf, x.device)
        else:
            _need(sf is None and out_sf is None, "scale factors are for FP8 only")
        idx_dtype = torch.int64 if self.h.topk_idx_dtype == EP_I64 else torch.int32
        if out_topk_idx is None:
            out_topk_idx = torch.empty((M, K), dtype=idx_dtype, device=x.device)
        _need(out_topk_idx.dtype == idx_dtype and tuple(out_topk_idx.shape) == (M, K),
              "out_topk_idx must be [max_tokens, K] of the layout's id dtype")
        if out_topk_weights is None:
            out_topk_weights = torch.empty((M, K), dtype=torch.float32, device=x.device)
        if topk_weights is not None:
            _dev(topk_weights, "topk_weights")
        _check(ep_dispatch_rank(self.h, _ptr(x), EP_FP8_E4M3 if fp8 else EP_BF16, H, _ptr(sf),
                                sf_ts, sf_hs, packs, _ptr(topk_weights), _ptr(out_x),
                                _ptr(out_sf),
                                o_ts, o_hs, _ptr(out_topk_idx), _ptr(out_topk_weights),
                                _stream()), "ep_dispatch_rank")
        return out_x, out_sf, out_topk_idx, out_topk_weights

    def dispatch_rank_quant(self, x: torch.Tensor, scale_format="f32",
                            topk_weights: Optional[torch.Tensor] = None, out_x=None, out_sf=None,
                            out_topk_idx=None, out_topk_weights=None,
                            col_major_sf: bool = False):
        """Quantise bf16 x [T, H] to FP8 and dispatch into the rank layout in
        one pass.  Returns (codes uint8 [max_tokens, H], scales [max_tokens,
        packs], out_topk_idx, out_topk_weights)."""
        T, K = self.h.num_tokens, self.h.num_topk
        M = self.h.max_tokens
        _dev(x, "x")
        _need(x.dtype == torch.bfloat16 and x.dim() == 2 and x.shape[0] == T,
              "x must be bf16 [num_tokens, H]")
        H = x.shape[1]
        fmt = _sf_format(scale_format)
        packs = ep_sf_packs(H, fmt)
        _need(packs > 0, "hidden must be a positive multiple of 128")
        if out_x is None:
            out_x = torch.empty((M, H), dtype=torch.uint8, device=x.device)
        _dev(out_x, "out_x")
        _need(out_x.dtype in (torch.uint8, torch.float8_e4m3fn) and tuple(out_x.shape) == (M, H),
              "out_x must be FP8 codes [max_tokens, H]")
        out_sf = _quant_sf_out(out_sf, M, packs, fmt, col_major_sf, x.device)
        o_ts, o_hs = out_sf.stride()
        idx_dtype = torch.int64 if self.h.topk_idx_dtype == EP_I64 else torch.int32
        if out_topk_idx is None:
            out_topk_idx = torch.empty((M, K), dtype=idx_dtype, device=x.device)
        _need(out_topk_idx.dtype == idx_dtype and tuple(out_topk_idx.shape) == (M, K),
              "out_topk_idx must be [max_tokens, K] of the layout's id dtype")
        if out_topk_weights is None:
            out_topk_weights = torch.empty((M, K), dtype=torch.float32, device=x.device)
        _need(out_topk_weights.dtype == torch.float32 and tuple(out_topk_weights.shape) == (M, K),
              "out_topk_weights must be fp32 [max_tokens, K]")
        if topk_weights is not None:
            _dev(topk_weights, "topk_weights")
            _need(topk_weights.dtype == torch.float32 and tuple(topk_weights.shape) == (T, K),
                  "topk_weights must be fp32 [T, K]")
        _check(ep_dispatch_rank_quant(self.h, _ptr(x), H, fmt, _ptr(topk_weights), _ptr(out_x),
                                      _ptr(out_sf), o_ts, o_hs, _ptr(out_topk_idx),
                                      _ptr(out_topk_weights), _stream()),
               "ep_dispatch_rank_quant")
        return out_x, out_sf, out_topk_idx, out_topk_weights

    def combine_rank(self, x: torch.Tensor, bias_0=None, bias_1=None, out=None) -> torch.Tensor:
        """x: bf16 [max_tokens, H] rank-layout rows; returns bf16 [T, H]."""
        T, M = self.h.num_tokens, self.h.max_tokens
        _dev(x, "x")
        _need(x.dtype == torch.bfloat16 and x.dim() == 2 and x.shape[0] == M,
              "x must be bf16 [max_tokens, H]")
        H = x.shape[1]
        for name, b in (("bias_0", bias_0), ("bias_1", bias_1)):
            if b is not None:
                _dev(b, name)
                _need(b.dtype == torch.bfloat16 and tuple(b.shape) == (T, H),
                      f"{name} must be bf16 [T, H]")
        if out is None:
            out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
        _check(ep_combine_rank(self.h, _ptr(x), H, _ptr(bias_0), _ptr(bias_1), _ptr(out),
                               _stream()), "ep_combine_rank")
        return out
