// C ABI of the layout / dispatch / combine library: argument validation,
// workspace carving and kernel launches.  The semantics of each entry point
// are documented in include/ep.h.  Nothing here allocates device memory or
// synchronises, except ep_handle_read_counts and ep_handle_import.
#include "../../include/ep.h"

#include <cstring>
#include <vector>

#include "ep_internal.h"

namespace {

constexpr size_t kCarveAlign = 256;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Carve {
    size_t counts, psum, dst, src_meta, scalars, status, recv_row, recv_src, total;
    int64_t tiles;
};

bool sizes_ok(int32_t max_tokens, int32_t K, int32_t E, int32_t A, int64_t capacity) {
    return max_tokens >= 0 && K >= 1 && E >= 1 && A >= 1 && capacity >= 0;
}

ep_status limits(int32_t max_tokens, int32_t K, int32_t E, int64_t capacity) {
    if (K > ep::kMaxTopk || E > ep::kMaxExperts) return EP_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(max_tokens) * K > INT32_MAX) return EP_ERR_UNSUPPORTED;
    if (capacity > INT32_MAX) return EP_ERR_UNSUPPORTED;
    return EP_OK;
}

Carve carve(int32_t max_tokens, int32_t K, int32_t E, int64_t capacity) {
    Carve c{};
    const int64_t slots = static_cast<int64_t>(max_tokens) * K;
    c.tiles = ep::layout_status_tiles(max_tokens, K);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = round_up(off + (bytes ? bytes : 4), kCarveAlign);
        return at;
    };
    c.counts = take(sizeof(int32_t) * static_cast<size_t>(E));
    c.psum = take(sizeof(int32_t) * static_cast<size_t>(E + 1));
    c.dst = take(sizeof(int32_t) * static_cast<size_t>(slots));
    c.src_meta = take(sizeof(int32_t) * static_cast<size_t>(capacity));
    c.scalars = take(sizeof(int32_t) * EP_NUM_SCALARS);
    c.status = take(sizeof(uint64_t) * static_cast<size_t>(c.tiles) * static_cast<size_t>(E + 2));
    c.recv_row = take(sizeof(int32_t) * static_cast<size_t>(max_tokens));
    c.recv_src = take(sizeof(int32_t) * static_cast<size_t>(max_tokens));
    c.total = off;
    return c;
}

ep_status hip_status(hipError_t e) { return e == hipSuccess ? EP_OK : EP_ERR_HIP; }

// Events for the next layout / dispatch / combine call on this host thread.
thread_local ep::CallEvents g_next_events;

ep::CallEvents take_events() {
    const ep::CallEvents ev = g_next_events;
    g_next_events = ep::CallEvents{};
    return ev;
}

// A handle from ep_handle_init (or a plain copy of one): workspace carved and
// sizes within the limits it was carved for.
bool handle_ready(const ep_handle *h) {
    return h && h->counts && h->psum && h->dst_slot && h->src_meta && h->scalars &&
           h->tile_status && h->recv_row && h->recv_src && h->max_tokens >= 0 &&
           h->num_topk >= 1 && h->num_topk <= ep::kMaxTopk && h->num_experts >= 1 &&
           h->num_experts <= ep::kMaxExperts && h->expert_alignment >= 1 && h->capacity >= 0;
}

}  // namespace

extern "C" {

size_t ep_handle_sizeof(void) { return sizeof(ep_handle); }

int64_t ep_capacity_bound(int32_t T, int32_t K, int32_t E, int32_t A) {
    if (T < 0 || K <= 0 || E <= 0 || A <= 0) return -1;
    const int64_t per_token = K < E ? K : E;
    const int64_t n = static_cast<int64_t>(T) * per_token + static_cast<int64_t>(A - 1) * E;
    return (n + A - 1) / A * A;
}

size_t ep_workspace_bytes(int32_t max_tokens, int32_t K, int32_t E, int32_t A, int64_t capacity) {
    if (!sizes_ok(max_tokens, K, E, A, capacity)) return 0;
    if (limits(max_tokens, K, E, capacity) != EP_OK) return 0;
    return carve(max_tokens, K, E, capacity).total;
}

ep_status ep_handle_init(ep_handle *h, int32_t max_tokens, int32_t K, int32_t E, int32_t A,
                         int64_t capacity, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!h || !ws) return h ? EP_ERR_WORKSPACE : EP_ERR_NULL;
    if (!sizes_ok(max_tokens, K, E, A, capacity)) return EP_ERR_SHAPE;
    const ep_status lim = limits(max_tokens, K, E, capacity);
    if (lim != EP_OK) return lim;
    if (!aligned(ws, kCarveAlign)) return EP_ERR_MISALIGNED;
    const Carve c = carve(max_tokens, K, E, capacity);
    if (ws_bytes < c.total) return EP_ERR_WORKSPACE;
    char *base = static_cast<char *>(ws);
    ep_handle n{};
    n.max_tokens = max_tokens;
    n.num_tokens = 0;
    n.num_topk = K;
    n.num_experts = E;
    n.expert_alignment = A;
    n.laid_out = 0;
    n.capacity = capacity;
    n.counts = reinterpret_cast<int32_t *>(base + c.counts);
    n.psum = reinterpret_cast<int32_t *>(base + c.psum);
    n.dst_slot = reinterpret_cast<int32_t *>(base + c.dst);
    n.src_meta = reinterpret_cast<int32_t *>(base + c.src_meta);
    n.scalars = reinterpret_cast<int32_t *>(base + c.scalars);
    n.tile_status = reinterpret_cast<uint64_t *>(base + c.status);
    n.topk_idx = nullptr;
    n.topk_idx_dtype = EP_I64;
    n.status_tiles = static_cast<int32_t>(c.tiles);
    n.recv_row = reinterpret_cast<int32_t *>(base + c.recv_row);
    n.recv_src = reinterpret_cast<int32_t *>(base + c.recv_src);
    const hipError_t e = ep::launch_handle_clear(n.scalars, n.tile_status,
                                                 c.tiles * static_cast<int64_t>(E + 2), stream);
    if (e != hipSuccess) return EP_ERR_HIP;
    *h = n;
    return EP_OK;
}

ep_status ep_time_next_call(hipEvent_t start, hipEvent_t stop) {
    g_next_events.start = start;
    g_next_events.stop = stop;
    return EP_OK;
}

// Checks of a layout call and its kernel arguments (nothing launched).  The
// scans' ticket, epoch and tile status words come from the handle's
// workspace or, for ep_layout_noalloc, from the library's static scratch.
static ep_status layout_prepare(const ep_handle *h, const void *topk_idx, ep_dtype idx_dtype,
                                int32_t num_tokens, int32_t *cumulative_stats,
                                bool static_scratch, ep::LayoutArgs *a) {
    if (!h) return EP_ERR_NULL;
    if (!handle_ready(h)) return EP_ERR_WORKSPACE;
    if (idx_dtype != EP_I64 && idx_dtype != EP_I32) return EP_ERR_DTYPE;
    if (num_tokens < 0 || num_tokens > h->max_tokens) return EP_ERR_SHAPE;
    const int64_t tiles = ep::layout_status_tiles(num_tokens, h->num_topk);
    if (static_scratch) {
        if (tiles * (h->num_experts + 2) > ep::kScratchStatusWords) return EP_ERR_WORKSPACE;
    } else if (tiles > h->status_tiles) {
        return EP_ERR_WORKSPACE;
    }
    if (num_tokens > 0 && !topk_idx) return EP_ERR_NULL;
    if (!aligned(topk_idx, idx_dtype == EP_I64 ? 8 : 4)) return EP_ERR_MISALIGNED;
    if (!aligned(cumulative_stats, 4)) return EP_ERR_MISALIGNED;
    *a = ep::LayoutArgs{};
    a->topk_idx = topk_idx;
    a->idx_is_i64 = idx_dtype == EP_I64;
    a->num_tokens = num_tokens;
    a->num_topk = h->num_topk;
    a->num_experts = h->num_experts;
    a->alignment = h->expert_alignment;
    a->capacity = h->capacity;
    a->counts = h->counts;
    a->psum = h->psum;
    a->dst = h->dst_slot;
    a->src_meta = h->src_meta;
    a->scalars = h->scalars;
    a->tile_status = h->tile_status;
    a->ticket = h->scalars + EP_SCALAR_TICKET;
    a->epoch = h->scalars + EP_SCALAR_EPOCH;
    a->cumulative_stats = cumulative_stats;
    a->recv_row = h->recv_row;
    a->recv_src = h->recv_src;
    return EP_OK;
}

static void layout_done(ep_handle *h, const void *topk_idx, ep_dtype idx_dtype,
                        int32_t num_tokens) {
    h->num_tokens = num_tokens;
    h->topk_idx = topk_idx;
    h->topk_idx_dtype = idx_dtype;
    h->laid_out = 1;
}

static ep_status layout_call(ep_handle *h, const void *topk_idx, ep_dtype idx_dtype,
                             int32_t num_tokens, int32_t *cumulative_stats, hipStream_t stream,
                             bool static_scratch) {
    const ep::CallEvents ev = take_events();
    ep::LayoutArgs a;
    const ep_status st =
        layout_prepare(h, topk_idx, idx_dtype, num_tokens, cumulative_stats, static_scratch, &a);
    if (st != EP_OK) return st;
    if (static_scratch &&
        ep::layout_scratch(stream, &a.tile_status, &a.ticket, &a.epoch) != hipSuccess)
        return EP_ERR_HIP;
    if (ep::launch_layout(a, stream, ev) != hipSuccess) return EP_ERR_HIP;
    layout_done(h, topk_idx, idx_dtype, num_tokens);
    return EP_OK;
}

ep_status ep_layout(ep_handle *h, const void *topk_idx, ep_dtype idx_dtype, int32_t num_tokens,
                    int32_t *cumulative_stats, hipStream_t stream) {
    return layout_call(h, topk_idx, idx_dtype, num_tokens, cumulative_stats, stream, false);
}

ep_status ep_layout_noalloc(ep_handle *h, const void *topk_idx, ep_dtype idx_dtype,
                            int32_t num_tokens, int32_t *cumulative_stats, hipStream_t stream) {
    return layout_call(h, topk_idx, idx_dtype, num_tokens, cumulative_stats, stream, true);
}

ep_status ep_handle_read_counts(const ep_handle *h, int32_t *counts, int32_t *psum,
                                int64_t *num_expanded, int32_t *num_recv_tokens,
                                uint32_t *error_bits, int32_t *invalid_count,
                                hipStream_t stream) {
    if (!h) return EP_ERR_NULL;
    if (!handle_ready(h)) return EP_ERR_WORKSPACE;
    if (!h->laid_out) return EP_ERR_NOT_LAID_OUT;
    int32_t sc[EP_NUM_SCALARS];
    hipError_t e = hipStreamSynchronize(stream);
    if (e == hipSuccess)
        e = hipMemcpy(sc, h->scalars, sizeof(sc), hipMemcpyDeviceToHost);
    if (e == hipSuccess && counts)
        e = hipMemcpy(counts, h->counts, sizeof(int32_t) * h->num_experts, hipMemcpyDeviceToHost);
    if (e == hipSuccess && psum)
        e = hipMemcpy(psum, h->psum, sizeof(int32_t) * (h->num_experts + 1),
                      hipMemcpyDeviceToHost);
    if (e != hipSuccess) return EP_ERR_HIP;
    if (num_expanded) *num_expanded = sc[EP_SCALAR_NUM_EXPANDED];
    if (num_recv_tokens) *num_recv_tokens = sc[EP_SCALAR_NUM_RECV_TOKENS];
    if (error_bits) *error_bits = static_cast<uint32_t>(sc[EP_SCALAR_ERROR_BITS]);
    if (invalid_count) *invalid_count = sc[EP_SCALAR_INVALID_COUNT];
    const uint32_t bits = static_cast<uint32_t>(sc[EP_SCALAR_ERROR_BITS]);
    if (bits & EP_ERRBIT_SCAN_TIMEOUT) return EP_ERR_TIMEOUT;
    if (bits & EP_ERRBIT_CAPACITY) return EP_ERR_CAPACITY;
    if (bits & EP_ERRBIT_INVALID_ID) return EP_ERR_INVALID_ID;
    return EP_OK;
}

ep_status ep_handle_import(ep_handle *h, const void *topk_idx, ep_dtype idx_dtype,
                           int32_t num_tokens, const int32_t *counts, const int32_t *psum,
                           const int32_t *dst_slot, const int32_t *src_meta,
                           int32_t num_recv_tokens, hipStream_t stream) {
    if (!h || !counts || !psum) return EP_ERR_NULL;
    if (!handle_ready(h)) return EP_ERR_WORKSPACE;
    if (idx_dtype != EP_I64 && idx_dtype != EP_I32) return EP_ERR_DTYPE;
    if (num_tokens < 0 || num_tokens > h->max_tokens) return EP_ERR_SHAPE;
    if (num_tokens > 0 && (!topk_idx || !dst_slot)) return EP_ERR_NULL;
    const int32_t E = h->num_experts;
    if (num_tokens == 0 && num_recv_tokens != 0) return EP_ERR_SHAPE;
    const int64_t expanded = psum[E];
    if (expanded < 0 || expanded > h->capacity) return EP_ERR_CAPACITY;
    if (expanded > 0 && !src_meta) return EP_ERR_NULL;
    const int64_t slots = static_cast<int64_t>(num_tokens) * h->num_topk;
    // Every row the kernels will touch must lie inside [0, psum[E]).
    if (psum[0] != 0) return EP_ERR_SHAPE;
    for (int32_t e = 0; e < E; ++e)
        if (counts[e] < 0 || static_cast<int64_t>(psum[e]) + counts[e] > psum[e + 1])
            return EP_ERR_SHAPE;
    for (int64_t i = 0; i < slots; ++i)
        if (dst_slot[i] < -1 || dst_slot[i] >= expanded) return EP_ERR_SHAPE;
    // src_meta must be the inverse of dst_slot: every row of an expert's run
    // names a slot that points back at it and every gap row is -1 (the row
    // copies and combine walk dst_slot; the dispatch's scale copy and the
    // bias gradient walk src_meta).
    int64_t routed = 0;
    for (int64_t i = 0; i < slots; ++i) routed += dst_slot[i] >= 0;
    int64_t runs = 0;
    for (int32_t e = 0; e < E; ++e) {
        for (int64_t r = psum[e]; r < psum[e + 1]; ++r) {
            const int32_t i = src_meta[r];
            if (r < static_cast<int64_t>(psum[e]) + counts[e]) {
                if (i < 0 || i >= slots || dst_slot[i] != r) return EP_ERR_SHAPE;
                ++runs;
            } else if (i != -1) {
                return EP_ERR_SHAPE;
            }
        }
    }
    if (runs != routed) return EP_ERR_SHAPE;
    int32_t sc[3] = {num_recv_tokens, 0, 0};
    const int32_t exp32 = static_cast<int32_t>(expanded);
    hipError_t e = hipStreamSynchronize(stream);
    if (e == hipSuccess)
        e = hipMemcpy(h->counts, counts, sizeof(int32_t) * E, hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = hipMemcpy(h->psum, psum, sizeof(int32_t) * (E + 1), hipMemcpyHostToDevice);
    if (e == hipSuccess && slots)
        e = hipMemcpy(h->dst_slot, dst_slot, sizeof(int32_t) * slots, hipMemcpyHostToDevice);
    if (e == hipSuccess && expanded)
        e = hipMemcpy(h->src_meta, src_meta, sizeof(int32_t) * expanded, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(h->scalars, sc, sizeof(sc), hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = hipMemcpy(h->scalars + EP_SCALAR_NUM_EXPANDED, &exp32, sizeof(exp32),
                      hipMemcpyHostToDevice);
    // The rank layout comes from the device's numbering of the slot rows
    // (tokens with a routed slot, in token order), which also recounts the
    // received tokens into the scalars.
    int32_t recv = 0;
    if (e == hipSuccess && num_tokens > 0)
        e = ep::launch_rank_rows(h->dst_slot, num_tokens, h->num_topk, h->recv_row, h->recv_src,
                                 h->scalars + EP_SCALAR_NUM_RECV_TOKENS, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e == hipSuccess)
        e = hipMemcpy(&recv, h->scalars + EP_SCALAR_NUM_RECV_TOKENS, sizeof(recv),
                      hipMemcpyDeviceToHost);
    if (e == hipSuccess && recv != num_recv_tokens) {
        h->laid_out = 0;
        return EP_ERR_SHAPE;
    }
    if (e != hipSuccess) return EP_ERR_HIP;
    h->num_tokens = num_tokens;
    h->topk_idx = topk_idx;
    h->topk_idx_dtype = idx_dtype;
    h->laid_out = 1;
    return EP_OK;
}

// Scale-pack arguments shared by the two dispatches: returns EP_OK and the
// pack count (0 for bf16) or the status to report.  `reads`: the call reads
// token rows; `writes`: it may write output rows.
static ep_status check_sf(bool fp8, int32_t hidden, const void *sf, const void *out_sf,
                          int32_t num_sf_packs, bool reads, bool writes, int64_t sf_ts,
                          int64_t sf_hs, int64_t out_ts, int64_t out_hs, int32_t *packs) {
    *packs = 0;
    if (!fp8) return (sf || out_sf || num_sf_packs != 0) ? EP_ERR_DTYPE : EP_OK;
    if (num_sf_packs < 0) return EP_ERR_SHAPE;
    const int32_t n = num_sf_packs == 0 ? hidden / 128 : num_sf_packs;
    if (n > 64 * ep::kMaxSfPerLane) return EP_ERR_UNSUPPORTED;
    if ((writes && !out_sf) || (reads && !sf)) return EP_ERR_NULL;
    if (sf_ts < 0 || sf_hs < 0 || out_ts < 0 || out_hs < 0) return EP_ERR_SHAPE;
    if (!aligned(sf, 4) || !aligned(out_sf, 4)) return EP_ERR_MISALIGNED;
    *packs = n;
    return EP_OK;
}

int64_t ep_tma_aligned_rows(int64_t rows) {
    if (rows < 0) return -1;
    return (rows + 3) / 4 * 4;
}

// Checks of a copying dispatch over `num_tokens` tokens of handle h and its
// kernel arguments (nothing launched).
static ep_status dispatch_prepare(const ep_handle *h, int32_t num_tokens, const void *x,
                                  ep_dtype x_dtype, int32_t hidden, const void *sf,
                                  int64_t sf_token_stride, int64_t sf_hidden_stride,
                                  int32_t num_sf_packs, const float *topk_weights, void *out_x,
                                  void *out_sf, int64_t out_sf_token_stride,
                                  int64_t out_sf_hidden_stride, float *out_w,
                                  int32_t flags, ep::DispatchArgs *a) {
    if (flags & ~(EP_DISPATCH_ZERO_PADDING | EP_DISPATCH_STREAMING)) return EP_ERR_UNSUPPORTED;
    const bool zero_padding = (flags & EP_DISPATCH_ZERO_PADDING) != 0;
    if (x_dtype != EP_BF16 && x_dtype != EP_FP8_E4M3) return EP_ERR_DTYPE;
    if (hidden <= 0) return EP_ERR_SHAPE;
    const bool fp8 = x_dtype == EP_FP8_E4M3;
    if (fp8 ? (hidden % 128) != 0 : (hidden % 8) != 0) return EP_ERR_MISALIGNED;
    // With no tokens nothing is read, and only zero padding can write (the
    // gap rows of an imported layout, inside the capacity).
    const bool reads = num_tokens > 0;
    const bool writes = reads || (zero_padding && h->capacity > 0);
    int32_t packs = 0;
    const ep_status st = check_sf(fp8, hidden, sf, out_sf, num_sf_packs, reads, writes,
                                  sf_token_stride, sf_hidden_stride, out_sf_token_stride,
                                  out_sf_hidden_stride, &packs);
    if (st != EP_OK) return st;
    if ((writes && !out_x) || (reads && !x)) return EP_ERR_NULL;
    if (!aligned(x, 16) || !aligned(out_x, 16)) return EP_ERR_MISALIGNED;
    if (!aligned(topk_weights, 4) || !aligned(out_w, 4)) return EP_ERR_MISALIGNED;
    const int64_t row_bytes = fp8 ? hidden : 2 * static_cast<int64_t>(hidden);
    *a = ep::DispatchArgs{};
    a->x = x;
    a->row_vecs = row_bytes / 16;
    a->num_tokens = num_tokens;
    a->num_topk = h->num_topk;
    a->num_experts = h->num_experts;
    a->alignment = h->expert_alignment;
    a->capacity = h->capacity;
    a->dst = h->dst_slot;
    a->counts = h->counts;
    a->psum = h->psum;
    a->scalars = h->scalars;
    a->w = topk_weights;
    a->out_x = out_x;
    a->sf = static_cast<const uint32_t *>(sf);
    a->sf_ts = sf_token_stride;
    a->sf_hs = sf_hidden_stride;
    a->num_sf = packs;
    a->out_sf = static_cast<uint32_t *>(out_sf);
    a->out_ts = out_sf_token_stride;
    a->out_hs = out_sf_hidden_stride;
    a->out_w = out_w;
    a->zero_padding = zero_padding;
    a->streaming = (flags & EP_DISPATCH_STREAMING) != 0;
    a->src_meta = h->src_meta;
    return EP_OK;
}

ep_status ep_dispatch(const ep_handle *h, const void *x, ep_dtype x_dtype, int32_t hidden,
                      const void *sf, int64_t sf_token_stride, int64_t sf_hidden_stride,
                      int32_t num_sf_packs, const float *topk_weights, void *out_x, void *out_sf,
                      int64_t out_sf_token_stride, int64_t out_sf_hidden_stride, float *out_w,
                      int32_t flags, hipStream_t stream) {
    const ep::CallEvents ev = take_events();
    if (!h) return EP_ERR_NULL;
    if (!handle_ready(h)) return EP_ERR_WORKSPACE;
    if (!h->laid_out) return EP_ERR_NOT_LAID_OUT;
    ep::DispatchArgs a;
    const ep_status st = dispatch_prepare(h, h->num_tokens, x, x_dtype, hidden, sf,
                                          sf_token_stride, sf_hidden_stride, num_sf_packs,
                                          topk_weights, out_x, out_sf, out_sf_token_stride,
                                          out_sf_hidden_stride, out_w, flags, &a);
    if (st != EP_OK) return st;
    return hip_status(ep::launch_dispatch(a, stream, ev));
}

ep_status ep_layout_dispatch(ep_handle *h, const void *topk_idx, ep_dtype idx_dtype,
                             int32_t num_tokens, int32_t *cumulative_stats, const void *x,
                             ep_dtype x_dtype, int32_t hidden, const void *sf,
                             int64_t sf_token_stride, int64_t sf_hidden_stride,
                             int32_t num_sf_packs, const float *topk_weights, void *out_x,
                             void *out_sf, int64_t out_sf_token_stride,
                             int64_t out_sf_hidden_stride, float *out_w, int32_t flags,
                             hipStream_t stream) {
    const ep::CallEvents ev = take_events();
    ep::LayoutArgs la;
    ep_status st = layout_prepare(h, topk_idx, idx_dtype, num_tokens, cumulative_stats, false, &la);
    if (st != EP_OK) return st;
    ep::DispatchArgs da;
    st = dispatch_prepare(h, num_tokens, x, x_dtype, hidden, sf, sf_token_stride,
                          sf_hidden_stride, num_sf_packs, topk_weights, out_x, out_sf,
                          out_sf_token_stride, out_sf_hidden_stride, out_w, flags, &da);
    if (st != EP_OK) return st;
    ep::CallEvents first, last;
    first.start = ev.start;
    last.stop = ev.stop;
    if (ep::launch_layout(la, stream, first) != hipSuccess) return EP_ERR_HIP;
    layout_done(h, topk_idx, idx_dtype, num_tokens);
    return hip_status(ep::launch_dispatch(da, stream, last));
}

int32_t ep_sf_packs(int32_t hidden, ep_sf_format fmt) {
    if (hidden <= 0 || hidden % 128 != 0) return -1;
    if (fmt == EP_SF_F32) return hidden / 128;
    if (fmt == EP_SF_UE8M0) return (hidden / 128 + 3) / 4;
    return -1;
}

// Shared checks of the two quantising calls; fills the copy-free fields.
static ep_status quant_args(const void *x, int32_t hidden, ep_sf_format fmt, const void *out_x,
                            const void *out_sf, int64_t ts, int64_t hs, bool reads, bool writes,
                            ep::DispatchArgs *a) {
    if (fmt != EP_SF_F32 && fmt != EP_SF_UE8M0) return EP_ERR_DTYPE;
    if (hidden <= 0) return EP_ERR_SHAPE;
    if (hidden % 128 != 0) return EP_ERR_MISALIGNED;
    if (ts < 0 || hs < 0) return EP_ERR_SHAPE;
    if ((reads && !x) || (writes && (!out_x || !out_sf))) return EP_ERR_NULL;
    if (!aligned(x, 16) || !aligned(out_x, 16) || !aligned(out_sf, 4)) return EP_ERR_MISALIGNED;
    a->x = x;
    a->row_vecs = hidden / 16;
    a->out_x = const_cast<void *>(out_x);
    a->num_sf = ep_sf_packs(hidden, fmt);
    a->out_sf = static_cast<uint32_t *>(const_cast<void *>(out_sf));
    a->out_ts = ts;
    a->out_hs = hs;
    a->quant = static_cast<int32_t>(fmt) + 1;
    return EP_OK;
}

ep_status ep_quantize_fp8(const void *x, int32_t num_tokens, int32_t hidden, ep_sf_format fmt,
                          void *out_q, void *out_sf, int64_t out_sf_token_stride,
                          int64_t out_sf_hidden_stride, hipStream_t stream) {
    const ep::CallEvents ev = take_events();
    if (num_tokens < 0) return EP_ERR_SHAPE;
    ep::DispatchArgs a{};
    const ep_status st = quant_args(x, hidden, fmt, out_q, out_sf, out_sf_token_stride,
                                    out_sf_hidden_stride, num_tokens > 0, num_tokens > 0, &a);
    if (st != EP_OK) return st;
    a.num_tokens = num_tokens;
    a.num_topk = 1;
    a.alignment = 1;
    a.capacity = num_tokens;          // one destination row per token: its own
    return hip_status(ep::launch_dispatch(a, stream, ev));
}

ep_status ep_dispatch_quant(const ep_handle *h, const void *x, int32_t hidden, ep_sf_format fmt,
                            const float *topk_weights, void *out_x, void *out_sf,
                            int64_t out_sf_token_stride, int64_t out_sf_hidden_stride,
                            float *out_w, int32_t zero_padding, hipStream_t stream) {
    const ep::CallEvents ev = take_events();
    if (!h) return EP_ERR_NULL;
    if (!handle_ready(h)) return EP_ERR_WORKSPACE;
    if (!h->laid_out) return EP_ERR_NOT_LAID_OUT;
    ep::DispatchArgs a{};
    const bool reads = h->num_tokens > 0;
    const bool writes = reads || (zero_padding != 0 && h->capacity > 0);
    const ep_status st = quant_args(x, hidden, fmt, out_x, out_sf, out_sf_token_stride,
                                    out_sf_hidden_stride, reads, writes, &a);
    if (st != EP_OK) return st;
    if (!aligned(topk_weights, 4) || !aligned(out_w, 4)) return EP_ERR_MISALIGNED;
    a.num_tokens = h->num_tokens;
    a.num_topk = h->num_topk;
    a.num_experts = h->num_experts;
    a.alignment = h->expert_alignment;
    a.capacity = h->capacity;
    a.dst = h->dst_slot;
    a.counts = h->counts;
    a.psum = h->psum;
    a.scalars = h->scalars;
    a.w = topk_weights;
    a.out_w = out_w;
    a.zero_padding = zero_padding != 0;
    return hip_status(ep::launch_dispatch(a, stream, ev));
}

ep_status ep_combine(const ep_handle *h, const void *y, ep_dtype y_dtype, int32_t hidden,
                     const float *topk_weights, const void *bias, const void *bias_0,
                     const void *bias_1, void *out, hipStream_t stream) {
    const ep::CallEvents ev = take_events();
    if (!h) return EP_ERR_NULL;
    if (!handle_ready(h)) return EP_ERR_WORKSPACE;
    if (!h->laid_out) return EP_ERR_NOT_LAID_OUT;
    if (y_dtype != EP_BF16) return EP_ERR_DTYPE;
    if (hidden <= 0) return EP_ERR_SHAPE;
    if (hidden % 8 != 0) return EP_ERR_MISALIGNED;
    if (h->num_tokens > 0 && (!y || !out)) return EP_ERR_NULL;
    if (bias && h->num_tokens > 0 && !h->topk_idx) return EP_ERR_NULL;
    if (!aligned(y, 16) || !aligned(out, 16) || !aligned(bias, 16) || !aligned(bias_0, 16) ||
        !aligned(bias_1, 16))
        return EP_ERR_MISALIGNED;
    if (!aligned(topk_weights, 4)) return EP_ERR_MISALIGNED;
    ep::CombineArgs a{};
    a.y = y;
    a.row_vecs = hidden / 8;
    a.num_tokens = h->num_tokens;
    a.num_topk = h->num_topk;
    a.num_experts = h->num_experts;
    a.capacity = h->capacity;
    a.dst = h->dst_slot;
    a.scalars = h->scalars;
    a.w = topk_weights;
    a.bias = bias;
    a.topk_idx = h->topk_idx;
    a.idx_is_i64 = h->topk_idx_dtype == EP_I64;
    a.bias_0 = bias_0;
    a.bias_1 = bias_1;
    a.out = out;
    return hip_status(ep::launch_combine(a, stream, ev));
}

ep_status ep_combine_backward(const ep_handle *h, const void *grad_out, int32_t hidden,
                              const float *topk_weights, const void *y, const void *bias,
                              void *grad_y, float *grad_topk_weights, float *grad_bias,
                              hipStream_t stream) {
    const ep::CallEvents ev = take_events();
    if (!h) return EP_ERR_NULL;
    if (!handle_ready(h)) return EP_ERR_WORKSPACE;
    if (!h->laid_out) return EP_ERR_NOT_LAID_OUT;
    if (hidden <= 0) return EP_ERR_SHAPE;
    if (hidden % 8 != 0) return EP_ERR_MISALIGNED;
    const bool rows = h->num_tokens > 0;
    if ((grad_y || grad_topk_weights || grad_bias) && rows && !grad_out) return EP_ERR_NULL;
    if (grad_topk_weights && rows && !y) return EP_ERR_NULL;
    if (bias && grad_topk_weights && rows && !h->topk_idx) return EP_ERR_NULL;
    if (!aligned(grad_out, 16) || !aligned(y, 16) || !aligned(bias, 16) || !aligned(grad_y, 16))
        return EP_ERR_MISALIGNED;
    if (!aligned(topk_weights, 4) || !aligned(grad_topk_weights, 4) || !aligned(grad_bias, 4))
        return EP_ERR_MISALIGNED;
    ep::BackwardArgs a{};
    a.g = grad_out;
    a.row_vecs = hidden / 8;
    a.num_tokens = h->num_tokens;
    a.num_topk = h->num_topk;
    a.num_experts = h->num_experts;
    a.capacity = h->capacity;
    a.dst = h->dst_slot;
    a.counts = h->counts;
    a.psum = h->psum;
    a.src_meta = h->src_meta;
    a.scalars = h->scalars;
    a.w = topk_weights;
    a.y = y;
    a.bias = bias;
    a.topk_idx = h->topk_idx;
    a.idx_is_i64 = h->topk_idx_dtype == EP_I64;
    a.grad_y = grad_y;
    a.grad_w = grad_topk_weights;
    a.grad_bias = grad_bias;
    return hip_status(ep::launch_combine_backward(a, stream, ev));
}

ep_status ep_dispatch_backward(const ep_handle *h, const void *grad_out_x, int32_t hidden,
                               const float *grad_out_w, void *grad_x, float *grad_topk_weights,
                               hipStream_t stream) {
    const ep::CallEvents ev = take_events();
    if (!h) return EP_ERR_NULL;
    if (!handle_ready(h)) return EP_ERR_WORKSPACE;
    if (!h->laid_out) return EP_ERR_NOT_LAID_OUT;
    if (hidden <= 0) return EP_ERR_SHAPE;
    if (hidden % 8 != 0) return EP_ERR_MISALIGNED;
    const bool rows = h->num_tokens > 0;
    if (grad_x && rows && !grad_out_x) return EP_ERR_NULL;
    if (!aligned(grad_out_x, 16) || !aligned(grad_x, 16)) return EP_ERR_MISALIGNED;
    if (!aligned(grad_out_w, 4) || !aligned(grad_topk_weights, 4)) return EP_ERR_MISALIGNED;
    const bool both = grad_x && grad_topk_weights && rows;
    if (grad_x && rows) {
        ep::CombineArgs c{};
        c.y = grad_out_x;
        c.row_vecs = hidden / 8;
        c.num_tokens = h->num_tokens;
        c.num_topk = h->num_topk;
        c.num_experts = h->num_experts;
        c.capacity = h->capacity;
        c.dst = h->dst_slot;
        c.scalars = h->scalars;
        c.out = grad_x;
        ep::CallEvents first = ev;
        if (both) first.stop = nullptr;
        const hipError_t e = ep::launch_combine(c, stream, first);
        if (e != hipSuccess) return EP_ERR_HIP;
    }
    if (grad_topk_weights && rows) {
        ep::GatherArgs g{};
        g.row_values = grad_out_w;
        g.num_slots = static_cast<int64_t>(h->num_tokens) * h->num_topk;
        g.capacity = h->capacity;
        g.dst = h->dst_slot;
        g.scalars = h->scalars;
        g.out = grad_topk_weights;
        ep::CallEvents second = ev;
        if (both) second.start = nullptr;
        return hip_status(ep::launch_gather_rows(g, stream, second));
    }
    return EP_OK;
}

ep_status ep_dispatch_rank(const ep_handle *h, const void *x, ep_dtype x_dtype, int32_t hidden,
                           const void *sf, int64_t sf_token_stride, int64_t sf_hidden_stride,
                           int32_t num_sf_packs, const float *topk_weights, void *out_x,
                           void *out_sf, int64_t out_sf_token_stride,
                           int64_t out_sf_hidden_stride, void *out_topk_idx,
                           float *out_topk_weights, hipStream_t stream) {
    const ep::CallEvents ev = take_events();
    if (!h) return EP_ERR_NULL;
    if (!handle_ready(h)) return EP_ERR_WORKSPACE;
    if (!h->laid_out) return EP_ERR_NOT_LAID_OUT;
    if (x_dtype != EP_BF16 && x_dtype != EP_FP8_E4M3) return EP_ERR_DTYPE;
    if (hidden <= 0) return EP_ERR_SHAPE;
    const bool fp8 = x_dtype == EP_FP8_E4M3;
    if (fp8 ? (hidden % 128) != 0 : (hidden % 8) != 0) return EP_ERR_MISALIGNED;
    const bool rows = h->num_tokens > 0;
    int32_t packs = 0;
    const ep_status st = check_sf(fp8, hidden, sf, out_sf, num_sf_packs, rows, rows,
                                  sf_token_stride, sf_hidden_stride, out_sf_token_stride,
                                  out_sf_hidden_stride, &packs);
    if (st != EP_OK) return st;
    if (rows && (!out_x || !x)) return EP_ERR_NULL;
    if ((out_topk_idx || out_topk_weights) && rows && !h->topk_idx) return EP_ERR_NULL;
    if (!aligned(x, 16) || !aligned(out_x, 16)) return EP_ERR_MISALIGNED;
    if (!aligned(topk_weights, 4) || !aligned(out_topk_weights, 4) ||
        !aligned(out_topk_idx, h->topk_idx_dtype == EP_I64 ? 8 : 4))
        return EP_ERR_MISALIGNED;
    ep::RankArgs a{};
    a.x = x;
    a.row_vecs = (fp8 ? hidden : 2 * static_cast<int64_t>(hidden)) / 16;
    a.num_tokens = h->num_tokens;
    a.num_topk = h->num_topk;
    a.num_experts = h->num_experts;
    a.recv_row = h->recv_row;
    a.scalars = h->scalars;
    a.topk_idx = h->topk_idx;
    a.idx_is_i64 = h->topk_idx_dtype == EP_I64;
    a.w = topk_weights;
    a.sf = static_cast<const uint32_t *>(sf);
    a.sf_ts = sf_token_stride;
    a.sf_hs = sf_hidden_stride;
    a.num_sf = packs;
    a.out = out_x;
    a.out_sf = static_cast<uint32_t *>(out_sf);
    a.out_ts = out_sf_token_stride;
    a.out_hs = out_sf_hidden_stride;
    a.out_idx = out_topk_idx;
    a.out_w = out_topk_weights;
    return hip_status(ep::launch_dispatch_rank(a, stream, ev));
}

ep_status ep_dispatch_rank_quant(const ep_handle *h, const void *x, int32_t hidden,
                                 ep_sf_format fmt, const float *topk_weights, void *out_x,
                                 void *out_sf, int64_t out_sf_token_stride,
                                 int64_t out_sf_hidden_stride, void *out_topk_idx,
                                 float *out_topk_weights, hipStream_t stream) {
    const ep::CallEvents ev = take_events();
    if (!h) return EP_ERR_NULL;
    if (!handle_ready(h)) return EP_ERR_WORKSPACE;
    if (!h->laid_out) return EP_ERR_NOT_LAID_OUT;
    const bool rows = h->num_tokens > 0;
    ep::DispatchArgs a{};
    const ep_status st = quant_args(x, hidden, fmt, out_x, out_sf, out_sf_token_stride,
                                    out_sf_hidden_stride, rows, rows, &a);
    if (st != EP_OK) return st;
    const bool meta = out_topk_idx || out_topk_weights;
    if (meta && rows && !h->topk_idx) return EP_ERR_NULL;
    if (!aligned(topk_weights, 4) || !aligned(out_topk_weights, 4) ||
        !aligned(out_topk_idx, h->topk_idx_dtype == EP_I64 ? 8 : 4))
        return EP_ERR_MISALIGNED;
    if (!rows) return EP_OK;
    // The quantising dispatch with one destination per token, its rank row
    // (or none); the wave that quantises a row's first pass also writes the
    // row's received ids and weights.  Like the copying rank dispatch it
    // stops only on a scan timeout (the rank layout does not depend on
    // capacity).
    a.num_tokens = h->num_tokens;
    a.num_topk = 1;
    a.num_experts = h->num_experts;
    a.alignment = 1;
    a.capacity = h->num_tokens;             // rank rows lie in [0, num_tokens)
    a.dst = h->recv_row;
    a.scalars = h->scalars;
    a.stop_bits = EP_ERRBIT_SCAN_TIMEOUT;
    if (meta) {
        a.meta_idx = h->topk_idx;
        a.meta_i64 = h->topk_idx_dtype == EP_I64;
        a.meta_topk = h->num_topk;
        a.meta_w = topk_weights;
        a.out_meta_idx = out_topk_idx;
        a.out_meta_w = out_topk_weights;
    }
    return hip_status(ep::launch_dispatch(a, stream, ev));
}

ep_status ep_combine_rank(const ep_handle *h, const void *x, int32_t hidden, const void *bias_0,
                          const void *bias_1, void *out, hipStream_t stream) {
    const ep::CallEvents ev = take_events();
    if (!h) return EP_ERR_NULL;
    if (!handle_ready(h)) return EP_ERR_WORKSPACE;
    if (!h->laid_out) return EP_ERR_NOT_LAID_OUT;
    if (hidden <= 0) return EP_ERR_SHAPE;
    if (hidden % 8 != 0) return EP_ERR_MISALIGNED;
    if (h->num_tokens > 0 && (!x || !out)) return EP_ERR_NULL;
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(bias_0, 16) || !aligned(bias_1, 16))
        return EP_ERR_MISALIGNED;
    ep::RankArgs a{};
    a.x = x;
    a.row_vecs = hidden / 8;
    a.num_tokens = h->num_tokens;
    a.num_topk = h->num_topk;
    a.num_experts = h->num_experts;
    a.recv_row = h->recv_row;
    a.scalars = h->scalars;
    a.bias_0 = bias_0;
    a.bias_1 = bias_1;
    a.out = out;
    return hip_status(ep::launch_combine_rank(a, stream, ev));
}

const char *ep_status_str(ep_status s) {
    switch (s) {
    case EP_OK: return "EP_OK: success";
    case EP_ERR_NULL: return "EP_ERR_NULL: a required pointer is NULL";
    case EP_ERR_SHAPE: return "EP_ERR_SHAPE: a size is out of range or inconsistent";
    case EP_ERR_DTYPE: return "EP_ERR_DTYPE: element type not accepted by this call";
    case EP_ERR_UNSUPPORTED:
        return "EP_ERR_UNSUPPORTED: beyond the library's limits (K <= 64, E <= 1024, "
               "capacity and T*K < 2^31)";
    case EP_ERR_MISALIGNED: return "EP_ERR_MISALIGNED: pointer or row size not aligned";
    case EP_ERR_WORKSPACE: return "EP_ERR_WORKSPACE: workspace missing or too small";
    case EP_ERR_NOT_LAID_OUT: return "EP_ERR_NOT_LAID_OUT: no layout on this handle yet";
    case EP_ERR_CAPACITY: return "EP_ERR_CAPACITY: expanded rows exceed the capacity";
    case EP_ERR_INVALID_ID: return "EP_ERR_INVALID_ID: an expert id outside [-1, E) was seen";
    case EP_ERR_HIP: return "EP_ERR_HIP: a HIP call or kernel launch failed";
    case EP_ERR_TIMEOUT:
        return "EP_ERR_TIMEOUT: the layout scan's bounded wait gave up; the layout is void";
    }
    return "unknown ep_status";
}

}  // extern "C"
