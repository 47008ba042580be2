// Internal declarations shared by the library's translation units.
// Not installed; the public interface is include/ep.h.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ep.h"

namespace ep {

// 16-byte vector as a native clang vector (usable with the nontemporal
// load/store builtins, which lower to global_load/store_dwordx4 ... nt).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Layout tiles: kLayoutThreads threads x R rounds of 64 consecutive slots per
// wave, always whole tokens.  Batches that fit in kSmallTilesMax tiles of
// kRoundsSmall rounds use those short tiles (more blocks share the ranking);
// larger batches use kRoundsLarge rounds (fewer tiles' counts to sum).
constexpr int kLayoutThreads = 256;
constexpr int kLayoutWaves = kLayoutThreads / 64;
constexpr int kRoundsSmall = 4;
constexpr int kRoundsLarge = 8;
constexpr int kSmallTilesMax = 64;
constexpr int kTileSlots = kLayoutThreads * kRoundsLarge;   // the longest tile
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopk = 64;
static_assert(kLayoutThreads * kRoundsSmall >= kMaxTopk, "a tile must hold at least one token");
// Buckets of the scan: experts, then ids outside [-1, E), then received tokens.
constexpr int kMaxBuckets = kMaxExperts + 2;
constexpr int kMaxSfPerLane = 4;                             // FP8 hidden <= 32768

inline int layout_tokens_per_tile(int num_topk, int rounds) {
    const int t = kLayoutThreads * rounds / num_topk;
    return t < 1 ? 1 : t;
}

inline int64_t layout_tiles(int64_t num_tokens, int num_topk, int rounds) {
    const int64_t tpt = layout_tokens_per_tile(num_topk, rounds);
    const int64_t t = (num_tokens + tpt - 1) / tpt;
    return t < 1 ? 1 : t;
}

// Rounds per tile for a batch of num_tokens.
inline int layout_rounds(int64_t num_tokens, int num_topk) {
    return layout_tiles(num_tokens, num_topk, kRoundsSmall) <= kSmallTilesMax ? kRoundsSmall
                                                                               : kRoundsLarge;
}

// Tiles whose status words a handle for up to max_tokens tokens must hold.
inline int64_t layout_status_tiles(int64_t max_tokens, int num_topk) {
    const int64_t small = layout_tiles(max_tokens, num_topk, kRoundsSmall);
    const int64_t large = layout_tiles(max_tokens, num_topk, kRoundsLarge);
    const int64_t s = small < kSmallTilesMax ? small : kSmallTilesMax;
    return s > large ? s : large;
}

// Launch with optional events attached to the kernel dispatch itself
// (AMD's hipExtLaunchKernel): `start` is stamped when the kernel begins and
// `stop` when it ends, so a timed interval holds kernel execution only.
template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                         hipEvent_t start, hipEvent_t stop, Args... args) {
    if (start || stop)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, start, stop, 0u, args...);
    else
        kernel<<<grid, block, 0, stream>>>(args...);
    return hipGetLastError();
}

// Compute units of the current device (cached per device; 256 on MI355X).
inline int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Grid of a persistent kernel: `units` work items, at most blocks_per_cu
// resident blocks per compute unit (0 = one block per unit).
inline int64_t persistent_grid(int64_t units, int blocks_per_cu) {
    if (blocks_per_cu <= 0) return units;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * blocks_per_cu;
    return units < cap ? units : cap;
}

// Events handed to the next entry point by ep_time_next_call (null = none).
struct CallEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

struct LayoutArgs {
    const void *topk_idx;
    bool idx_is_i64;
    int32_t num_tokens, num_topk, num_experts, alignment;
    int64_t capacity;
    int32_t *counts, *psum, *dst, *src_meta, *scalars;
    uint64_t *tile_status;
    // Tile ticket and call epoch of the scans over tile_status (the handle's
    // scalars, or the header of the library's static scratch).
    int32_t *ticket, *epoch;
    int32_t *cumulative_stats;
    int32_t *recv_row, *recv_src;
};

struct DispatchArgs {
    const void *x;
    int64_t row_vecs;            // 16-byte vectors per row
    int32_t num_tokens, num_topk, num_experts, alignment;
    int64_t capacity;            // rows of out_x / out_sf / out_w
    const int32_t *dst, *counts, *psum, *scalars;
    const float *w;
    void *out_x;
    const uint32_t *sf;          // 4-byte scale packs, copied as bits
    int64_t sf_ts, sf_hs;
    int32_t num_sf;              // packs per token
    uint32_t *out_sf;
    int64_t out_ts, out_hs;
    float *out_w;
    bool zero_padding;
    bool streaming;              // non-temporal stores of the copied rows (copying form)
    int32_t quant;               // 0: copy x; EP_SF_F32 + 1 / EP_SF_UE8M0 + 1: quantise bf16 x
    // Source slot of every expanded row (the layout's src_meta): when set, a
    // copying dispatch moves the scale packs and weights in expanded-row
    // order, each row's from its source slot, instead of from the token's
    // first-pass wave.
    const int32_t *src_meta = nullptr;
    uint32_t stop_bits = EP_ERRBIT_FATAL;  // error bits in *scalars that make it write nothing
    // Rank-row metadata (quantising rank dispatch, num_topk 1): the token's
    // meta_topk ids (valid ones, else -1) and weights (valid ones, else 0)
    // go to its one destination row; null outputs skip them.
    const void *meta_idx = nullptr;
    bool meta_i64 = false;
    int32_t meta_topk = 0;
    const float *meta_w = nullptr;
    void *out_meta_idx = nullptr;
    float *out_meta_w = nullptr;
};

struct CombineArgs {
    const void *y;
    int64_t row_vecs;            // 16-byte vectors (8 bf16) per row
    int32_t num_tokens, num_topk, num_experts;
    int64_t capacity;            // rows of y
    const int32_t *dst, *scalars;
    const float *w;
    const void *bias;            // bf16 [E, H] or null
    const void *topk_idx;        // ids, read only when bias is set
    bool idx_is_i64;
    const void *bias_0, *bias_1; // bf16 [T, H] per-token biases or null
    void *out;
};

struct RankArgs {
    const void *x;               // dispatch: [T, H] rows; combine: [rows, H]
    int64_t row_vecs;
    int32_t num_tokens, num_topk, num_experts;
    const int32_t *recv_row, *scalars;
    const void *topk_idx;
    bool idx_is_i64;
    const float *w;
    const uint32_t *sf;          // 4-byte scale packs, copied as bits
    int64_t sf_ts, sf_hs;
    int32_t num_sf;
    void *out;                   // dispatch: [max_tokens, H]; combine: bf16 [T, H]
    uint32_t *out_sf;
    int64_t out_ts, out_hs;
    void *out_idx;               // same dtype as topk_idx
    float *out_w;
    const void *bias_0, *bias_1;
};

struct BackwardArgs {
    const void *g;               // bf16 [T, H] gradient of combine's output
    int64_t row_vecs;            // 16-byte vectors (8 bf16) per row
    int32_t num_tokens, num_topk, num_experts;
    int64_t capacity;
    const int32_t *dst, *counts, *psum, *src_meta, *scalars;
    const float *w;              // [T, K] or null
    const void *y;               // bf16 [capacity, H] (weight gradient)
    const void *bias;            // bf16 [E, H] or null
    const void *topk_idx;
    bool idx_is_i64;
    void *grad_y;                // bf16 [capacity, H] or null
    float *grad_w;               // [T, K] or null
    float *grad_bias;            // [E, H] or null
};

struct GatherArgs {
    const float *row_values;     // [capacity] or null (gathers zeros)
    int64_t num_slots, capacity;
    const int32_t *dst, *scalars;
    float *out;                  // [T, K]
};

hipError_t launch_handle_clear(int32_t *scalars, uint64_t *tile_status,
                               int64_t status_words, hipStream_t stream);
hipError_t launch_layout(const LayoutArgs &a, hipStream_t stream, CallEvents ev);
// Status words of the library's static scratch (ep_layout_noalloc) on the
// current device; set up on the first call per device.
constexpr int64_t kScratchBytes = EP_LAYOUT_SCRATCH_BYTES;
constexpr int64_t kScratchHeaderBytes = 256;
constexpr int64_t kScratchStatusWords = (kScratchBytes - kScratchHeaderBytes) / 8;
hipError_t layout_scratch(hipStream_t stream, uint64_t **status, int32_t **ticket,
                          int32_t **epoch);
hipError_t launch_dispatch(const DispatchArgs &a, hipStream_t stream, CallEvents ev);
hipError_t launch_combine(const CombineArgs &a, hipStream_t stream, CallEvents ev);
hipError_t launch_combine_backward(const BackwardArgs &a, hipStream_t stream, CallEvents ev);
hipError_t launch_gather_rows(const GatherArgs &a, hipStream_t stream, CallEvents ev);
hipError_t launch_dispatch_rank(const RankArgs &a, hipStream_t stream, CallEvents ev);
// Rank rows (recv_row, recv_src) and the received count from a layout's slot
// rows: the tokens with a slot row >= 0, numbered in token order.
hipError_t launch_rank_rows(const int32_t *dst, int64_t num_tokens, int num_topk,
                            int32_t *recv_row, int32_t *recv_src, int32_t *num_recv,
                            hipStream_t stream);
hipError_t launch_combine_rank(const RankArgs &a, hipStream_t stream, CallEvents ev);

}  // namespace ep
