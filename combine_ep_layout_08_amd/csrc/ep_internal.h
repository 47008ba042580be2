// Internal declarations shared by the library's translation units.
// Not installed; the public interface is include/ep.h.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

// 16-byte vector as a native clang vector (usable with the nontemporal
// load/store builtins, which lower to global_load/store_dwordx4 ... nt).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Layout scan: one tile is kLayoutThreads threads x kLayoutRounds rounds of
// 64 consecutive slots per wave.
constexpr int kLayoutThreads = 256;
constexpr int kLayoutWaves = kLayoutThreads / 64;
constexpr int kLayoutRounds = 8;
constexpr int kTileSlots = kLayoutThreads * kLayoutRounds;   // 2048
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopk = 64;
constexpr int kMaxBuckets = kMaxExperts + 1;                 // + invalid-id bucket
constexpr int kMaxSfPerLane = 4;                             // FP8 hidden <= 32768

inline int64_t layout_tiles(int64_t num_slots) {
    int64_t t = (num_slots + kTileSlots - 1) / kTileSlots;
    return t < 1 ? 1 : t;
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
    int32_t *cumulative_stats;
};

struct DispatchArgs {
    const void *x;
    int64_t row_vecs;            // 16-byte vectors per row
    int32_t num_tokens, num_topk, num_experts, alignment;
    int64_t capacity;            // rows of out_x / out_sf / out_w
    const int32_t *dst, *counts, *psum, *scalars;
    const float *w;
    void *out_x;
    const float *sf;
    int64_t sf_ts, sf_hs;
    int32_t num_sf;
    float *out_sf;
    int64_t out_ts, out_hs;
    float *out_w;
    bool zero_padding;
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
    void *out;
};

hipError_t launch_handle_clear(int32_t *scalars, uint64_t *tile_status,
                               int64_t status_words, hipStream_t stream);
hipError_t launch_layout(const LayoutArgs &a, hipStream_t stream, CallEvents ev);
hipError_t launch_dispatch(const DispatchArgs &a, hipStream_t stream, CallEvents ev);
hipError_t launch_combine(const CombineArgs &a, hipStream_t stream, CallEvents ev);

}  // namespace ep
