// Bandwidth ceilings on gfx950: plain kernels whose only work is the memory
// traffic of a pattern, so the measured fraction of each layout / dispatch /
// combine call can be read against what HBM (and the MALL in front of it)
// gives for the same access pattern, not only against the 8 TB/s peak.
//
// Built into its own library (libep_ceilings.so) for the benchmark; the
// product library does not use it.  The patterns:
//   read        sequential 16-byte loads of a buffer (folded into one word per
//               block so no load is dead)
//   write       sequential 16-byte stores of a constant
//   copy        sequential loads and stores, 1:1
//   row_store   the dispatch's store pattern without its loads: one wave per
//               (token, 1 KB pass of a row) stores a constant to each of the
//               token's slot rows given by a slot -> row table (rows of the
//               expanded layout in the order the dispatch writes them), with
//               ordinary or non-temporal stores as the dispatch can
//   gather      the combine's pattern without its arithmetic: one thread per
//               (token, 16-byte column) loads that column of each of the
//               token's K slot rows, XORs them and stores one vector (K reads
//               per write: 8:1 at top-8)
//   empty       a grid that does nothing (the floor of a timed launch)
// Page: DeepEP notes ch.7 "V2: how dispatch builds expert inputs", s7.4 (the
// copy / permute the expanded layout costs) names the traffic being bounded.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ep_ceilings.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                  hipEvent_t start, hipEvent_t stop, Args... args) {
    if (start || stop)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, start, stop, 0u, args...);
    else
        kernel<<<grid, block, 0, stream>>>(args...);
    return hipGetLastError();
}

template <bool NT>
__device__ inline u32x4 load16(const u32x4 *p) {
    if (NT) return __builtin_nontemporal_load(p);
    return *p;
}

template <bool NT>
__device__ inline void store16(u32x4 *p, u32x4 v) {
    if (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// The sequential kernels: a block covers kThreads * VPT consecutive vectors
// per round (each thread VPT of them, kThreads apart, all requested before
// any is used); rounds stride over the buffer by the grid.
template <int VPT, bool NT>
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4 *src, int64_t n,
                                                        uint32_t *sink) {
    const int64_t span = static_cast<int64_t>(kThreads) * VPT;
    uint32_t x = 0;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * span + threadIdx.x; base < n;
         base += static_cast<int64_t>(gridDim.x) * span) {
        u32x4 v[VPT];
#pragma unroll
        for (int q = 0; q < VPT; ++q) {
            const int64_t i = base + static_cast<int64_t>(q) * kThreads;
            v[q] = i < n ? load16<NT>(src + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int q = 0; q < VPT; ++q) x ^= v[q].x ^ v[q].y ^ v[q].z ^ v[q].w;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off, 64);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = x;
}

template <int VPT, bool NT>
__global__ __launch_bounds__(kThreads) void write_kernel(u32x4 *dst, int64_t n, uint32_t value) {
    const int64_t span = static_cast<int64_t>(kThreads) * VPT;
    const u32x4 v = u32x4{value, value, value, value};
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * span + threadIdx.x; base < n;
         base += static_cast<int64_t>(gridDim.x) * span) {
#pragma unroll
        for (int q = 0; q < VPT; ++q) {
            const int64_t i = base + static_cast<int64_t>(q) * kThreads;
            if (i < n) store16<NT>(dst + i, v);
        }
    }
}

template <int VPT, bool NT>
__global__ __launch_bounds__(kThreads) void copy_kernel(u32x4 *dst, const u32x4 *src,
                                                        int64_t n) {
    const int64_t span = static_cast<int64_t>(kThreads) * VPT;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * span + threadIdx.x; base < n;
         base += static_cast<int64_t>(gridDim.x) * span) {
        u32x4 v[VPT];
#pragma unroll
        for (int q = 0; q < VPT; ++q) {
            const int64_t i = base + static_cast<int64_t>(q) * kThreads;
            if (i < n) v[q] = load16<NT>(src + i);
        }
#pragma unroll
        for (int q = 0; q < VPT; ++q) {
            const int64_t i = base + static_cast<int64_t>(q) * kThreads;
            if (i < n) store16<NT>(dst + i, v[q]);
        }
    }
}

// Grid of a sequential kernel: `blocks` > 0 caps it (the rounds then
// stride), 0 gives one round per block.
int64_t seq_blocks(int64_t n, int vpt, int32_t blocks) {
    const int64_t span = static_cast<int64_t>(kThreads) * vpt;
    const int64_t rounds = (n + span - 1) / span;
    return blocks > 0 && blocks < rounds ? blocks : rounds;
}

// Dispatch on the tunables: vectors per thread (1, 2, 4, 8, 16) and
// non-temporal access.
template <template <int, bool> class Pick, typename... Args>
hipError_t seq_launch(int vpt, bool nt, int64_t blocks, hipStream_t stream, hipEvent_t start,
                      hipEvent_t stop, Args... args) {
    const dim3 g(static_cast<unsigned>(blocks)), b(kThreads);
#define EPC_CASE(V)                                                                          \
    if (vpt == V)                                                                            \
        return nt ? launch(Pick<V, true>::fn(), g, b, stream, start, stop, args...)          \
                  : launch(Pick<V, false>::fn(), g, b, stream, start, stop, args...);
    EPC_CASE(1) EPC_CASE(2) EPC_CASE(4) EPC_CASE(8) EPC_CASE(16)
#undef EPC_CASE
    return hipErrorInvalidValue;
}

template <int V, bool NT> struct PickRead {
    static auto fn() { return &read_kernel<V, NT>; }
};
template <int V, bool NT> struct PickWrite {
    static auto fn() { return &write_kernel<V, NT>; }
};
template <int V, bool NT> struct PickCopy {
    static auto fn() { return &copy_kernel<V, NT>; }
};

bool valid_vpt(int32_t v) { return v == 1 || v == 2 || v == 4 || v == 8 || v == 16; }

// One wave per (token, pass of 64 vectors): the token's K slot rows (-1 or
// rows outside [0, rows) skipped) each get the pass stored.
template <bool NT>
__global__ __launch_bounds__(kThreads) void row_store_kernel(u32x4 *dst, const int32_t *slot_row,
                                                             int64_t tokens, int K,
                                                             int64_t row_vecs, int64_t rows,
                                                             int passes) {
    const int lane = threadIdx.x & 63;
    const int64_t wv = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
    const int64_t t = wv / passes;
    if (t >= tokens) return;
    const int64_t c = (wv - t * passes) * 64 + lane;
    int32_t my_row = lane < K ? slot_row[t * K + lane] : -1;
    if (my_row >= rows) my_row = -1;
    const u32x4 v = u32x4{static_cast<uint32_t>(t), 1u, 2u, 3u};
    for (int k = 0; k < K; ++k) {
        const int32_t r = __builtin_amdgcn_readlane(my_row, k);
        if (r < 0) continue;
        if (c >= row_vecs) continue;
        u32x4 *p = dst + static_cast<int64_t>(r) * row_vecs + c;
        if constexpr (NT)
            __builtin_nontemporal_store(v, p);
        else
            *p = v;
    }
}

// One thread per (token, 16-byte column): XOR of that column over the
// token's slot rows (non-temporal loads, as the combine's expert rows),
// stored to the token's output row.
__global__ __launch_bounds__(kThreads) void gather_kernel(u32x4 *out, const u32x4 *in,
                                                          const int32_t *slot_row, int64_t tokens,
                                                          int K, int64_t row_vecs, int64_t rows) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const int64_t t = gid / row_vecs;
    if (t >= tokens) return;
    const int64_t c = gid - t * row_vecs;
    u32x4 acc = u32x4{0u, 0u, 0u, 0u};
    for (int k0 = 0; k0 < K; k0 += 8) {
        u32x4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int32_t r = k0 + j < K ? slot_row[t * K + k0 + j] : -1;
            v[j] = (r >= 0 && r < rows)
                       ? __builtin_nontemporal_load(in + static_cast<int64_t>(r) * row_vecs + c)
                       : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) acc ^= v[j];
    }
    __builtin_nontemporal_store(acc, out + t * row_vecs + c);
}

// Does nothing: the floor of a launch timed by events on its dispatch.
__global__ void empty_kernel() {}

int status(hipError_t e) { return e == hipSuccess ? 0 : static_cast<int>(e); }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

int64_t epc_read_sink_words(size_t bytes, int32_t vec_per_thread, int32_t blocks) {
    if (!valid_vpt(vec_per_thread) || blocks < 0) return -1;
    return seq_blocks(static_cast<int64_t>(bytes / 16), vec_per_thread, blocks) * (kThreads / 64);
}

int epc_read(const void *src, size_t bytes, uint32_t *sink, int32_t vec_per_thread,
             int32_t blocks, int32_t nontemporal, hipStream_t stream, hipEvent_t start,
             hipEvent_t stop) {
    if ((bytes & 15u) || !aligned16(src) || (bytes && (!src || !sink)) ||
        !valid_vpt(vec_per_thread) || blocks < 0)
        return -1;
    const int64_t n = static_cast<int64_t>(bytes / 16);
    const int64_t g = seq_blocks(n, vec_per_thread, blocks);
    if (g == 0 || g > INT32_MAX) return g == 0 ? 0 : -1;
    return status(seq_launch<PickRead>(vec_per_thread, nontemporal != 0, g, stream, start, stop,
                                       static_cast<const u32x4 *>(src), n, sink));
}

int epc_write(void *dst, size_t bytes, uint32_t value, int32_t vec_per_thread, int32_t blocks,
              int32_t nontemporal, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    if ((bytes & 15u) || !aligned16(dst) || (bytes && !dst) || !valid_vpt(vec_per_thread) ||
        blocks < 0)
        return -1;
    const int64_t n = static_cast<int64_t>(bytes / 16);
    const int64_t g = seq_blocks(n, vec_per_thread, blocks);
    if (g == 0 || g > INT32_MAX) return g == 0 ? 0 : -1;
    return status(seq_launch<PickWrite>(vec_per_thread, nontemporal != 0, g, stream, start, stop,
                                        static_cast<u32x4 *>(dst), n, value));
}

int epc_copy(void *dst, const void *src, size_t bytes, int32_t vec_per_thread, int32_t blocks,
             int32_t nontemporal, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    if ((bytes & 15u) || !aligned16(dst) || !aligned16(src) || (bytes && (!dst || !src)) ||
        !valid_vpt(vec_per_thread) || blocks < 0)
        return -1;
    const int64_t n = static_cast<int64_t>(bytes / 16);
    const int64_t g = seq_blocks(n, vec_per_thread, blocks);
    if (g == 0 || g > INT32_MAX) return g == 0 ? 0 : -1;
    return status(seq_launch<PickCopy>(vec_per_thread, nontemporal != 0, g, stream, start, stop,
                                       static_cast<u32x4 *>(dst),
                                       static_cast<const u32x4 *>(src), n));
}

int epc_row_store(void *dst, int64_t rows, int64_t row_bytes, const int32_t *slot_row,
                  int64_t tokens, int32_t K, int32_t nontemporal, hipStream_t stream,
                  hipEvent_t start, hipEvent_t stop) {
    if (rows < 0 || tokens < 0 || K < 1 || K > 64 || row_bytes <= 0 || (row_bytes & 15) ||
        !aligned16(dst) || (tokens && (!dst || !slot_row)))
        return -1;
    const int64_t row_vecs = row_bytes / 16;
    const int64_t passes = (row_vecs + 63) / 64;
    const int64_t blocks = (tokens * passes + kThreads / 64 - 1) / (kThreads / 64);
    if (blocks == 0 || blocks > INT32_MAX) return blocks == 0 ? 0 : -1;
    auto kernel = nontemporal ? row_store_kernel<true> : row_store_kernel<false>;
    return status(launch(kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), stream,
                         start, stop, static_cast<u32x4 *>(dst), slot_row, tokens,
                         static_cast<int>(K), row_vecs, rows, static_cast<int>(passes)));
}

int epc_gather(void *out, const void *in, int64_t rows, int64_t row_bytes,
               const int32_t *slot_row, int64_t tokens, int32_t K, hipStream_t stream,
               hipEvent_t start, hipEvent_t stop) {
    if (rows < 0 || tokens < 0 || K < 1 || K > 64 || row_bytes <= 0 || (row_bytes & 15) ||
        !aligned16(out) || !aligned16(in) || (tokens && (!out || !in || !slot_row)))
        return -1;
    const int64_t row_vecs = row_bytes / 16;
    const int64_t blocks = (tokens * row_vecs + kThreads - 1) / kThreads;
    if (blocks == 0 || blocks > INT32_MAX) return blocks == 0 ? 0 : -1;
    return status(launch(gather_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                         stream, start, stop, static_cast<u32x4 *>(out),
                         static_cast<const u32x4 *>(in), slot_row, tokens, static_cast<int>(K),
                         row_vecs, rows));
}

int epc_empty(int32_t blocks, int32_t threads, hipStream_t stream, hipEvent_t start,
              hipEvent_t stop) {
    if (blocks < 1 || threads < 1 || threads > 1024) return -1;
    return status(launch(empty_kernel, dim3(static_cast<unsigned>(blocks)),
                         dim3(static_cast<unsigned>(threads)), stream, start, stop));
}

}  // extern "C"
