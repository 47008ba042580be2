// Backward of combine and the slot gather used by the backward of dispatch,
// on gfx950.
//
// The DeepEP README's training example pairs the two directions: the
// backward of combine is a dispatch of the output gradient, the backward of
// dispatch is a combine of the gradient rows, and the combined top-k weights
// carry the weights' gradient.  With the combine of this library,
//   out[t] = sum_k w[t,k] * (y[r] + b[e]),   r = dst[t,k], e = topk_idx[t,k],
// and g = d loss / d out (bf16 [T, H]):
//   grad_y[r]      = bf16(fl32(w[t,k] * g[t]))   (g[t] itself without weights)
//   grad_w[t,k]    = sum_h g[t][h] * (y[r][h] + b[e][h])
//   grad_bias[e]   = sum over expert e's rows of w * g[t]
// The two sums are accumulated in binary64, where every term is exact (a
// bf16 times a binary32 or a bf16 sum), and rounded once to binary32: the
// result is the correctly rounded value up to binary64 rounding, whatever
// the order of the partial sums.
//
// Kernels:
//  * combine_backward (row pass): one block per token whose threads tile the
//    row's 16-byte columns (up to 1024 threads, striding beyond).  The
//    gradient is read once; grad_y and the weight gradient come out of the
//    same pass (two separate passes re-read g and did not overlap the y
//    reads with the grad_y writes).  Per chunk of 8 slots, one binary64
//    partial per slot; a shuffle tree and an ordered pass over the waves
//    finish each dot.
//  * bias_grad: one block per (expert, 64 columns); the block's 4 waves take
//    every 4th row of the expert's segment, 8 rows in flight per lane, and
//    the 4 binary64 partials are added in wave order.
//  * gather_rows: one thread per slot, out[t,k] = values[dst[t,k]] (0 if
//    empty): the weight gradient of dispatch's per-row weights.
#include "ep_internal.h"
#include "../../include/ep.h"

namespace ep {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 8;
constexpr int kRsrcWord3 = 0x00020000;   // gfx9 raw buffer, 32-bit format

// Row view whose loads past `bytes` return zero (bytes = 0 for an unused
// slot), so a chunk's loads need no branch.
__device__ inline __amdgpu_buffer_rsrc_t row_rsrc(const void *base, int64_t row, int32_t bytes,
                                                  bool valid) {
    const char *p = static_cast<const char *>(base) + (valid ? row * bytes : 0);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(p), 0, valid ? bytes : 0,
                                             kRsrcWord3);
}

__device__ inline void unpack8(const u32x4 v, float f[8]) {
    f[0] = __uint_as_float(v.x << 16);
    f[1] = __uint_as_float(v.x & 0xFFFF0000u);
    f[2] = __uint_as_float(v.y << 16);
    f[3] = __uint_as_float(v.y & 0xFFFF0000u);
    f[4] = __uint_as_float(v.z << 16);
    f[5] = __uint_as_float(v.z & 0xFFFF0000u);
    f[6] = __uint_as_float(v.w << 16);
    f[7] = __uint_as_float(v.w & 0xFFFF0000u);
}

// binary32 -> bf16 bits, round to nearest, ties to even; NaN -> 0x7FC0.
__device__ inline uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ inline u32x4 scale_bf16x8(const u32x4 v, float s) {
#pragma clang fp contract(off)
    float f[8];
    unpack8(v, f);
    u32x4 o;
    o.x = bf16_rne(s * f[0]) | (bf16_rne(s * f[1]) << 16);
    o.y = bf16_rne(s * f[2]) | (bf16_rne(s * f[3]) << 16);
    o.z = bf16_rne(s * f[4]) | (bf16_rne(s * f[5]) << 16);
    o.w = bf16_rne(s * f[6]) | (bf16_rne(s * f[7]) << 16);
    return o;
}

// Row pass block size: ceil(row vectors / EP_BACKWARD_VECS_PER_THREAD)
// threads rounded up to whole waves, raised for small batches until the
// grid holds about kBackwardTargetThreads threads (one 256-thread block per
// compute unit), at most the row's vectors, 1024, or 512 with expert biases
// (whose second set of row loads needs the larger register budget).
#ifndef EP_BACKWARD_VECS_PER_THREAD
#define EP_BACKWARD_VECS_PER_THREAD 16
#endif
// grad_y rows go out with non-temporal stores: at prefill (4096 x 7168,
// 470 MB of grad_y, more than the MALL holds), interleaved on one box,
// ordinary stores measured 170 us after a cache flush but 213 us back to
// back and 222-227 us with the write-back of what they leave dirty, against
// 208-210 / 195 / 207-210 us for non-temporal ones.
#ifndef EP_BACKWARD_NT_STORE
#define EP_BACKWARD_NT_STORE 1
#endif
constexpr int kMaxRowThreads = 1024;
constexpr int64_t kBackwardTargetThreads = 256 * 256;
constexpr int row_threads_cap(bool has_bias) { return has_bias ? 512 : kMaxRowThreads; }

// Row pass: one block per token, threads tiling the row's 16-byte columns.
// The gradient vector is loaded once; per chunk of 8 slots the expert rows
// (and expert biases) are loaded branch-free, the scaled gradient is stored
// to each routed row, and binary64 dot partials are kept per slot.
template <bool WANT_Y, bool WANT_W, bool HAS_W, bool HAS_BIAS, typename IdxT>
__global__ __launch_bounds__(row_threads_cap(WANT_W && HAS_BIAS)) void combine_backward_kernel(
    BackwardArgs a) {
    __shared__ double s_part[kMaxRowThreads / 64][kChunk];
    if (a.scalars[EP_SCALAR_ERROR_BITS] & EP_ERRBIT_FATAL) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int waves = static_cast<int>(blockDim.x / 64);
    const int64_t t = blockIdx.x;
    const int K = a.num_topk, E = a.num_experts;
    const int64_t V = a.row_vecs;
    const int32_t row_bytes = static_cast<int32_t>(V * 16);
    const u32x4 *g = static_cast<const u32x4 *>(a.g) + t * V;
    u32x4 *gy = static_cast<u32x4 *>(a.grad_y);
    const IdxT *idx = static_cast<const IdxT *>(a.topk_idx);
    for (int k0 = 0; k0 < K; k0 += kChunk) {
        int32_t r[kChunk];
        int64_t e[kChunk];
        float wk[kChunk];
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            r[j] = k0 + j < K ? a.dst[t * K + k0 + j] : -1;
            if (r[j] >= a.capacity) r[j] = -1;
            e[j] = (WANT_W && HAS_BIAS && r[j] >= 0) ? static_cast<int64_t>(idx[t * K + k0 + j])
                                                      : -1;
            if (e[j] >= E) e[j] = -1;
            wk[j] = (WANT_Y && HAS_W && r[j] >= 0) ? a.w[t * K + k0 + j] : 1.0f;
        }
        double acc[kChunk];
#pragma unroll
        for (int j = 0; j < kChunk; ++j) acc[j] = 0.0;
        for (int64_t c = threadIdx.x; c < V; c += blockDim.x) {
            const u32x4 gv = g[c];
            const int32_t col = static_cast<int32_t>(c * 16);
            u32x4 yv[kChunk], bv[kChunk];
            if (WANT_W) {
#pragma unroll
                for (int j = 0; j < kChunk; ++j) {
                    yv[j] = __builtin_amdgcn_raw_buffer_load_b128(
                        row_rsrc(a.y, r[j], row_bytes, r[j] >= 0), col, 0, 2);
                    if (HAS_BIAS)
                        bv[j] = __builtin_amdgcn_raw_buffer_load_b128(
                            row_rsrc(a.bias, e[j], row_bytes, e[j] >= 0), col, 0, 0);
                }
            }
            if (WANT_Y) {
#pragma unroll
                for (int j = 0; j < kChunk; ++j)
                    if (r[j] >= 0) {
                        const u32x4 o = HAS_W ? scale_bf16x8(gv, wk[j]) : gv;
                        u32x4 *d = gy + static_cast<int64_t>(r[j]) * V + c;
                        if (EP_BACKWARD_NT_STORE) __builtin_nontemporal_store(o, d);
                        else *d = o;
                    }
            }
            if (WANT_W) {
                float gf[8];
                unpack8(gv, gf);
#pragma unroll
                for (int j = 0; j < kChunk; ++j) {
                    if (r[j] < 0) continue;
                    float yf[8], bf[8];
                    unpack8(yv[j], yf);
                    if (HAS_BIAS) unpack8(bv[j], bf);     // zeros when e[j] < 0
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        double v = static_cast<double>(yf[i]);
                        if (HAS_BIAS) v += static_cast<double>(bf[i]);
                        acc[j] += static_cast<double>(gf[i]) * v;
                    }
                }
            }
        }
        if (WANT_W) {
#pragma unroll
            for (int j = 0; j < kChunk; ++j) {
                double x = acc[j];
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
                if (lane == 0) s_part[wave][j] = x;
            }
            __syncthreads();
            if (threadIdx.x < kChunk && k0 + static_cast<int>(threadIdx.x) < K) {
                const int j = threadIdx.x;
                double sum = 0.0;
                for (int w = 0; w < waves; ++w) sum += s_part[w][j];
                a.grad_w[t * K + k0 + j] = r[j] >= 0 ? static_cast<float>(sum) : 0.0f;
            }
            __syncthreads();
        }
    }
}

template <bool HAS_W>
__global__ __launch_bounds__(kThreads) void bias_grad_kernel(BackwardArgs a, int col_groups) {
    __shared__ double s_part[kThreads / 64][64][8];
    if (a.scalars[EP_SCALAR_ERROR_BITS] & EP_ERRBIT_FATAL) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = blockIdx.x / col_groups;
    const int64_t c = static_cast<int64_t>(blockIdx.x % col_groups) * 64 + lane;
    const int64_t V = a.row_vecs;
    const int K = a.num_topk;
    const int64_t r0 = a.psum[e];
    int64_t r1 = r0 + a.counts[e];
    if (r1 > a.capacity) r1 = a.capacity;
    const u32x4 *g = static_cast<const u32x4 *>(a.g);
    double acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0;
    constexpr int W = kThreads / 64;
    for (int64_t rb = r0 + wave; rb < r1; rb += W * kChunk) {
        int32_t s[kChunk];
        u32x4 gv[kChunk];
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const int64_t r = rb + static_cast<int64_t>(j) * W;
            s[j] = r < r1 ? a.src_meta[r] : -1;
            if (s[j] >= static_cast<int64_t>(a.num_tokens) * K) s[j] = -1;
        }
#pragma unroll
        for (int j = 0; j < kChunk; ++j)
            if (s[j] >= 0 && c < V) gv[j] = g[static_cast<int64_t>(s[j] / K) * V + c];
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            if (s[j] < 0 || c >= V) continue;
            float f[8];
            unpack8(gv[j], f);
            const double wk = HAS_W ? static_cast<double>(a.w[s[j]]) : 1.0;
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += HAS_W ? wk * static_cast<double>(f[i])
                                                        : static_cast<double>(f[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) s_part[wave][lane][i] = acc[i];
    __syncthreads();
    if (wave == 0 && c < V) {
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            double sum = 0.0;
#pragma unroll
            for (int w = 0; w < W; ++w) sum += s_part[w][lane][i];
            o[i] = static_cast<float>(sum);
        }
        float *out = a.grad_bias + static_cast<int64_t>(e) * V * 8 + c * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = o[i];
    }
}

__global__ void gather_rows_kernel(GatherArgs a) {
    if (a.scalars[EP_SCALAR_ERROR_BITS] & EP_ERRBIT_FATAL) return;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= a.num_slots) return;
    const int32_t r = a.dst[i];
    a.out[i] = (r >= 0 && r < a.capacity && a.row_values) ? a.row_values[r] : 0.0f;
}

template <bool WANT_Y, bool WANT_W, bool HAS_W>
hipError_t launch_rows3(const BackwardArgs &a, hipStream_t s, hipEvent_t st, hipEvent_t sp) {
    const bool has_bias = WANT_W && a.bias;
    const int64_t per = EP_BACKWARD_VECS_PER_THREAD;
    int64_t threads = (a.row_vecs + per - 1) / per;
    const int64_t spread = (kBackwardTargetThreads + a.num_tokens - 1) / a.num_tokens;
    if (threads < spread) threads = spread < a.row_vecs ? spread : a.row_vecs;
    threads = (threads + 63) / 64 * 64;
    if (threads > row_threads_cap(has_bias)) threads = row_threads_cap(has_bias);
    const dim3 grid(static_cast<unsigned>(a.num_tokens)), block(static_cast<unsigned>(threads));
    if (has_bias) {
        if (a.idx_is_i64)
            return launch_kernel(combine_backward_kernel<WANT_Y, WANT_W, HAS_W, true, int64_t>,
                                 grid, block, s, st, sp, a);
        return launch_kernel(combine_backward_kernel<WANT_Y, WANT_W, HAS_W, true, int32_t>, grid,
                             block, s, st, sp, a);
    }
    return launch_kernel(combine_backward_kernel<WANT_Y, WANT_W, HAS_W, false, int64_t>, grid,
                         block, s, st, sp, a);
}

template <bool WANT_Y, bool WANT_W>
hipError_t launch_rows2(const BackwardArgs &a, hipStream_t s, hipEvent_t st, hipEvent_t sp) {
    return a.w ? launch_rows3<WANT_Y, WANT_W, true>(a, s, st, sp)
               : launch_rows3<WANT_Y, WANT_W, false>(a, s, st, sp);
}

}  // namespace

hipError_t launch_combine_backward(const BackwardArgs &a, hipStream_t stream, CallEvents ev) {
    // The row pass (grad_y and/or grad_w) and the bias pass; the call's start
    // event goes on the first kernel launched and its stop event on the last.
    const bool rows = (a.grad_y || a.grad_w) && a.num_tokens > 0;
    const bool bias = a.grad_bias != nullptr;
    if (!rows && !bias) return hipSuccess;
    hipError_t e = hipSuccess;
    if (rows) {
        hipEvent_t sp = bias ? nullptr : ev.stop;
        if (a.grad_y && a.grad_w) e = launch_rows2<true, true>(a, stream, ev.start, sp);
        else if (a.grad_y) e = launch_rows2<true, false>(a, stream, ev.start, sp);
        else e = launch_rows2<false, true>(a, stream, ev.start, sp);
        if (e != hipSuccess) return e;
    }
    if (bias) {
        const int groups = static_cast<int>((a.row_vecs + 63) / 64);
        const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.num_experts) * groups));
        hipEvent_t st = rows ? nullptr : ev.start;
        e = a.w ? launch_kernel(bias_grad_kernel<true>, grid, dim3(kThreads), stream, st, ev.stop,
                                a, groups)
                : launch_kernel(bias_grad_kernel<false>, grid, dim3(kThreads), stream, st,
                                ev.stop, a, groups);
    }
    return e;
}

hipError_t launch_gather_rows(const GatherArgs &a, hipStream_t stream, CallEvents ev) {
    if (a.num_slots == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((a.num_slots + 255) / 256));
    return launch_kernel(gather_rows_kernel, grid, dim3(256), stream, ev.start, ev.stop, a);
}

}  // namespace ep
