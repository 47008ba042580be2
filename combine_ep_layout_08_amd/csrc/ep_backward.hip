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
//  * scatter_scaled: one wave per token; the gradient row is loaded once into
//    registers and stored, scaled per slot, to every routed row (like
//    dispatch).
//  * weight_grad: one block per token; threads stride over the row's 16-byte
//    columns and keep one binary64 partial per slot of a chunk of 8; a
//    shuffle tree and an ordered pass over the 4 waves finish each dot.
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

template <int VPL, bool HAS_W>
__global__ __launch_bounds__(kThreads) void scatter_scaled_kernel(BackwardArgs a) {
    if (a.scalars[EP_SCALAR_ERROR_BITS] & EP_ERRBIT_FATAL) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + wave;
    if (t >= a.num_tokens) return;
    const int K = a.num_topk;
    const int64_t V = a.row_vecs;
    int32_t my_dst = lane < K ? a.dst[t * K + lane] : -1;
    if (my_dst >= a.capacity) my_dst = -1;
    const float my_w = (HAS_W && lane < K) ? a.w[t * K + lane] : 1.0f;
    const u32x4 *src = static_cast<const u32x4 *>(a.g) + t * V;
    u32x4 *out = static_cast<u32x4 *>(a.grad_y);
    for (int64_t c0 = 0; c0 < V; c0 += 64 * VPL) {
        u32x4 v[VPL];
#pragma unroll
        for (int q = 0; q < VPL; ++q) {
            const int64_t c = c0 + q * 64 + lane;
            if (c < V) v[q] = src[c];
        }
        for (int k = 0; k < K; ++k) {
            const int32_t r = __builtin_amdgcn_readlane(my_dst, k);
            if (r < 0) continue;
            const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), k));
            u32x4 *d = out + static_cast<int64_t>(r) * V;
#pragma unroll
            for (int q = 0; q < VPL; ++q) {
                const int64_t c = c0 + q * 64 + lane;
                if (c < V) d[c] = HAS_W ? scale_bf16x8(v[q], wk) : v[q];
            }
        }
    }
}

template <bool HAS_BIAS, typename IdxT>
__global__ __launch_bounds__(kThreads) void weight_grad_kernel(BackwardArgs a) {
    __shared__ double s_part[kThreads / 64][kChunk];
    if (a.scalars[EP_SCALAR_ERROR_BITS] & EP_ERRBIT_FATAL) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t t = blockIdx.x;
    const int K = a.num_topk, E = a.num_experts;
    const int64_t V = a.row_vecs;
    const u32x4 *g = static_cast<const u32x4 *>(a.g) + t * V;
    const IdxT *idx = static_cast<const IdxT *>(a.topk_idx);
    for (int k0 = 0; k0 < K; k0 += kChunk) {
        int32_t r[kChunk];
        int64_t e[kChunk];
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            r[j] = k0 + j < K ? a.dst[t * K + k0 + j] : -1;
            if (r[j] >= a.capacity) r[j] = -1;
            e[j] = (HAS_BIAS && r[j] >= 0) ? static_cast<int64_t>(idx[t * K + k0 + j]) : -1;
            if (e[j] >= E) e[j] = -1;
        }
        double acc[kChunk];
#pragma unroll
        for (int j = 0; j < kChunk; ++j) acc[j] = 0.0;
        const int32_t row_bytes = static_cast<int32_t>(V * 16);
        for (int64_t c = threadIdx.x; c < V; c += kThreads) {
            float gf[8];
            unpack8(g[c], gf);
            u32x4 yv[kChunk], bv[kChunk];
            const int32_t col = static_cast<int32_t>(c * 16);
#pragma unroll
            for (int j = 0; j < kChunk; ++j) {
                yv[j] = __builtin_amdgcn_raw_buffer_load_b128(
                    row_rsrc(a.y, r[j], row_bytes, r[j] >= 0), col, 0, 2);
                if (HAS_BIAS)
                    bv[j] = __builtin_amdgcn_raw_buffer_load_b128(
                        row_rsrc(a.bias, e[j], row_bytes, e[j] >= 0), col, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < kChunk; ++j) {
                if (r[j] < 0) continue;
                float yf[8], bf[8];
                unpack8(yv[j], yf);
                if (HAS_BIAS && e[j] >= 0) unpack8(bv[j], bf);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    double v = static_cast<double>(yf[i]);
                    if (HAS_BIAS && e[j] >= 0) v += static_cast<double>(bf[i]);
                    acc[j] += static_cast<double>(gf[i]) * v;
                }
            }
        }
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
#pragma unroll
            for (int w = 0; w < kThreads / 64; ++w) sum += s_part[w][j];
            a.grad_w[t * K + k0 + j] = r[j] >= 0 ? static_cast<float>(sum) : 0.0f;
        }
        __syncthreads();
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

template <int VPL>
hipError_t launch_scatter(const BackwardArgs &a, hipStream_t s, hipEvent_t start,
                          hipEvent_t stop) {
    const dim3 grid(static_cast<unsigned>((a.num_tokens + 3) / 4));
    if (a.w)
        return launch_kernel(scatter_scaled_kernel<VPL, true>, grid, dim3(kThreads), s, start,
                             stop, a);
    return launch_kernel(scatter_scaled_kernel<VPL, false>, grid, dim3(kThreads), s, start, stop,
                         a);
}

}  // namespace

hipError_t launch_combine_backward(const BackwardArgs &a, hipStream_t stream, CallEvents ev) {
    // Up to three kernels; the call's start event goes on the first launched
    // and its stop event on the last.
    const int n = (a.grad_y && a.num_tokens > 0) + (a.grad_w && a.num_tokens > 0) +
                  (a.grad_bias != nullptr);
    if (n == 0) return hipSuccess;
    int done = 0;
    auto evs = [&](hipEvent_t *st, hipEvent_t *sp) {
        *st = done == 0 ? ev.start : nullptr;
        *sp = done == n - 1 ? ev.stop : nullptr;
        ++done;
    };
    hipError_t e = hipSuccess;
    hipEvent_t st, sp;
    if (a.grad_y && a.num_tokens > 0) {
        evs(&st, &sp);
        const int64_t per_lane = (a.row_vecs + 63) / 64;
        if (per_lane <= 1) e = launch_scatter<1>(a, stream, st, sp);
        else if (per_lane <= 2) e = launch_scatter<2>(a, stream, st, sp);
        else if (per_lane <= 4) e = launch_scatter<4>(a, stream, st, sp);
        else if (per_lane <= 8) e = launch_scatter<8>(a, stream, st, sp);
        else e = launch_scatter<16>(a, stream, st, sp);
        if (e != hipSuccess) return e;
    }
    if (a.grad_w && a.num_tokens > 0) {
        evs(&st, &sp);
        const dim3 grid(static_cast<unsigned>(a.num_tokens));
        if (a.bias)
            e = a.idx_is_i64
                    ? launch_kernel(weight_grad_kernel<true, int64_t>, grid, dim3(kThreads), stream,
                                    st, sp, a)
                    : launch_kernel(weight_grad_kernel<true, int32_t>, grid, dim3(kThreads), stream,
                                    st, sp, a);
        else
            e = launch_kernel(weight_grad_kernel<false, int64_t>, grid, dim3(kThreads), stream, st,
                              sp, a);
        if (e != hipSuccess) return e;
    }
    if (a.grad_bias) {
        evs(&st, &sp);
        const int groups = static_cast<int>((a.row_vecs + 63) / 64);
        const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.num_experts) * groups));
        e = a.w ? launch_kernel(bias_grad_kernel<true>, grid, dim3(kThreads), stream, st, sp, a,
                                groups)
                : launch_kernel(bias_grad_kernel<false>, grid, dim3(kThreads), stream, st, sp, a,
                                groups);
    }
    return e;
}

hipError_t launch_gather_rows(const GatherArgs &a, hipStream_t stream, CallEvents ev) {
    if (a.num_slots == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((a.num_slots + 255) / 256));
    return launch_kernel(gather_rows_kernel, grid, dim3(256), stream, ev.start, ev.stop, a);
}

}  // namespace ep
