// Non-expanded ("rank") layout: dispatch and combine on gfx950.
//
// DeepEP notes ch.7 "V2: how dispatch builds expert inputs", s7.4: besides the
// expert-expanded layout there is the normal layout, each received token once
// ([received_tokens, hidden] plus top-k metadata), and s7.3: the epilogue
// writes the received top-k ids and weights.  Ch.8 s8.1: combine takes
// bias_0 and bias_1.  At one rank a token is received when it has a valid
// slot; ep_layout gives each such token its row (recv_row) in token order.
//
// dispatch_rank: one wave per token copies the row (16-byte vectors,
// non-temporal stores: faster at every size measured, e.g. 4096 FP8 rows of
// 7168 11.7-12.8 -> 9.9-10.2 us, 32768 bf16 rows 199 -> 178 us, 32768 FP8
// rows 107 -> 72 us; non-temporal loads measured slower), its FP8 scales
// and its top-k ids / weights (-1 / 0 on empty or invalid slots) to row
// recv_row[t].
// combine_rank: one thread per 16-byte output vector; the token's row (or
// +0.0), then bias_0, then bias_1, in binary32, rounded to bf16 (RNE).
#include "ep_internal.h"
#include "../../include/ep.h"

namespace ep {
namespace {

constexpr int kThreads = 256;

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

template <int VPL, typename IdxT>
__global__ __launch_bounds__(kThreads) void dispatch_rank_kernel(RankArgs a) {
    if (a.scalars[EP_SCALAR_ERROR_BITS] & EP_ERRBIT_SCAN_TIMEOUT) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + wave;
    if (t >= a.num_tokens) return;
    const int64_t row = a.recv_row[t];
    if (row < 0 || row >= a.num_tokens) return;
    const int K = a.num_topk;
    const int64_t V = a.row_vecs;
    const u32x4 *src = static_cast<const u32x4 *>(a.x) + t * V;
    u32x4 *dst = static_cast<u32x4 *>(a.out) + row * V;
    for (int64_t c0 = 0; c0 < V; c0 += 64 * VPL) {
        u32x4 v[VPL];
#pragma unroll
        for (int q = 0; q < VPL; ++q) {
            const int64_t c = c0 + q * 64 + lane;
            if (c < V) v[q] = src[c];
        }
#pragma unroll
        for (int q = 0; q < VPL; ++q) {
            const int64_t c = c0 + q * 64 + lane;
            if (c < V) __builtin_nontemporal_store(v[q], dst + c);
        }
    }
    for (int j = lane; j < a.num_sf; j += 64)
        a.out_sf[row * a.out_ts + j * a.out_hs] = a.sf[t * a.sf_ts + j * a.sf_hs];
    if (lane < K) {
        const IdxT *idx = static_cast<const IdxT *>(a.topk_idx);
        const int64_t e = static_cast<int64_t>(idx[t * K + lane]);
        const bool valid = e >= 0 && e < a.num_experts;
        if (a.out_idx)
            static_cast<IdxT *>(a.out_idx)[row * K + lane] = valid ? static_cast<IdxT>(e)
                                                                   : static_cast<IdxT>(-1);
        if (a.out_w)
            a.out_w[row * K + lane] = valid ? (a.w ? a.w[t * K + lane] : 1.0f) : 0.0f;
    }
}

__global__ __launch_bounds__(kThreads) void combine_rank_kernel(RankArgs a, int groups) {
#pragma clang fp contract(off)
    if (a.scalars[EP_SCALAR_ERROR_BITS] & EP_ERRBIT_SCAN_TIMEOUT) return;
    const int64_t t = blockIdx.x / groups;
    const int64_t v = static_cast<int64_t>(blockIdx.x % groups) * blockDim.x + threadIdx.x;
    if (v >= a.row_vecs) return;
    const int64_t V = a.row_vecs;
    const int64_t row = a.recv_row[t];
    float acc[8];
    if (row >= 0 && row < a.num_tokens) {
        unpack8(static_cast<const u32x4 *>(a.x)[row * V + v], acc);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    }
    float b[8];
    if (a.bias_0) {
        unpack8(static_cast<const u32x4 *>(a.bias_0)[t * V + v], b);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = acc[i] + b[i];
    }
    if (a.bias_1) {
        unpack8(static_cast<const u32x4 *>(a.bias_1)[t * V + v], b);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = acc[i] + b[i];
    }
    u32x4 o;
    o.x = bf16_rne(acc[0]) | (bf16_rne(acc[1]) << 16);
    o.y = bf16_rne(acc[2]) | (bf16_rne(acc[3]) << 16);
    o.z = bf16_rne(acc[4]) | (bf16_rne(acc[5]) << 16);
    o.w = bf16_rne(acc[6]) | (bf16_rne(acc[7]) << 16);
    static_cast<u32x4 *>(a.out)[t * V + v] = o;
}

template <int VPL>
hipError_t launch_drank(const RankArgs &a, hipStream_t s, CallEvents ev) {
    const dim3 grid(static_cast<unsigned>((a.num_tokens + 3) / 4));
    if (a.idx_is_i64)
        return launch_kernel(dispatch_rank_kernel<VPL, int64_t>, grid, dim3(kThreads), s,
                             ev.start, ev.stop, a);
    return launch_kernel(dispatch_rank_kernel<VPL, int32_t>, grid, dim3(kThreads), s, ev.start,
                         ev.stop, a);
}

// Rank rows of a layout given as slot rows (ep_handle_import): token t is
// received when one of its K slots has a row (dst >= 0); received tokens get
// rows 0, 1, ... in token order.  One block of kRowsThreads threads, each
// taking a run of consecutive tokens: count its received tokens, exclusive
// scan over the block, then number them.  Writes recv_row [T], recv_src
// [received] and the received count.
constexpr int kRowsThreads = 1024;

__global__ __launch_bounds__(kRowsThreads) void rank_rows_kernel(const int32_t *dst, int64_t T,
                                                                 int K, int32_t *recv_row,
                                                                 int32_t *recv_src,
                                                                 int32_t *num_recv) {
    __shared__ int64_t s_wave[kRowsThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t per = (T + kRowsThreads - 1) / kRowsThreads;
    const int64_t t0 = tid * per;
    const int64_t t1 = t0 + per < T ? t0 + per : T;
    int64_t cnt = 0;
    for (int64_t t = t0; t < t1; ++t) {
        bool any = false;
        for (int k = 0; k < K; ++k) any = any || dst[t * K + k] >= 0;
        cnt += any;
    }
    int64_t x = cnt;                                   // inclusive scan in the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int64_t base = 0, total = 0;
    for (int w = 0; w < kRowsThreads / 64; ++w) {
        if (w < wave) base += s_wave[w];
        total += s_wave[w];
    }
    int64_t row = base + x - cnt;
    for (int64_t t = t0; t < t1; ++t) {
        bool any = false;
        for (int k = 0; k < K; ++k) any = any || dst[t * K + k] >= 0;
        if (any) {
            recv_row[t] = static_cast<int32_t>(row);
            recv_src[row] = static_cast<int32_t>(t);
            ++row;
        } else {
            recv_row[t] = -1;
        }
    }
    if (tid == 0) *num_recv = static_cast<int32_t>(total);
}

}  // namespace

hipError_t launch_rank_rows(const int32_t *dst, int64_t num_tokens, int num_topk,
                            int32_t *recv_row, int32_t *recv_src, int32_t *num_recv,
                            hipStream_t stream) {
    rank_rows_kernel<<<dim3(1), dim3(kRowsThreads), 0, stream>>>(dst, num_tokens, num_topk,
                                                                 recv_row, recv_src, num_recv);
    return hipGetLastError();
}

hipError_t launch_dispatch_rank(const RankArgs &a, hipStream_t stream, CallEvents ev) {
    if (a.num_tokens == 0) return hipSuccess;
    const int64_t per_lane = (a.row_vecs + 63) / 64;
    if (per_lane <= 1) return launch_drank<1>(a, stream, ev);
    if (per_lane <= 2) return launch_drank<2>(a, stream, ev);
    if (per_lane <= 4) return launch_drank<4>(a, stream, ev);
    if (per_lane <= 8) return launch_drank<8>(a, stream, ev);
    return launch_drank<16>(a, stream, ev);
}

hipError_t launch_combine_rank(const RankArgs &a, hipStream_t stream, CallEvents ev) {
    if (a.num_tokens == 0) return hipSuccess;
    int threads = 256;
    int64_t best = -1;
    for (int b : {256, 128, 64}) {
        const int64_t waste = (a.row_vecs + b - 1) / b * b - a.row_vecs;
        if (best < 0 || waste < best) {
            best = waste;
            threads = b;
        }
    }
    const int groups = static_cast<int>((a.row_vecs + threads - 1) / threads);
    const int64_t blocks = static_cast<int64_t>(a.num_tokens) * groups;
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    return launch_kernel(combine_rank_kernel, dim3(static_cast<unsigned>(blocks)), dim3(threads),
                         stream, ev.start, ev.stop, a, groups);
}

}  // namespace ep
