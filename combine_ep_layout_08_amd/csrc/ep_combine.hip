// Combine on gfx950: follow the layout back to token order and reduce.
//
// What is computed follows DeepEP notes ch.8 "V2: combine, handle and async
// overlap", s8.1 (combine reads the handle's routing state and reduces the
// expert outputs back to the source token; bias and gate-weight reduction can
// be fused; x is bf16 and the top-k weights fp32) and the vLLM PR 52781 digest
// (implementation breakdown: bf16 input required, weights may be None):
//
//   out[t][h] = bf16_rne( sum over valid k = 0..K-1, in this order, of
//                         w[t,k] * (y[dst[t,k]][h] + bias[e_k][h]) )
//
// in binary32 from +0.0, every add and multiply rounded separately (no
// contraction), a missing weight meaning the product is skipped.
//
// A block owns whole tokens; each thread owns 16-byte column vectors (8 bf16)
// of the token's output row.  The token's destination rows are block-uniform
// (scalar loads).  For each chunk of up to 8 slots, all rows' vectors are
// loaded before any is accumulated; the accumulation itself runs in slot
// order.
#include "ep_internal.h"
#include "../../include/ep.h"

namespace ep {
namespace {

constexpr int kSlotChunk = 8;

__device__ inline void unpack_bf16x8(const u32x4 v, float f[8]) {
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

// Buffer resource word 3 for gfx9-family raw buffers (32-bit data format).
constexpr int kRsrcWord3 = 0x00020000;

// Launch shape.  A work unit is one group of a token's columns: blockDim *
// kVecsPerThread 16-byte vectors of its output row, one block per unit, the
// block size (256, 128 or 64 threads) picked to tile the row with the fewest
// idle lanes.  Each thread keeps kVecsPerThread * kSlotChunk row loads in
// flight.  Measured on MI355X, many short blocks beat a persistent grid that
// walks whole rows (89 us vs 102-120 us on the prefill workload), so the
// persistent form is off by default (EP_COMBINE_BLOCKS_PER_CU > 0 enables it).
#ifndef EP_COMBINE_BLOCKS_PER_CU
#define EP_COMBINE_BLOCKS_PER_CU 0
#endif
#ifndef EP_COMBINE_VECS_PER_THREAD
#define EP_COMBINE_VECS_PER_THREAD 1
#endif
// Cache policy of the expert-row loads (gfx94x/gfx950 bits: 0 = sc0, 1 = nt,
// 4 = sc1); rows are read once, so they stream.
#ifndef EP_COMBINE_LOAD_POLICY
#define EP_COMBINE_LOAD_POLICY 2
#endif
// Output stores are non-temporal unless this is 0.
#ifndef EP_COMBINE_NT_STORE
#define EP_COMBINE_NT_STORE 1
#endif
// Block size: 0 = pick 256 / 128 / 64 to tile the row, else this many threads.
#ifndef EP_COMBINE_THREADS
#define EP_COMBINE_THREADS 0
#endif
constexpr int kMaxCombineThreads = 256;
constexpr int kBlocksPerCu = EP_COMBINE_BLOCKS_PER_CU;
constexpr int kVecsPerThread = EP_COMBINE_VECS_PER_THREAD;
constexpr int kLoadPolicy = EP_COMBINE_LOAD_POLICY;

// Range-checked row view: a load at a byte offset >= `bytes` returns zero and
// touches no memory.  Empty slots get bytes = 0, so their loads are free and
// every slot of a chunk can be loaded without a branch; the same check makes
// the columns past the row's end safe to load.
__device__ inline __amdgpu_buffer_rsrc_t row_rsrc(const void *base, int64_t row, int32_t bytes,
                                                  bool valid) {
    const char *p = static_cast<const char *>(base) + (valid ? row * bytes : 0);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(p), 0, valid ? bytes : 0,
                                             kRsrcWord3);
}

// One group of columns of one token: loads of every slot first, then the
// slot-order binary32 accumulation, then the bf16 store.
template <bool HAS_BIAS, bool HAS_W, bool HAS_TB, typename IdxT>
__device__ inline void combine_columns(const CombineArgs &a, int64_t t, int64_t v0) {
#pragma clang fp contract(off)
    const int K = a.num_topk;
    const int32_t row_bytes = static_cast<int32_t>(a.row_vecs * 16);
    int32_t col[kVecsPerThread];
#pragma unroll
    for (int u = 0; u < kVecsPerThread; ++u)
        col[u] = static_cast<int32_t>((v0 + static_cast<int64_t>(u) * blockDim.x) * 16);
    const IdxT *idx = static_cast<const IdxT *>(a.topk_idx);
    const int32_t *dst = a.dst + t * K;

    float acc[kVecsPerThread][8];
#pragma unroll
    for (int u = 0; u < kVecsPerThread; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[u][i] = 0.0f;

    for (int k0 = 0; k0 < K; k0 += kSlotChunk) {
        int32_t r[kSlotChunk];
        u32x4 d[kSlotChunk][kVecsPerThread], bb[kSlotChunk][kVecsPerThread];
#pragma unroll
        for (int j = 0; j < kSlotChunk; ++j) {
            r[j] = (k0 + j < K) ? dst[k0 + j] : -1;
            if (r[j] >= a.capacity) r[j] = -1;          // never read past y
        }
        // Issue every load of the chunk before using any of them.
#pragma unroll
        for (int j = 0; j < kSlotChunk; ++j) {
            const bool ok = r[j] >= 0;
            const __amdgpu_buffer_rsrc_t ry = row_rsrc(a.y, r[j], row_bytes, ok);
#pragma unroll
            for (int u = 0; u < kVecsPerThread; ++u)
                d[j][u] = __builtin_amdgcn_raw_buffer_load_b128(ry, col[u], 0, kLoadPolicy);
            if (HAS_BIAS) {
                const int64_t e = ok ? static_cast<int64_t>(idx[t * K + k0 + j]) : 0;
                const bool e_ok = ok && e >= 0 && e < a.num_experts;
                const __amdgpu_buffer_rsrc_t rb = row_rsrc(a.bias, e, row_bytes, e_ok);
#pragma unroll
                for (int u = 0; u < kVecsPerThread; ++u)
                    bb[j][u] = __builtin_amdgcn_raw_buffer_load_b128(rb, col[u], 0, 0);
            }
        }
        // Accumulate in slot order.
#pragma unroll
        for (int j = 0; j < kSlotChunk; ++j) {
            if (r[j] < 0) continue;
            const float wk = HAS_W ? a.w[t * K + k0 + j] : 1.0f;
#pragma unroll
            for (int u = 0; u < kVecsPerThread; ++u) {
                float f[8];
                unpack_bf16x8(d[j][u], f);
                if (HAS_BIAS) {
                    float b[8];
                    unpack_bf16x8(bb[j][u], b);
#pragma unroll
                    for (int i = 0; i < 8; ++i) f[i] = f[i] + b[i];
                }
                if (HAS_W) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) f[i] = wk * f[i];
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[u][i] = acc[u][i] + f[i];
            }
        }
    }
    // Per-token biases after the reduction: bias_0, then bias_1.
    if (HAS_TB) {
#pragma unroll
        for (int u = 0; u < kVecsPerThread; ++u) {
            const int64_t v = v0 + static_cast<int64_t>(u) * blockDim.x;
            if (v >= a.row_vecs) break;
            float b[8];
            if (a.bias_0) {
                unpack_bf16x8(static_cast<const u32x4 *>(a.bias_0)[t * a.row_vecs + v], b);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[u][i] = acc[u][i] + b[i];
            }
            if (a.bias_1) {
                unpack_bf16x8(static_cast<const u32x4 *>(a.bias_1)[t * a.row_vecs + v], b);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[u][i] = acc[u][i] + b[i];
            }
        }
    }
    u32x4 *out = static_cast<u32x4 *>(a.out) + t * a.row_vecs;
#pragma unroll
    for (int u = 0; u < kVecsPerThread; ++u) {
        const int64_t v = v0 + static_cast<int64_t>(u) * blockDim.x;
        if (v >= a.row_vecs) break;
        u32x4 o;
        o.x = bf16_rne(acc[u][0]) | (bf16_rne(acc[u][1]) << 16);
        o.y = bf16_rne(acc[u][2]) | (bf16_rne(acc[u][3]) << 16);
        o.z = bf16_rne(acc[u][4]) | (bf16_rne(acc[u][5]) << 16);
        o.w = bf16_rne(acc[u][6]) | (bf16_rne(acc[u][7]) << 16);
        if (EP_COMBINE_NT_STORE)
            __builtin_nontemporal_store(o, out + v);
        else
            out[v] = o;
    }
}

template <bool HAS_BIAS, bool HAS_W, bool HAS_TB, typename IdxT>
__global__ __launch_bounds__(kMaxCombineThreads) void combine_kernel(CombineArgs a,
                                                                    int groups_per_token) {
    if (a.scalars[EP_SCALAR_ERROR_BITS] & EP_ERRBIT_FATAL) return;
    const int64_t group = static_cast<int64_t>(blockDim.x) * kVecsPerThread;
    if (kBlocksPerCu == 0) {
        // One unit per block, straight-line (measurably faster than the loop).
        const int64_t t = blockIdx.x / groups_per_token;
        const int64_t v0 = (blockIdx.x % groups_per_token) * group + threadIdx.x;
        if (v0 < a.row_vecs) combine_columns<HAS_BIAS, HAS_W, HAS_TB, IdxT>(a, t, v0);
        return;
    }
    const int64_t units = static_cast<int64_t>(a.num_tokens) * groups_per_token;
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
        const int64_t t = u / groups_per_token;
        const int64_t v0 = (u % groups_per_token) * group + threadIdx.x;
        if (v0 < a.row_vecs) combine_columns<HAS_BIAS, HAS_W, HAS_TB, IdxT>(a, t, v0);
    }
}

template <bool HAS_BIAS, bool HAS_W, bool HAS_TB>
hipError_t launch_bw(const CombineArgs &a, hipStream_t stream, CallEvents ev) {
    // Block size among 256 / 128 / 64 threads that wastes the fewest lanes
    // on the row's vector count (ties go to the larger block).
    int threads = kMaxCombineThreads;
    int64_t best = -1;
    for (int b : {256, 128, 64}) {
        const int64_t span = static_cast<int64_t>(b) * kVecsPerThread;
        const int64_t waste = (a.row_vecs + span - 1) / span * span - a.row_vecs;
        if (best < 0 || waste < best) {
            best = waste;
            threads = b;
        }
    }
    if (EP_COMBINE_THREADS > 0) threads = EP_COMBINE_THREADS;
    const int64_t span = static_cast<int64_t>(threads) * kVecsPerThread;
    const int gpt = static_cast<int>((a.row_vecs + span - 1) / span);
    const int64_t blocks = persistent_grid(static_cast<int64_t>(a.num_tokens) * gpt, kBlocksPerCu);
    if (blocks == 0) return hipSuccess;
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    const dim3 grid(static_cast<unsigned>(blocks)), block(threads);
    if (a.idx_is_i64)
        return launch_kernel(combine_kernel<HAS_BIAS, HAS_W, HAS_TB, int64_t>, grid, block,
                             stream, ev.start, ev.stop, a, gpt);
    return launch_kernel(combine_kernel<HAS_BIAS, HAS_W, HAS_TB, int32_t>, grid, block, stream,
                         ev.start, ev.stop, a, gpt);
}

}  // namespace

template <bool HAS_TB>
hipError_t launch_tb(const CombineArgs &a, hipStream_t stream, CallEvents ev) {
    if (a.bias)
        return a.w ? launch_bw<true, true, HAS_TB>(a, stream, ev)
                   : launch_bw<true, false, HAS_TB>(a, stream, ev);
    return a.w ? launch_bw<false, true, HAS_TB>(a, stream, ev)
               : launch_bw<false, false, HAS_TB>(a, stream, ev);
}

hipError_t launch_combine(const CombineArgs &a, hipStream_t stream, CallEvents ev) {
    if (a.bias_0 || a.bias_1) return launch_tb<true>(a, stream, ev);
    return launch_tb<false>(a, stream, ev);
}

}  // namespace ep
