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
// Each thread owns one 16-byte column vector (8 bf16) of one token's output
// row.  The token's destination rows are block-uniform (scalar loads).  For
// each chunk of up to 8 slots, all rows' vectors are loaded before any is
// accumulated, so a thread keeps 8 x 16 bytes in flight; the accumulation
// itself runs in slot order.
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
// Cache policy bits of gfx94x/gfx950 buffer instructions: bit 1 = NT (stream).
constexpr int kStreamLoad = 2;

// Range-checked row view: a load at a byte offset >= `bytes` returns zero and
// touches no memory.  Empty slots get bytes = 0, so their loads are free and
// every slot of a chunk can be loaded without a branch.
__device__ inline __amdgpu_buffer_rsrc_t row_rsrc(const void *base, int64_t row, int32_t bytes,
                                                  bool valid) {
    const char *p = static_cast<const char *>(base) + (valid ? row * bytes : 0);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(p), 0, valid ? bytes : 0,
                                             kRsrcWord3);
}

template <bool HAS_BIAS, bool HAS_W, typename IdxT>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a, int blocks_per_token) {
#pragma clang fp contract(off)
    if (a.scalars[EP_SCALAR_ERROR_BITS] & EP_ERRBIT_FATAL) return;
    const int64_t t = blockIdx.x / blocks_per_token;
    const int64_t v = static_cast<int64_t>(blockIdx.x % blocks_per_token) * blockDim.x + threadIdx.x;
    if (v >= a.row_vecs) return;
    const int K = a.num_topk;
    const int32_t row_bytes = static_cast<int32_t>(a.row_vecs * 16);
    const int32_t col = static_cast<int32_t>(v * 16);
    const IdxT *idx = static_cast<const IdxT *>(a.topk_idx);
    const int32_t *dst = a.dst + t * K;

    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;

    for (int k0 = 0; k0 < K; k0 += kSlotChunk) {
        int32_t r[kSlotChunk];
        u32x4 d[kSlotChunk], bb[kSlotChunk];
#pragma unroll
        for (int j = 0; j < kSlotChunk; ++j) {
            r[j] = (k0 + j < K) ? dst[k0 + j] : -1;
            if (r[j] >= a.capacity) r[j] = -1;          // never read past y
        }
        // Issue every load of the chunk before using any of them.
#pragma unroll
        for (int j = 0; j < kSlotChunk; ++j) {
            const bool ok = r[j] >= 0;
            d[j] = __builtin_amdgcn_raw_buffer_load_b128(row_rsrc(a.y, r[j], row_bytes, ok), col,
                                                         0, kStreamLoad);
            if (HAS_BIAS) {
                const int64_t e = ok ? static_cast<int64_t>(idx[t * K + k0 + j]) : 0;
                const bool e_ok = ok && e >= 0 && e < a.num_experts;
                bb[j] = __builtin_amdgcn_raw_buffer_load_b128(
                    row_rsrc(a.bias, e, row_bytes, e_ok), col, 0, 0);
            }
        }
        // Accumulate in slot order.
#pragma unroll
        for (int j = 0; j < kSlotChunk; ++j) {
            if (r[j] < 0) continue;
            float f[8];
            unpack_bf16x8(d[j], f);
            if (HAS_BIAS) {
                float b[8];
                unpack_bf16x8(bb[j], b);
#pragma unroll
                for (int i = 0; i < 8; ++i) f[i] = f[i] + b[i];
            }
            if (HAS_W) {
                const float wk = a.w[t * K + k0 + j];
#pragma unroll
                for (int i = 0; i < 8; ++i) f[i] = wk * f[i];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = acc[i] + f[i];
        }
    }
    u32x4 o;
    o.x = bf16_rne(acc[0]) | (bf16_rne(acc[1]) << 16);
    o.y = bf16_rne(acc[2]) | (bf16_rne(acc[3]) << 16);
    o.z = bf16_rne(acc[4]) | (bf16_rne(acc[5]) << 16);
    o.w = bf16_rne(acc[6]) | (bf16_rne(acc[7]) << 16);
    __builtin_nontemporal_store(o, static_cast<u32x4 *>(a.out) + t * a.row_vecs + v);
}

template <bool HAS_BIAS, bool HAS_W>
hipError_t launch_bw(const CombineArgs &a, hipStream_t stream) {
    // Block size among 256 / 128 / 64 threads that wastes the fewest lanes
    // on the row's vector count (ties go to the larger block).
    int threads = 256;
    int64_t best = -1;
    for (int b : {256, 128, 64}) {
        const int64_t waste = (a.row_vecs + b - 1) / b * b - a.row_vecs;
        if (best < 0 || waste < best) {
            best = waste;
            threads = b;
        }
    }
    const int bpt = static_cast<int>((a.row_vecs + threads - 1) / threads);
    const int64_t blocks = static_cast<int64_t>(a.num_tokens) * bpt;
    if (blocks == 0) return hipSuccess;
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    if (a.idx_is_i64)
        combine_kernel<HAS_BIAS, HAS_W, int64_t>
            <<<static_cast<unsigned>(blocks), threads, 0, stream>>>(a, bpt);
    else
        combine_kernel<HAS_BIAS, HAS_W, int32_t>
            <<<static_cast<unsigned>(blocks), threads, 0, stream>>>(a, bpt);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, hipStream_t stream) {
    if (a.bias)
        return a.w ? launch_bw<true, true>(a, stream) : launch_bw<true, false>(a, stream);
    return a.w ? launch_bw<false, true>(a, stream) : launch_bw<false, false>(a, stream);
}

}  // namespace ep
