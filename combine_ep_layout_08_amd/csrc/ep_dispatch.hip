// Dispatch copy epilogue into the expert-expanded layout on gfx950.
//
// What is computed follows DeepEP notes ch.7 "V2: how dispatch builds expert
// inputs": s7.1 (x is a bf16 matrix or FP8 bytes plus scale factors, here
// any 4-byte packs: fp32 per 128 channels or packed UE8M0 exponents;
// top-k weights optional), s7.3 (the copy epilogue writes each received row
// into its expert's aligned range, copies scale factors with their own token
// and hidden strides and the received weights, and optionally zero-fills the
// alignment gaps), s7.4 (contiguous aligned expert ranges for grouped GEMM).
//
// On one GPU the whole epilogue is HBM traffic: read every token row once and
// write it to each of its slots' rows.  Token blocks: one wave per token; the
// wave loads the row into registers as 16-byte vectors (64 lanes x VPL vectors
// per chunk) and stores the chunk once for every valid slot, so x is read
// from HBM exactly once.  The K destination rows are wave-uniform (readlane
// into scalar registers).  Gap blocks, when zero padding is on: one block per
// (expert, 4-row chunk of the gap), one wave per gap row.
#include "ep_internal.h"
#include "../../include/ep.h"

namespace ep {
namespace {

constexpr int kDispatchThreads = 256;
constexpr int kWavesPerBlock = kDispatchThreads / 64;
constexpr int kGapRowsPerBlock = kWavesPerBlock;

// Launch shape: waves that share one token's row (each copies a contiguous
// part of it), and whether row stores are non-temporal (streamed past the
// caches).
#ifndef EP_DISPATCH_WAVES_PER_TOKEN
#define EP_DISPATCH_WAVES_PER_TOKEN 1
#endif
#ifndef EP_DISPATCH_NT_STORE
#define EP_DISPATCH_NT_STORE 0
#endif
// Resident blocks per compute unit of a persistent grid (0 = one block per
// work unit, the default: measured equal or faster on MI355X).
#ifndef EP_DISPATCH_BLOCKS_PER_CU
#define EP_DISPATCH_BLOCKS_PER_CU 0
#endif
constexpr int kDispatchBlocksPerCu = EP_DISPATCH_BLOCKS_PER_CU;
constexpr int kWavesPerToken = EP_DISPATCH_WAVES_PER_TOKEN;
constexpr int kTokensPerBlock = kWavesPerBlock / kWavesPerToken;
static_assert(kWavesPerBlock % kWavesPerToken == 0, "waves per token must divide 4");

__device__ inline void store_row_vec(u32x4 *p, u32x4 v) {
    if (EP_DISPATCH_NT_STORE)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// Copy one token's part of the row (one wave) to every valid slot's row.
template <int VPL>
__device__ inline void dispatch_token(const DispatchArgs &a, int64_t t, int part, int lane) {
    const int64_t V = a.row_vecs;
    u32x4 *out = static_cast<u32x4 *>(a.out_x);
    const int K = a.num_topk;
    // Rows outside [0, capacity) are skipped, so no layout content can send a
    // store out of the output buffers.
    int32_t my_dst = lane < K ? a.dst[t * K + lane] : -1;
    if (my_dst >= a.capacity) my_dst = -1;
    if (part == 0) {
        if (a.out_w && my_dst >= 0) a.out_w[my_dst] = a.w ? a.w[t * K + lane] : 1.0f;
        if (a.num_sf) {
            // A token's scale packs (at most 64 * kMaxSfPerLane) go to
            // registers once and are stored for every valid slot.
            uint32_t sfv[kMaxSfPerLane];
#pragma unroll
            for (int q = 0; q < kMaxSfPerLane; ++q) {
                const int j = lane + 64 * q;
                sfv[q] = j < a.num_sf ? a.sf[t * a.sf_ts + j * a.sf_hs] : 0u;
            }
            for (int k = 0; k < K; ++k) {
                const int32_t r = __builtin_amdgcn_readlane(my_dst, k);
                if (r < 0) continue;
#pragma unroll
                for (int q = 0; q < kMaxSfPerLane; ++q) {
                    const int j = lane + 64 * q;
                    if (j < a.num_sf) a.out_sf[r * a.out_ts + j * a.out_hs] = sfv[q];
                }
            }
        }
    }
    const int64_t per_part = (V + kWavesPerToken - 1) / kWavesPerToken;
    const int64_t p0 = part * per_part;
    const int64_t p1 = p0 + per_part < V ? p0 + per_part : V;
    const u32x4 *src = static_cast<const u32x4 *>(a.x) + t * V;
    for (int64_t c0 = p0; c0 < p1; c0 += 64 * VPL) {
        u32x4 v[VPL];
#pragma unroll
        for (int q = 0; q < VPL; ++q) {
            const int64_t c = c0 + q * 64 + lane;
            if (c < p1) v[q] = src[c];
        }
        for (int k = 0; k < K; ++k) {
            const int32_t r = __builtin_amdgcn_readlane(my_dst, k);
            if (r < 0) continue;
            u32x4 *d = out + static_cast<int64_t>(r) * V;
#pragma unroll
            for (int q = 0; q < VPL; ++q) {
                const int64_t c = c0 + q * 64 + lane;
                if (c < p1) store_row_vec(d + c, v[q]);
            }
        }
    }
}

// Zero one alignment-gap row (one wave): rows [psum[e] + counts[e], psum[e+1]).
__device__ inline void dispatch_gap_row(const DispatchArgs &a, int e, int64_t r, int lane) {
    if (r >= a.psum[e + 1] || r >= a.capacity) return;
    const int64_t V = a.row_vecs;
    const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
    u32x4 *d = static_cast<u32x4 *>(a.out_x) + r * V;
    for (int64_t c = lane; c < V; c += 64) store_row_vec(d + c, zero);
    for (int j = lane; j < a.num_sf; j += 64) a.out_sf[r * a.out_ts + j * a.out_hs] = 0u;
    if (a.out_w && lane == 0) a.out_w[r] = 0.0f;
}

// Grid over work units (one block per unit unless a persistent grid is
// configured): units [0, token_units) copy kTokensPerBlock tokens each, the
// rest zero kGapRowsPerBlock gap rows each.
template <int VPL>
__global__ __launch_bounds__(kDispatchThreads) void dispatch_kernel(DispatchArgs a,
                                                                   int64_t token_units,
                                                                   int64_t total_units,
                                                                   int gap_chunks) {
    if (a.scalars[EP_SCALAR_ERROR_BITS] & EP_ERRBIT_FATAL) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int64_t u = blockIdx.x; u < total_units; u += gridDim.x) {
        if (u < token_units) {
            const int64_t t = u * kTokensPerBlock + wave / kWavesPerToken;
            if (t < a.num_tokens) dispatch_token<VPL>(a, t, wave % kWavesPerToken, lane);
        } else {
            const int64_t g = u - token_units;
            const int e = static_cast<int>(g / gap_chunks);
            const int64_t chunk = g % gap_chunks;
            const int64_t r = static_cast<int64_t>(a.psum[e]) + a.counts[e] +
                              chunk * kGapRowsPerBlock + wave;
            dispatch_gap_row(a, e, r, lane);
        }
    }
}

template <int VPL>
hipError_t launch_vpl(const DispatchArgs &a, hipStream_t stream, CallEvents ev) {
    const int64_t token_units = (a.num_tokens + kTokensPerBlock - 1) / kTokensPerBlock;
    int gap_chunks = 0;
    if (a.zero_padding && a.alignment > 1)
        gap_chunks = (a.alignment - 1 + kGapRowsPerBlock - 1) / kGapRowsPerBlock;
    const int64_t total = token_units + static_cast<int64_t>(gap_chunks) * a.num_experts;
    const int64_t blocks = persistent_grid(total, kDispatchBlocksPerCu);
    if (blocks == 0) return hipSuccess;
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    return launch_kernel(dispatch_kernel<VPL>, dim3(static_cast<unsigned>(blocks)),
                         dim3(kDispatchThreads), stream, ev.start, ev.stop, a, token_units, total,
                         gap_chunks > 0 ? gap_chunks : 1);
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs &a, hipStream_t stream, CallEvents ev) {
    const int64_t per_wave = (a.row_vecs + kWavesPerToken - 1) / kWavesPerToken;
    const int64_t per_lane = (per_wave + 63) / 64;
    if (per_lane <= 1) return launch_vpl<1>(a, stream, ev);
    if (per_lane <= 2) return launch_vpl<2>(a, stream, ev);
    if (per_lane <= 4) return launch_vpl<4>(a, stream, ev);
    if (per_lane <= 8) return launch_vpl<8>(a, stream, ev);
    return launch_vpl<16>(a, stream, ev);
}

}  // namespace ep
