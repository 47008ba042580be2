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
// write it to each of its slots' rows.  Token blocks: one wave per (token,
// pass); the wave loads its pass of the row into registers as 16-byte
// vectors (64 lanes x VPL vectors) and stores it once for every valid slot,
// so x is read from HBM exactly once.  The K destination rows are
// wave-uniform (readlane into scalar registers).  Gap blocks, when zero padding is on: one block per
// (expert, 4-row chunk of the gap), one wave per gap row.
#include "ep_internal.h"
#include "../../include/ep.h"

namespace ep {
namespace {

constexpr int kDispatchThreads = 256;
constexpr int kWavesPerBlock = kDispatchThreads / 64;
constexpr int kGapRowsPerBlock = kWavesPerBlock;

// Launch shape: each wave copies one pass of a token's row, 64 * VPL
// 16-byte vectors, to every slot; EP_DISPATCH_MAX_VPL caps VPL (a smaller
// cap spreads a token over more waves).  The copying kernel keeps 16 VGPRs
// (8 waves per SIMD) and requests a wave's row loads, slot rows and the
// error word together (one round trip to memory before its stores).
// Against an earlier form with 105 VGPRs (4 waves per SIMD) and three
// dependent round trips, interleaved on one box: FP8 prefill dispatch
// (4096 x 7168) 47.9 -> 42.9 us back to back and 51.8 -> 47.0 us after a
// cache flush, decode 34.6 -> 33.0 us after a flush; the bf16 dispatches
// whose outputs exceed the MALL (16384 x 4096, 32768 x 7168) 0-7 % slower
// (bound by HBM writes there).  Capping occupancy at 4 or 6 waves per SIMD
// (EP_DISPATCH_WAVES_PER_EU) was slower at every size (prefill 48.1 / 44.3
// us against 43.3).  A persistent grid of 2-8 blocks per CU whose waves
// walk several passes, each requesting the next pass's loads before storing
// the current one, measured 56-68 us after a flush against 46.4 at prefill
// and 10-12 % slower at 16384 x 4096 and 32768 x 7168.  VPL 2 or 4 gained at 32768 x 7168 on one box and lost
// on another, equal at prefill.  Non-temporal loads of the token rows
// (EP_DISPATCH_NT_LOAD) within 0.5 us of ordinary ones on the prefill
// dispatch and 2-3 % slower at larger sizes in the earlier form, so off.
//
// Stores of the rows: the caller chooses (EP_DISPATCH_STREAMING).  Ordinary
// stores leave the rows in the MALL, dirty, for a consumer that reads them
// next (a grouped GEMM) and for the write-back later; non-temporal
// (streaming) stores send them on to HBM during the call.  FP8 prefill
// (4096 x 7168), interleaved on one box: ordinary 46.1 us after a cache
// flush, 43.3 back to back, 79.0-79.4 us with the write-back of what it
// leaves dirty; streaming 53.0 / 45.8 / 56.6-57.0 us.
#ifndef EP_DISPATCH_MAX_VPL
#define EP_DISPATCH_MAX_VPL 1
#endif
#ifndef EP_DISPATCH_NT_LOAD
#define EP_DISPATCH_NT_LOAD 0
#endif
// Resident blocks per compute unit of a persistent grid for the quantising
// dispatch (0 = one block per work unit, the default: measured equal or
// faster on MI355X).
#ifndef EP_DISPATCH_BLOCKS_PER_CU
#define EP_DISPATCH_BLOCKS_PER_CU 0
#endif
constexpr int kDispatchBlocksPerCu = EP_DISPATCH_BLOCKS_PER_CU;

// Scale packs and per-row weights of a copying dispatch, when the layout's
// source slots are given: moved by blocks of their own in expanded-row order
// (for packs each wave takes kSfRowsPerWave consecutive rows, for weights 64,
// one per lane, so neighbouring rows' values share cache lines written
// together) rather than by each token's first-pass wave, whose stores (224
// bytes of packs, 4 bytes of weight per slot) land one row here, one there
// and leave partly written lines.  At most kSfBlocks such blocks stride over
// the rows below psum[E], placed first in the grid.  Measured on the FP8
// prefill dispatch (4096 x 7168, 56 fp32 packs per row), interleaved runs on
// one box, current kernel: 43.9 -> 42.9 us back to back, 50.1 -> 47.0 us
// after a cache flush; 2048 / 4096 blocks 45.4 / 46.0 us (48.7 / 51.6
// flushed), 8 rows per wave 45.0 (51.1), 2 rows per wave over 4096 blocks
// 45.0 (49.6); a wave taking its 2 or 3 strided row groups at once (every
// source slot, then every pack load requested before any is used) 44.7 /
// 45.2 us (49.5 / 50.5 flushed).  Weights in the earlier form: 53.6 us stored by the token
// waves against 49.0 us without a weight output.
#ifndef EP_DISPATCH_SF_BY_ROW
#define EP_DISPATCH_SF_BY_ROW 1
#endif
#ifndef EP_DISPATCH_SF_ROWS_PER_WAVE
#define EP_DISPATCH_SF_ROWS_PER_WAVE 4
#endif
#ifndef EP_DISPATCH_SF_BLOCKS
#define EP_DISPATCH_SF_BLOCKS 1024
#endif
constexpr int kSfRowsPerWave = EP_DISPATCH_SF_ROWS_PER_WAVE;
constexpr int64_t kSfBlocks = EP_DISPATCH_SF_BLOCKS;

template <bool NT>
__device__ inline void store_row_vec(u32x4 *p, u32x4 v) {
    if constexpr (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// True when the layout's error word holds a bit that voids this call.
__device__ inline bool dispatch_stopped(const DispatchArgs &a) {
    return a.scalars && (a.scalars[EP_SCALAR_ERROR_BITS] & a.stop_bits);
}

// Stores of one pass of token t's row (one wave), held in v, to every valid
// slot row in my_dst (lane k holds slot k's row, -1 if none); pass 0 also
// stores the scale packs and weight when they are not moved in expanded-row
// order.
template <int VPL, bool NT>
__device__ inline void store_token_pass(const DispatchArgs &a, int64_t t, int64_t pass, int lane,
                                        const u32x4 (&v)[VPL], int32_t my_dst) {
    const int64_t V = a.row_vecs;
    const int K = a.num_topk;
    if (pass == 0 && !a.src_meta) {
        if (a.out_w && my_dst >= 0) a.out_w[my_dst] = a.w ? a.w[t * K + lane] : 1.0f;
        // A token's scale packs, 64 at a time: loaded once, stored to every
        // valid slot's row.
        for (int j = lane; j - lane < a.num_sf; j += 64) {
            const uint32_t p = j < a.num_sf ? a.sf[t * a.sf_ts + j * a.sf_hs] : 0u;
            for (int k = 0; k < K; ++k) {
                const int32_t r = __builtin_amdgcn_readlane(my_dst, k);
                if (r >= 0 && j < a.num_sf) a.out_sf[r * a.out_ts + j * a.out_hs] = p;
            }
        }
    }
    u32x4 *out = static_cast<u32x4 *>(a.out_x);
    const int64_t c0 = pass * 64 * VPL;
    for (int k = 0; k < K; ++k) {
        const int32_t r = __builtin_amdgcn_readlane(my_dst, k);
        if (r < 0) continue;
        u32x4 *d = out + static_cast<int64_t>(r) * V;
#pragma unroll
        for (int q = 0; q < VPL; ++q) {
            const int64_t c = c0 + q * 64 + lane;
            if (c < V) store_row_vec<NT>(d + c, v[q]);
        }
    }
}

// Loads of one pass of token t's row and of its slot rows (rows outside
// [0, capacity) become -1, so no layout content can send a store out of
// the output buffers).
template <int VPL>
__device__ inline void load_token_pass(const DispatchArgs &a, int64_t t, int64_t pass, int lane,
                                       u32x4 (&v)[VPL], int32_t &my_dst) {
    const int64_t V = a.row_vecs;
    const int K = a.num_topk;
    const u32x4 *src = static_cast<const u32x4 *>(a.x) + t * V;
    const int64_t c0 = pass * 64 * VPL;
#pragma unroll
    for (int q = 0; q < VPL; ++q) {
        const int64_t c = c0 + q * 64 + lane;
        if (c < V) v[q] = EP_DISPATCH_NT_LOAD ? __builtin_nontemporal_load(src + c) : src[c];
    }
    my_dst = lane < K ? a.dst[t * K + lane] : -1;
    if (my_dst >= a.capacity) my_dst = -1;
}

// Copy one pass of a token's row (one wave: vectors [64*VPL*pass, +64*VPL))
// to every valid slot's row.  The row loads, the slot rows and the error
// word are all requested before the wave waits on any of them (one round
// trip to memory instead of three).
template <int VPL, bool NT>
__device__ inline void dispatch_token(const DispatchArgs &a, int64_t t, int64_t pass, int lane) {
    u32x4 v[VPL];
    int32_t my_dst;
    load_token_pass<VPL>(a, t, pass, lane, v, my_dst);
    if (dispatch_stopped(a)) return;
    store_token_pass<VPL, NT>(a, t, pass, lane, v, my_dst);
}

// Scale packs of kSfRowsPerWave consecutive expanded rows from r0 (one wave):
// each routed row's packs are its source token's (source slot / K); gap rows
// (source -1, zeroed by the gap units when asked) and rows from `end`
// (psum[E]) on are not written.  Packs go 64 at a time (one per lane and
// row), so a row of up to 64 packs takes one load and one store per lane.
__device__ inline void dispatch_sf_rows(const DispatchArgs &a, int64_t r0, int64_t end,
                                        int lane) {
    const int64_t num_slots = static_cast<int64_t>(a.num_tokens) * a.num_topk;
    int64_t tok[kSfRowsPerWave];
#pragma unroll
    for (int i = 0; i < kSfRowsPerWave; ++i) {
        const int64_t r = r0 + i;
        const int32_t slot = r < end ? a.src_meta[r] : -1;
        tok[i] = (slot >= 0 && slot < num_slots) ? slot / a.num_topk : -1;
    }
    for (int j = lane; j - lane < a.num_sf; j += 64) {
        uint32_t v[kSfRowsPerWave];
#pragma unroll
        for (int i = 0; i < kSfRowsPerWave; ++i)
            v[i] = (tok[i] >= 0 && j < a.num_sf) ? a.sf[tok[i] * a.sf_ts + j * a.sf_hs] : 0u;
#pragma unroll
        for (int i = 0; i < kSfRowsPerWave; ++i)
            if (tok[i] >= 0 && j < a.num_sf) a.out_sf[(r0 + i) * a.out_ts + j * a.out_hs] = v[i];
    }
}

// ---------------------------------------------------------------- FP8 quantiser
// The quantising form reads bf16 x and writes E4M3FN codes plus one scale
// pack set per token (per 128-channel block: s = max(amax, 1e-12) / 448 in
// binary32; fp32 packs hold s, UE8M0 packs hold s rounded up to a power of
// two as its exponent byte, four blocks per pack, lowest block in the low
// byte; codes are the nearest E4M3FN value of clamp(x / divisor, +-448),
// ties to even, NaN -> 0x7F).  Lane layout: each lane owns 16 consecutive
// channels (two 16-byte bf16 loads, one 16-byte store of codes), so 8 lanes
// form one block and reduce its amax among themselves.

constexpr int kQuantF32 = EP_SF_F32 + 1;
constexpr int kQuantUe8m0 = EP_SF_UE8M0 + 1;

// Code conversion: with EP_QUANT_HW_CVT (default) the gfx950 packed
// fp32 -> OCP E4M3 conversion (round to nearest even) on values clamped to
// +-448, NaN codes patched to 0x7F; otherwise the integer rounding of
// e4m3_code below.  Both give identical codes (checked against the oracle on
// every bf16 value and on full workloads); the hardware form measured ~6 %
// faster on the fused dispatch.  EP_QUANT_NT_STORE streams the code rows
// past the caches (measured 72 -> 59 us on the prefill dispatch).
#ifndef EP_QUANT_HW_CVT
#define EP_QUANT_HW_CVT 1
#endif
#ifndef EP_QUANT_NT_STORE
#define EP_QUANT_NT_STORE 1
#endif

// binary32 (not NaN) -> E4M3FN code: magnitude clamped to 448, nearest,
// ties to even.  Normal range: round the 23-bit mantissa to 3 bits on the
// bit pattern (a carry moves into the exponent); below 2^-6 the codes are
// the multiples of 2^-9, found by rounding |v| * 512 to an integer.
__device__ inline uint32_t e4m3_code(float v) {
    if (v != v) return 0x7Fu;
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x43E00000u) a = 0x43E00000u;                   // 448
    uint32_t code;
    if (a >= 0x3C800000u)                                    // 2^-6
        code = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
    else
        code = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.0f));
    return code | sign;
}

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

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Largest |x| bf16 bit pattern over the block (the lane's 16 values, two per
// word with packed 16-bit maxima, then the block's 8 lanes).  Non-negative
// bf16 values order like their bits; a NaN pattern orders above infinity, so
// a result of 0x7F80 or more means the block holds an infinity or a NaN.
__device__ inline uint32_t block_max_bits(const u32x4 lo, const u32x4 hi) {
    const uint32_t words[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    u16x2 m = u16x2{0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i)
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, words[i] & 0x7FFF7FFFu));
    uint32_t r = m.x > m.y ? m.x : m.y;
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
        const uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(r), off, 8));
        r = o > r ? o : r;
    }
    return r;
}

// Codes of 16 quotients.  CLAMP: limit them to +-448 first (NaN becomes
// -448 there and is patched by the caller); without it the quotients must
// already lie within one ulp of [-448, 448], which round to +-448.
// EP_QUANT_FAST_CLAMP keeps the clamp on the finite-block path too (with
// it, and the sign fix the negated remainder makes unnecessary, the
// standalone fp32 quantiser measured 19.0 us against 18.1 without).
#ifndef EP_QUANT_FAST_CLAMP
#define EP_QUANT_FAST_CLAMP 0
#endif
template <bool CLAMP>
__device__ inline u32x4 e4m3_pack16(const float v[16]) {
    uint32_t w[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        if (EP_QUANT_HW_CVT) {
            float c[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                c[i] = CLAMP ? __builtin_fminf(__builtin_fmaxf(v[4 * g + i], -448.0f), 448.0f)
                             : v[4 * g + i];
            int word = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
            word = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], word, true);
            w[g] = static_cast<uint32_t>(word);
        } else {
            w[g] = e4m3_code(v[4 * g]) | (e4m3_code(v[4 * g + 1]) << 8) |
                   (e4m3_code(v[4 * g + 2]) << 16) | (e4m3_code(v[4 * g + 3]) << 24);
        }
    }
    return u32x4{w[0], w[1], w[2], w[3]};
}

// Quantise one 16-channel vector pair (lane-owned) of a valid block: returns
// the 16 codes and, in *pack, the block's fp32 scale bits or exponent byte.
//
// Blocks of finite values (the common case) take a short path: fp32 scales
// divide through one correctly rounded reciprocal y = 1/s per block, q0 =
// x*y, then one remainder correction with fused multiply-adds (Markstein's
// division scheme), written as q = q0 - n*y with n = q0*s - x so that
// x = -0 yields -0.  For every bf16 x with |x| <= amax and every block
// maximum amax, this q is the correctly rounded x/s bit for bit wherever
// |x/s| >= 2^-11; below that both give the zero code of x's sign.  A
// host-side test enumerates that whole domain.  The quotients lie within
// one ulp of [-448, 448] (s is amax/448 rounded), so they need no clamp.
// Blocks holding an infinity or a NaN take the general path: NaN skipped in
// amax, true divisions, clamped quotients, NaN codes.
template <int MODE>
__device__ inline u32x4 quantise16(const u32x4 lo, const u32x4 hi, uint32_t *pack) {
#pragma clang fp contract(off)
    float f[16];
    unpack_bf16x8(lo, f);
    unpack_bf16x8(hi, f + 8);
    float v[16];
    const uint32_t mb = block_max_bits(lo, hi);
    if (mb < 0x7F80u) {
        const float amax = __uint_as_float(mb << 16);
        const float s = __fdiv_rn(amax > 1e-12f ? amax : 1e-12f, 448.0f);
        if (MODE == kQuantUe8m0) {
            // s <= 3.4e38 / 448, so the rounded-up power of two 2^k has
            // k <= 126 and x / 2^k equals x * 2^-k exactly.
            uint32_t e = (__float_as_uint(s) >> 23) & 0xFFu;
            if (__float_as_uint(s) & 0x7FFFFFu) ++e;
            *pack = e;
            const float y = __uint_as_float((254u - e) << 23);
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = f[i] * y;
        } else {
            *pack = __float_as_uint(s);
            const float y = __fdiv_rn(1.0f, s);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float q0 = f[i] * y;
                const float n = __builtin_fmaf(q0, s, -f[i]);     // -(x - q0*s), exact
                v[i] = __builtin_fmaf(-n, y, q0);
            }
        }
        return e4m3_pack16<EP_QUANT_FAST_CLAMP != 0>(v);
    }
    // amax on the bit patterns of |x|, NaN patterns skipped, infinity kept.
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t b = __float_as_uint(f[i]) & 0x7FFFFFFFu;
        if (b <= 0x7F800000u && b > m) m = b;
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
        const uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), off, 8));
        m = o > m ? o : m;
    }
    const float amax = __uint_as_float(m);
    const float s = __fdiv_rn(amax > 1e-12f ? amax : 1e-12f, 448.0f);
    float divisor = s;
    if (MODE == kQuantUe8m0) {
        uint32_t e = (__float_as_uint(s) >> 23) & 0xFFu;
        if (__float_as_uint(s) & 0x7FFFFFu) ++e;
        divisor = __uint_as_float(e << 23);
        *pack = e;
    } else {
        *pack = __float_as_uint(s);
    }
    if (MODE == kQuantUe8m0 && __float_as_uint(divisor) < (254u << 23)) {
        // x / 2^k equals x * 2^-k exactly: both are the exact quotient rounded
        // once, and 2^-k (k <= 126 here, a normal number) is representable.
        // Larger divisors (beyond any finite bf16 block) keep the division.
        const float y = __uint_as_float((254u << 23) - __float_as_uint(divisor));
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = f[i] * y;
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = __fdiv_rn(f[i], divisor);
    }
    u32x4 codes = e4m3_pack16<true>(v);
    uint32_t w[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (v[4 * g + i] != v[4 * g + i])
                w[g] = (w[g] & ~(0xFFu << (8 * i))) | (0x7Fu << (8 * i));
    return u32x4{w[0], w[1], w[2], w[3]};
}

// Received top-k ids and weights of token t at its rank row r (lanes below
// meta_topk): an id outside [0, num_experts) is written as -1 with weight 0.
__device__ inline void rank_meta(const DispatchArgs &a, int64_t t, int64_t r, int lane) {
    const int K = a.meta_topk;
    if (lane >= K) return;
    const int64_t e = a.meta_i64 ? static_cast<const int64_t *>(a.meta_idx)[t * K + lane]
                                 : static_cast<const int32_t *>(a.meta_idx)[t * K + lane];
    const bool valid = e >= 0 && e < a.num_experts;
    if (a.out_meta_idx) {
        if (a.meta_i64) static_cast<int64_t *>(a.out_meta_idx)[r * K + lane] = valid ? e : -1;
        else static_cast<int32_t *>(a.out_meta_idx)[r * K + lane] =
                 valid ? static_cast<int32_t>(e) : -1;
    }
    if (a.out_meta_w)
        a.out_meta_w[r * K + lane] = valid ? (a.meta_w ? a.meta_w[t * K + lane] : 1.0f) : 0.0f;
}

// Quantise one pass of a token's row (one wave: code vectors [c0, c0 +
// 64*QPL)) and store codes and scale packs to every valid slot's row; pass 0
// also stores the weight, or for a rank row the received ids and weights.
// Without a slot index (plain quantiser) the token's own row t is the one
// destination.
template <int QPL, int MODE>
__device__ inline void quant_token(const DispatchArgs &a, int64_t t, int64_t pass, int lane) {
    const int64_t V = a.row_vecs;                 // 16-byte code vectors per row
    u32x4 *out = static_cast<u32x4 *>(a.out_x);
    const int K = a.dst ? a.num_topk : 1;
    int32_t my_dst = a.dst ? (lane < K ? a.dst[t * K + lane] : -1)
                           : (lane == 0 ? static_cast<int32_t>(t) : -1);
    if (my_dst >= a.capacity) my_dst = -1;
    if (pass == 0 && a.out_w && my_dst >= 0) a.out_w[my_dst] = a.w ? a.w[t * K + lane] : 1.0f;
    if (pass == 0 && (a.out_meta_idx || a.out_meta_w)) {
        const int32_t r = __builtin_amdgcn_readlane(my_dst, 0);   // lane 0 holds the one row
        if (r >= 0) rank_meta(a, t, r, lane);
    }
    const u32x4 *src = static_cast<const u32x4 *>(a.x) + t * 2 * V;
    const int64_t c0 = pass * 64 * QPL;
    u32x4 v[QPL];
    uint32_t pk[QPL];
#pragma unroll
    for (int q = 0; q < QPL; ++q) {
        const int64_t c = c0 + q * 64 + lane;
        u32x4 lo = u32x4{0u, 0u, 0u, 0u}, hi = lo;
        if (c < V) {
            lo = src[2 * c];
            hi = src[2 * c + 1];
        }
        uint32_t p = 0;
        v[q] = quantise16<MODE>(lo, hi, &p);
        if (c >= V) p = 0;
        if (MODE == kQuantUe8m0) {
            // lanes 0 and 32 of each pass gather their four blocks' bytes
            const uint32_t b1 = static_cast<uint32_t>(__shfl(static_cast<int>(p), lane + 8));
            const uint32_t b2 = static_cast<uint32_t>(__shfl(static_cast<int>(p), lane + 16));
            const uint32_t b3 = static_cast<uint32_t>(__shfl(static_cast<int>(p), lane + 24));
            p = p | (b1 << 8) | (b2 << 16) | (b3 << 24);
        }
        pk[q] = p;
    }
    for (int k = 0; k < K; ++k) {
        const int32_t r = __builtin_amdgcn_readlane(my_dst, k);
        if (r < 0) continue;
        u32x4 *d = out + static_cast<int64_t>(r) * V;
#pragma unroll
        for (int q = 0; q < QPL; ++q) {
            const int64_t c = c0 + q * 64 + lane;
            if (c >= V) continue;
            if (EP_QUANT_NT_STORE) __builtin_nontemporal_store(v[q], d + c);
            else d[c] = v[q];
            const bool writer = MODE == kQuantUe8m0 ? (lane & 31) == 0 : (lane & 7) == 0;
            if (writer) {
                const int64_t j = MODE == kQuantUe8m0 ? c / 32 : c / 8;
                a.out_sf[r * a.out_ts + j * a.out_hs] = pk[q];
            }
        }
    }
}

// Zero one alignment-gap row (one wave): rows [psum[e] + counts[e], psum[e+1]).
template <bool NT>
__device__ inline void dispatch_gap_row(const DispatchArgs &a, int e, int64_t r, int lane) {
    if (r >= a.psum[e + 1] || r >= a.capacity) return;
    const int64_t V = a.row_vecs;
    const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
    u32x4 *d = static_cast<u32x4 *>(a.out_x) + r * V;
    for (int64_t c = lane; c < V; c += 64) store_row_vec<NT>(d + c, zero);
    for (int j = lane; j < a.num_sf; j += 64) a.out_sf[r * a.out_ts + j * a.out_hs] = 0u;
    if (a.out_w && lane == 0) a.out_w[r] = 0.0f;
}

// Copying dispatch, one work unit per block: blocks [0, sf_units) move the
// scale packs and weights in expanded-row order (when the layout's source
// slots are given), the next token_units blocks give each wave one (token,
// pass) to copy, the rest zero kGapRowsPerBlock gap rows each.  No loop over
// units: the kernel keeps few registers live (8 waves per SIMD).
#ifndef EP_DISPATCH_WAVES_PER_EU
#define EP_DISPATCH_WAVES_PER_EU 8
#endif
template <int VPL, bool NT>
__global__ __launch_bounds__(kDispatchThreads)
__attribute__((amdgpu_waves_per_eu(1, EP_DISPATCH_WAVES_PER_EU))) void dispatch_copy_kernel(DispatchArgs a,
                                                                        int64_t sf_units,
                                                                        int64_t token_units,
                                                                        int gap_chunks,
                                                                        int passes) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t u0 = blockIdx.x;
    if (u0 < sf_units) {
        if (dispatch_stopped(a)) return;
        // Rows below psum[E], striding over the sf_units blocks.
        const int64_t e = a.psum[a.num_experts];
        const int64_t end = e < a.capacity ? e : a.capacity;
        if (a.num_sf) {
            const int64_t step = sf_units * kWavesPerBlock * kSfRowsPerWave;
            for (int64_t r0 = (u0 * kWavesPerBlock + wave) * kSfRowsPerWave; r0 < end; r0 += step)
                dispatch_sf_rows(a, r0, end, lane);
        }
        if (a.out_w) {
            // Weights: 64 consecutive rows per wave, one per lane.
            const int64_t num_slots = static_cast<int64_t>(a.num_tokens) * a.num_topk;
            const int64_t wstep = sf_units * kWavesPerBlock * 64;
            for (int64_t r = (u0 * kWavesPerBlock + wave) * 64 + lane; r < end; r += wstep) {
                const int32_t slot = a.src_meta[r];
                if (slot >= 0 && slot < num_slots) a.out_w[r] = a.w ? a.w[slot] : 1.0f;
            }
        }
        return;
    }
    const int64_t u = u0 - sf_units;
    if (u < token_units) {
        const int64_t wv = u * kWavesPerBlock + wave;
        const int64_t t = wv / passes;
        if (t < a.num_tokens) dispatch_token<VPL, NT>(a, t, wv - t * passes, lane);
        return;
    }
    if (dispatch_stopped(a)) return;
    const int64_t g = u - token_units;
    const int e = static_cast<int>(g / gap_chunks);
    const int64_t chunk = g - static_cast<int64_t>(e) * gap_chunks;
    const int64_t r = static_cast<int64_t>(a.psum[e]) + a.counts[e] + chunk * kGapRowsPerBlock +
                      wave;
    dispatch_gap_row<NT>(a, e, r, lane);
}

// Quantising dispatch over work units (one block per unit unless a
// persistent grid is configured): units [0, token_units) give each wave one
// (token, pass) to quantise, `passes` per token; the rest zero
// kGapRowsPerBlock gap rows each.
template <int VPL, int MODE>
__global__ __launch_bounds__(kDispatchThreads) void dispatch_kernel(DispatchArgs a,
                                                                   int64_t token_units,
                                                                   int64_t total_units,
                                                                   int gap_chunks, int passes) {
    if (dispatch_stopped(a)) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int64_t u = blockIdx.x; u < total_units; u += gridDim.x) {
        if (u < token_units) {
            const int64_t wv = u * kWavesPerBlock + wave;
            const int64_t t = wv / passes;
            if (t >= a.num_tokens) continue;
            quant_token<VPL, MODE>(a, t, wv % passes, lane);
        } else {
            const int64_t g = u - token_units;
            const int e = static_cast<int>(g / gap_chunks);
            const int64_t chunk = g % gap_chunks;
            const int64_t r = static_cast<int64_t>(a.psum[e]) + a.counts[e] +
                              chunk * kGapRowsPerBlock + wave;
            dispatch_gap_row<false>(a, e, r, lane);
        }
    }
}

template <int VPL, int MODE>
hipError_t launch_vpl(const DispatchArgs &a, hipStream_t stream, CallEvents ev) {
    const int64_t passes = (a.row_vecs + 64 * VPL - 1) / (64 * VPL);
    const int64_t token_units = (a.num_tokens * passes + kWavesPerBlock - 1) / kWavesPerBlock;
    int gap_chunks = 0;
    if (a.zero_padding && a.alignment > 1)
        gap_chunks = (a.alignment - 1 + kGapRowsPerBlock - 1) / kGapRowsPerBlock;
    const int64_t gap_units = static_cast<int64_t>(gap_chunks) * a.num_experts;
    if constexpr (MODE != 0) {
        const int64_t total = token_units + gap_units;
        const int64_t blocks = persistent_grid(total, kDispatchBlocksPerCu);
        if (blocks == 0) return hipSuccess;
        if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
        return launch_kernel(dispatch_kernel<VPL, MODE>, dim3(static_cast<unsigned>(blocks)),
                             dim3(kDispatchThreads), stream, ev.start, ev.stop, a, token_units,
                             total, gap_chunks > 0 ? gap_chunks : 1, static_cast<int>(passes));
    } else {
    DispatchArgs b = a;
    int64_t sf_units = 0;
    // Only where routed rows fill a good part of the buffer: the scale units
    // stride over every row below psum[E], gap rows included, so with sparse
    // routing (decode: 1024 slots in 33536 rows) they would cost more than
    // the token waves' stores they replace.
    const int64_t slots = static_cast<int64_t>(a.num_tokens) * a.num_topk;
    if (EP_DISPATCH_SF_BY_ROW && a.src_meta && (a.num_sf > 0 || a.out_w) && slots > 0 &&
        slots * 4 >= a.capacity) {
        const int64_t rows_per_unit = kWavesPerBlock * (a.num_sf > 0 ? kSfRowsPerWave : 64);
        sf_units = (a.capacity + rows_per_unit - 1) / rows_per_unit;
        if (sf_units > kSfBlocks) sf_units = kSfBlocks;
    }
    if (sf_units == 0) b.src_meta = nullptr;      // token waves copy packs and weights
    const int64_t blocks = sf_units + token_units + gap_units;
    if (blocks == 0) return hipSuccess;
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    const int gc = gap_chunks > 0 ? gap_chunks : 1;
    const int np = static_cast<int>(passes);
    if (a.streaming)
        return launch_kernel(dispatch_copy_kernel<VPL, true>, dim3(static_cast<unsigned>(blocks)),
                             dim3(kDispatchThreads), stream, ev.start, ev.stop, b, sf_units,
                             token_units, gc, np);
    return launch_kernel(dispatch_copy_kernel<VPL, false>, dim3(static_cast<unsigned>(blocks)),
                         dim3(kDispatchThreads), stream, ev.start, ev.stop, b, sf_units,
                         token_units, gc, np);
    }
}

// Most code vectors a lane holds per pass of the quantiser; each pass of a
// row is its own wave, so a smaller value spreads a token over more waves
// (prefill, hidden 7168: 1 -> 49.7 us, 2 -> 52.1, 4 -> 55.3, 8 -> 60.2).
#ifndef EP_QUANT_MAX_QPL
#define EP_QUANT_MAX_QPL 1
#endif

template <int MODE>
hipError_t launch_quant(const DispatchArgs &a, hipStream_t stream, CallEvents ev) {
    const int64_t per_lane = (a.row_vecs + 63) / 64;
    if (per_lane <= 1 || EP_QUANT_MAX_QPL == 1) return launch_vpl<1, MODE>(a, stream, ev);
    if (per_lane <= 2 || EP_QUANT_MAX_QPL == 2) return launch_vpl<2, MODE>(a, stream, ev);
    if (per_lane <= 4 || EP_QUANT_MAX_QPL == 4) return launch_vpl<4, MODE>(a, stream, ev);
    return launch_vpl<8, MODE>(a, stream, ev);
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs &a, hipStream_t stream, CallEvents ev) {
    if (a.quant == kQuantF32) return launch_quant<kQuantF32>(a, stream, ev);
    if (a.quant == kQuantUe8m0) return launch_quant<kQuantUe8m0>(a, stream, ev);
    const int64_t per_lane = (a.row_vecs + 63) / 64;
    if (per_lane <= 1 || EP_DISPATCH_MAX_VPL == 1) return launch_vpl<1, 0>(a, stream, ev);
    if (per_lane <= 2 || EP_DISPATCH_MAX_VPL == 2) return launch_vpl<2, 0>(a, stream, ev);
    if (per_lane <= 4 || EP_DISPATCH_MAX_VPL == 4) return launch_vpl<4, 0>(a, stream, ev);
    if (per_lane <= 8 || EP_DISPATCH_MAX_VPL == 8) return launch_vpl<8, 0>(a, stream, ev);
    return launch_vpl<16, 0>(a, stream, ev);
}

}  // namespace ep
