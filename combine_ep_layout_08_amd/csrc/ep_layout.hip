// Routing layout on gfx950: per-expert counts, aligned exclusive prefix sums,
// the expanded row of every slot and the source slot of every expanded row.
//
// What is computed follows DeepEP notes ch.7 "V2: how dispatch builds expert
// inputs" (s7.1 input contract, -1 = empty slot; s7.2 counts / source metadata
// / slot index produced with dispatch; s7.3 expanded layout with per-expert
// alignment; s7.5 handle fields).  Inside an expert's segment rows follow the
// ascending slot index t*K+k (a stable counting sort).
//
// Three forms.  A batch that fits in one tile (at most 2048 slots) is laid
// out in one launch (layout_single, below; tiny 64 x 4 and decode 128 x 8:
// 11-13 -> 6 us).  Larger batches take two kernels over tiles of whole
// tokens.  Up to kCountPlaceMaxTiles long tiles (819200 slots):
// layout_count + layout_place (below), which exchange the tiles' counts
// through the kernel boundary and never wait on another block; measured
// 1-2 us faster than the lookback form at every size from 64 x 4 to
// 32768 x 8 slots.  Batches that fit in kSmallTilesMax short tiles
// (4 rounds, 1024 slots) use those: twice the blocks share the ranking, and
// every place thread still reads all tiles' counts in one or two round trips
// (prefill 4096 x 8: 16.3 -> 14.5 us).  Beyond kCountPlaceMaxTiles long
// tiles, where every place block reads too many tiles' counts, the
// single-pass lookback.  Cache-cold, K 8, E 256, one box, count + place
// against lookback: 257 tiles 35.6 / 40.6 us, 274 tiles 38.6 / 42.0, 391
// tiles 48.3 / 55.7, 512 tiles 85.6 / 69.8, 768 tiles 132.8 / 95.9, 1024
// tiles 224.9 / 124.7 (a lookback window of 32 or 64 predecessors instead
// of 16: 47.5 / 57.0 us at 274 tiles).  The lookback form:
//  1. layout_scan: one 256-thread block per long tile of whole tokens (at
//     most kTileSlots slots).  The block first loads all of its ids (every load in
//     flight at once), then each wave takes 64 slots per round: lanes holding
//     the same bucket find each other with one ballot per bucket-id bit
//     (match-any), a lane's rank is the popcount of matching lower lanes, and
//     the group leader bumps the wave's LDS counter.  An LDS pass over the 4
//     waves turns per-wave counts into in-tile offsets and the tile histogram.
//     Buckets: 0..E-1 the experts, E the ids outside [-1, E), E+1 the tokens
//     with a valid slot (a tile holds whole tokens, so it can count them).
//     A decoupled lookback over earlier tiles - one 64-bit status word per
//     (tile, bucket) holding epoch, aggregate/prefix flag and count, read and
//     written with agent-scope atomics so every XCD sees them - gives each
//     bucket's exclusive offset; each thread reads a window of 16 predecessors
//     per round trip.  Each valid slot gets its position inside its expert's
//     run, and each received token its rank-layout row (a block scan of the
//     tile's token flags after the earlier tiles' received count).  The tile
//     with the last ticket owns the inclusive totals: it writes counts, runs
//     the aligned block scan over experts into psum and sets the scalars.
//     Tiles take their index from an atomic ticket, so every tile a block
//     waits on has already started and waits end; a spin bound turns a
//     broken invariant into an error bit instead of a hang.
//  2. layout_finalize: thread per slot adds psum[e] to the position and
//     scatters the source metadata; one block per expert marks its alignment
//     gap with -1; block 0 bumps the epoch and resets the ticket.
#include "ep_internal.h"
#include "../../include/ep.h"

#include <mutex>

namespace ep {
namespace {

constexpr uint64_t kFlagAggregate = 1;
constexpr uint64_t kFlagPrefix = 2;
constexpr uint32_t kMaxSpins = 1u << 21;
#ifndef EP_LAYOUT_LOOKBACK_WINDOW
#define EP_LAYOUT_LOOKBACK_WINDOW 16
#endif
constexpr int kLookbackWindow = EP_LAYOUT_LOOKBACK_WINDOW;
constexpr int kBucketsPerThread = (kMaxBuckets + kLayoutThreads - 1) / kLayoutThreads;

__device__ inline uint64_t pack_status(uint32_t epoch, uint64_t flag, uint32_t value) {
    return (static_cast<uint64_t>(epoch) << 34) | (flag << 32) | value;
}

__device__ inline void store_status(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline uint64_t load_status(const uint64_t *p) {
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline int64_t align_up(int64_t c, int64_t a) { return (c + a - 1) / a * a; }

// Exclusive scan of one int64 per thread over a 256-thread block.
__device__ int64_t block_exclusive_scan(int64_t v, int64_t *s_wave, int64_t *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int64_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int64_t base = 0, sum = 0;
#pragma unroll
    for (int w = 0; w < kLayoutWaves; ++w) {
        const int64_t s = s_wave[w];
        if (w < wave) base += s;
        sum += s;
    }
    *total = sum;
    return base + x - v;
}

// Sum of the counts of tiles [0, tile) for one bucket, by decoupled lookback:
// each round trip reads up to kLookbackWindow predecessors at once and adds
// published aggregates up to the first prefix (done) or the first tile that
// has not published yet (poll it again).  Returns false if the spin bound
// was hit.
__device__ bool lookback(const uint64_t *status, int NB, int tile, int b, uint32_t epoch,
                         uint32_t *excl_out) {
    uint32_t excl = 0, spins = 0;
    int j = tile - 1;
    bool done = false;
    while (!done && j >= 0) {
        uint64_t s[kLookbackWindow];
#pragma unroll
        for (int w = 0; w < kLookbackWindow; ++w)
            s[w] = j - w >= 0 ? load_status(&status[static_cast<int64_t>(j - w) * NB + b]) : 0;
        int used = 0;
        bool blocked = false;
#pragma unroll
        for (int w = 0; w < kLookbackWindow; ++w) {
            if (done || blocked || j - w < 0) continue;
            const uint32_t tag = static_cast<uint32_t>(s[w] >> 34);
            const uint32_t flag = static_cast<uint32_t>(s[w] >> 32) & 3u;
            if (tag != epoch || flag == 0) {             // not published yet
                blocked = true;
                continue;
            }
            excl += static_cast<uint32_t>(s[w]);
            used = w + 1;
            if (flag == kFlagPrefix) done = true;
        }
        if (done) break;
        if (used == 0) {
            if (++spins > kMaxSpins) {
                *excl_out = excl;
                return false;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        j -= used;
    }
    *excl_out = excl;
    return true;
}

// Work of one tile shared by both layout forms.  Loads every id of the tile
// (all loads in flight), ranks each slot inside its wave by match-any (lanes
// with the same bucket find each other with one ballot per bucket-id bit; a
// lane's rank is the popcount of matching lower lanes; the group leader bumps
// the wave's LDS counter), flags received tokens in s_tok and counts them
// into bucket E+1, then turns the per-wave counts in s_hist into in-tile
// offsets, in place for every thread of the block on return.  Returns each
// slot's bucket (-1 empty, E invalid) and rank inside
// its wave, and in agg[q] the tile's count of bucket tid + q * kLayoutThreads.
template <typename IdxT, int R>
__device__ void rank_tile(const LayoutArgs &a, int64_t tile_base, int64_t tile_end,
                          int tokens_per_tile, int32_t (*s_hist)[kMaxBuckets], uint8_t *s_tok,
                          int bucket[R], int rank[R],
                          int32_t agg[kBucketsPerThread]) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = a.num_experts, NB = E + 2, K = a.num_topk;
    const int64_t wave_base = tile_base + static_cast<int64_t>(wave) * (R * 64);
    const IdxT *idx = static_cast<const IdxT *>(a.topk_idx);
    int64_t ids[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t i = wave_base + j * 64 + lane;
        ids[j] = i < tile_end ? static_cast<int64_t>(idx[i]) : -1;
    }
    for (int w = 0; w < kLayoutWaves; ++w)
        for (int b = tid; b < NB; b += kLayoutThreads) s_hist[w][b] = 0;
    for (int i = tid; i < kLayoutThreads * R; i += kLayoutThreads) s_tok[i] = 0;
    __syncthreads();
    const int nbits = 32 - __builtin_clz(static_cast<unsigned>(E));   // bits of 0..E
    const uint64_t below = (1ull << lane) - 1ull;
    // token of a slot inside the tile: s / K as a multiply-high by
    // ceil(2^32 / K), exact for s < 2^32 / K (here s < kLayoutThreads * R)
    const uint32_t k_magic = 0xFFFFFFFFu / static_cast<uint32_t>(K) + 1u;
    const uint32_t wave_slot0 = static_cast<uint32_t>(wave_base - tile_base);
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t e = ids[j];
        const int b = (e >= 0 && e < E) ? static_cast<int>(e) : (e == -1 ? -1 : E);
        uint64_t match = __ballot(b >= 0);
        for (int bit = 0; bit < nbits; ++bit) {
            const bool one = (b >> bit) & 1;
            const uint64_t bal = __ballot(one);
            match &= one ? bal : ~bal;
        }
        int r = 0;
        if (b >= 0) {
            const int before = __popcll(match & below);
            const int old = s_hist[wave][b];
            if (before == 0) s_hist[wave][b] = old + __popcll(match);
            r = old + before;
            if (b < E)                                 // this token has a valid slot
                s_tok[K == 1 ? wave_slot0 + j * 64 + lane
                             : __umulhi(wave_slot0 + j * 64 + lane, k_magic)] = 1;
        }
        bucket[j] = b;
        rank[j] = r;
    }
    __syncthreads();

    // Received tokens of the tile go into bucket E+1 (one partial per wave).
    {
        int c = 0;
        for (int i = tid; i < tokens_per_tile; i += kLayoutThreads) c += s_tok[i];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off, 64);
        if (lane == 0) s_hist[wave][E + 1] = c;
    }
    __syncthreads();

    // Per-wave counts -> in-tile offsets; tile aggregate per bucket.
#pragma unroll
    for (int q = 0; q < kBucketsPerThread; ++q) {
        const int b = tid + q * kLayoutThreads;
        agg[q] = 0;
        if (b < NB) {
            int32_t run = 0;
#pragma unroll
            for (int w = 0; w < kLayoutWaves; ++w) {
                const int32_t c = s_hist[w][b];
                s_hist[w][b] = run;
                run += c;
            }
            agg[q] = run;
        }
    }
    // Each bucket's offsets were written by the thread that owns the bucket;
    // callers read s_hist[wave][b] for their own slots' buckets, so every
    // offset must be in place before any thread goes on.
    __syncthreads();
}

// Aligned exclusive scan of the experts' totals (s_total, buckets 0..E+1)
// into s_psum, and the call's error verdict in *s_fatal (nonzero: capacity
// exceeded or an earlier timeout, passed in as the error word `sticky`; the
// layout is void).  Every block that
// calls it on the same totals gets the same result; with `publish` the block
// also writes the scalars, counts, psum and cumulative stats.  Ends after a
// block barrier.
__device__ void scan_experts(const LayoutArgs &a, const int32_t *s_total, int32_t *s_psum,
                             int64_t *s_wave, int32_t *s_fatal, bool publish, uint32_t sticky) {
    const int tid = threadIdx.x, E = a.num_experts;
    const int per = (E + kLayoutThreads - 1) / kLayoutThreads;
    const int b0 = tid * per;
    const int b1 = min(b0 + per, E);
    int64_t local = 0;
    for (int b = b0; b < b1; ++b) local += align_up(s_total[b], a.alignment);
    int64_t total = 0;
    int64_t run = block_exclusive_scan(local, s_wave, &total);
    for (int b = b0; b < b1; ++b) {
        s_psum[b] = static_cast<int32_t>(min(run, static_cast<int64_t>(INT32_MAX)));
        run += align_up(s_total[b], a.alignment);
    }
    if (tid == 0) {
        s_psum[E] = static_cast<int32_t>(min(total, static_cast<int64_t>(INT32_MAX)));
        // Every block reaches the same verdict: the capacity test uses the
        // same totals, and the sticky timeout bit (`sticky`, read when the
        // caller's kernel started) is the same in every block.
        uint32_t err = sticky & EP_ERRBIT_SCAN_TIMEOUT;
        if (total > a.capacity) err |= EP_ERRBIT_CAPACITY;
        if (s_total[E] > 0) err |= EP_ERRBIT_INVALID_ID;
        *s_fatal = (err & EP_ERRBIT_FATAL) != 0;
        if (publish) {
            a.scalars[EP_SCALAR_NUM_EXPANDED] = s_psum[E];
            a.scalars[EP_SCALAR_INVALID_COUNT] = s_total[E];
            a.scalars[EP_SCALAR_NUM_RECV_TOKENS] = s_total[E + 1];
            a.scalars[EP_SCALAR_ERROR_BITS] = static_cast<int32_t>(err);
        }
    }
    __syncthreads();
    if (publish) {
        for (int b = tid; b < E; b += kLayoutThreads) {
            a.counts[b] = s_total[b];
            if (a.cumulative_stats) a.cumulative_stats[b] += s_total[b];
        }
        for (int b = tid; b <= E; b += kLayoutThreads) a.psum[b] = s_psum[b];
    }
}

// Rank-layout rows of a tile's tokens [tok0, tok0 + tokens_per_tile): the
// received ones (flag set in s_tok) numbered from `first` in token order,
// the others -1.
__device__ void number_rank_rows(const LayoutArgs &a, int64_t tok0, int tokens_per_tile,
                                 const uint8_t *s_tok, int64_t first, int64_t *s_wave) {
    const int tid = threadIdx.x;
    const int tper = (tokens_per_tile + kLayoutThreads - 1) / kLayoutThreads;
    const int j0 = tid * tper;
    const int j1 = min(j0 + tper, tokens_per_tile);
    int64_t cnt = 0;
    for (int j = j0; j < j1; ++j) cnt += s_tok[j];
    int64_t unused = 0;
    int64_t row = first + block_exclusive_scan(cnt, s_wave, &unused);
    for (int j = j0; j < j1; ++j) {
        const int64_t t = tok0 + j;
        if (t >= a.num_tokens) break;
        if (s_tok[j]) {
            a.recv_row[t] = static_cast<int32_t>(row);
            a.recv_src[row] = static_cast<int32_t>(t);
            ++row;
        } else {
            a.recv_row[t] = -1;
        }
    }
}

template <typename IdxT>
__global__ __launch_bounds__(kLayoutThreads) void layout_scan_kernel(LayoutArgs a,
                                                                    int tokens_per_tile,
                                                                    int num_tiles) {
    __shared__ int32_t s_hist[kLayoutWaves][kMaxBuckets];
    __shared__ int32_t s_excl[kMaxBuckets];
    __shared__ int32_t s_total[kMaxBuckets];
    __shared__ uint8_t s_tok[kTileSlots];
    __shared__ int64_t s_wave[kLayoutWaves];
    __shared__ int32_t s_tile;
    __shared__ uint32_t s_epoch;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = a.num_experts, NB = E + 2, K = a.num_topk;
    const int B_INVALID = E, B_RECV = E + 1;
    if (tid == 0) {
        s_tile = __hip_atomic_fetch_add(a.ticket, 1, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
        s_epoch = static_cast<uint32_t>(*a.epoch);
    }
    __syncthreads();
    const int tile = s_tile;
    const uint32_t epoch = s_epoch;

    const int64_t num_slots = static_cast<int64_t>(a.num_tokens) * K;
    const int64_t tile_base = static_cast<int64_t>(tile) * tokens_per_tile * K;
    const int64_t tile_end_full = tile_base + static_cast<int64_t>(tokens_per_tile) * K;
    const int64_t tile_end = tile_end_full < num_slots ? tile_end_full : num_slots;
    const int64_t wave_base = tile_base + static_cast<int64_t>(wave) * (kRoundsLarge * 64);

    // 1-2. Rank the tile's slots; in-tile offsets and the tile's counts.
    int bucket[kRoundsLarge];
    int rank[kRoundsLarge];
    int32_t agg[kBucketsPerThread];
    rank_tile<IdxT, kRoundsLarge>(a, tile_base, tile_end, tokens_per_tile, s_hist, s_tok, bucket, rank, agg);

    // 3. Decoupled lookback across tiles.
    uint64_t *my_status = a.tile_status + static_cast<int64_t>(tile) * NB;
#pragma unroll
    for (int q = 0; q < kBucketsPerThread; ++q) {
        const int b = tid + q * kLayoutThreads;
        if (b < NB)
            store_status(&my_status[b],
                         pack_status(epoch, tile == 0 ? kFlagPrefix : kFlagAggregate,
                                     static_cast<uint32_t>(agg[q])));
    }
#pragma unroll
    for (int q = 0; q < kBucketsPerThread; ++q) {
        const int b = tid + q * kLayoutThreads;
        if (b >= NB) continue;
        uint32_t excl = 0;
        if (tile > 0) {
            if (!lookback(a.tile_status, NB, tile, b, epoch, &excl))
                atomicOr(reinterpret_cast<unsigned *>(&a.scalars[EP_SCALAR_ERROR_BITS]),
                         EP_ERRBIT_SCAN_TIMEOUT);
            store_status(&my_status[b],
                         pack_status(epoch, kFlagPrefix, excl + static_cast<uint32_t>(agg[q])));
        }
        s_excl[b] = static_cast<int32_t>(excl);
    }
    __syncthreads();

    // 4. Position of every valid slot inside its expert's run (-1 if empty).
#pragma unroll
    for (int j = 0; j < kRoundsLarge; ++j) {
        const int64_t i = wave_base + j * 64 + lane;
        if (i < tile_end) {
            const int b = bucket[j];
            a.dst[i] = (b >= 0 && b < E) ? s_excl[b] + s_hist[wave][b] + rank[j] : -1;
        }
    }

    // 5. Rank layout: the tile's received tokens get consecutive rows after
    //    the received tokens of earlier tiles (bucket E+1's exclusive count).
    number_rank_rows(a, static_cast<int64_t>(tile) * tokens_per_tile, tokens_per_tile, s_tok,
                     s_excl[B_RECV], s_wave);
    __syncthreads();                                   // s_wave is used again below

    // 6. The last tile owns the totals: counts, aligned scan, scalars.
    if (tile != num_tiles - 1) return;
#pragma unroll
    for (int q = 0; q < kBucketsPerThread; ++q) {
        const int b = tid + q * kLayoutThreads;
        if (b < NB) {
            const int32_t tot = s_excl[b] + agg[q];
            s_total[b] = tot;
            if (b < E) {
                a.counts[b] = tot;
                if (a.cumulative_stats) a.cumulative_stats[b] += tot;
            }
        }
    }
    __syncthreads();
    const int per = (E + kLayoutThreads - 1) / kLayoutThreads;
    const int b0 = tid * per;
    const int b1 = min(b0 + per, E);
    int64_t local = 0;
    for (int b = b0; b < b1; ++b) local += align_up(s_total[b], a.alignment);
    int64_t total = 0;
    int64_t run = block_exclusive_scan(local, s_wave, &total);
    for (int b = b0; b < b1; ++b) {
        a.psum[b] = static_cast<int32_t>(min(run, static_cast<int64_t>(INT32_MAX)));
        run += align_up(s_total[b], a.alignment);
    }
    if (tid == 0) {
        const int32_t expanded = static_cast<int32_t>(min(total, static_cast<int64_t>(INT32_MAX)));
        const int32_t invalid = s_total[B_INVALID];
        a.psum[E] = expanded;
        uint32_t err = static_cast<uint32_t>(a.scalars[EP_SCALAR_ERROR_BITS]) &
                       EP_ERRBIT_SCAN_TIMEOUT;
        if (total > a.capacity) err |= EP_ERRBIT_CAPACITY;
        if (invalid > 0) err |= EP_ERRBIT_INVALID_ID;
        a.scalars[EP_SCALAR_NUM_EXPANDED] = expanded;
        a.scalars[EP_SCALAR_INVALID_COUNT] = invalid;
        a.scalars[EP_SCALAR_NUM_RECV_TOKENS] = s_total[B_RECV];
        a.scalars[EP_SCALAR_ERROR_BITS] = static_cast<int32_t>(err);
    }
}

template <typename IdxT>
__global__ __launch_bounds__(256) void layout_finalize_kernel(LayoutArgs a, int slot_blocks) {
    const int tid = threadIdx.x;
    if (blockIdx.x == 0 && tid == 0) {
        *a.ticket = 0;
        uint32_t next = static_cast<uint32_t>(*a.epoch) + 1u;
        if (next >= (1u << 30)) next = 1u;
        *a.epoch = static_cast<int32_t>(next);
    }
    if (a.scalars[EP_SCALAR_ERROR_BITS] & EP_ERRBIT_FATAL) return;
    const int E = a.num_experts;
    if (static_cast<int>(blockIdx.x) < slot_blocks) {
        const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + tid;
        if (i >= static_cast<int64_t>(a.num_tokens) * a.num_topk) return;
        const IdxT *idx = static_cast<const IdxT *>(a.topk_idx);
        const int64_t e = static_cast<int64_t>(idx[i]);
        const int32_t pos = a.dst[i];
        if (e >= 0 && e < E) {
            const int32_t r = a.psum[e] + pos;
            a.dst[i] = r;
            if (r < a.capacity) a.src_meta[r] = static_cast<int32_t>(i);
        }
        return;
    }
    const int e = static_cast<int>(blockIdx.x) - slot_blocks;
    const int32_t g1 = a.psum[e + 1];
    const int64_t end = g1 < a.capacity ? g1 : a.capacity;
    for (int64_t r = static_cast<int64_t>(a.psum[e]) + a.counts[e] + tid; r < end; r += 256)
        a.src_meta[r] = -1;
}

// ---------------------------------------------------------------- one tile
// A batch that fits in one tile needs no exchange between blocks.  Block 0
// ranks every slot (rank_tile), scans the aligned counts, writes counts,
// psum, the scalars, every slot's row and source metadata and the rank rows.
// The alignment gaps are marked either by block 0's four waves (a one-block
// grid) or by the other blocks, each of which counts the batch's ids again
// (no ranking: at most kTileSlots of them), repeats the scan and marks the
// gaps of every (gridDim.x - 1)-th expert.  One launch; no block waits on
// another; no status words and no epoch.
template <typename IdxT, int R>
__global__ __launch_bounds__(kLayoutThreads) void layout_single_kernel(LayoutArgs a,
                                                                      int tokens_per_tile) {
    __shared__ int32_t s_hist[kLayoutWaves][kMaxBuckets];
    __shared__ int32_t s_total[kMaxBuckets];
    __shared__ int32_t s_psum[kMaxExperts + 1];
    __shared__ uint8_t s_tok[kLayoutThreads * R];
    __shared__ int64_t s_wave[kLayoutWaves];
    __shared__ int32_t s_fatal;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = a.num_experts, NB = E + 2;
    const int64_t num_slots = static_cast<int64_t>(a.num_tokens) * a.num_topk;
    const int64_t wave_base = static_cast<int64_t>(wave) * (R * 64);
    const uint32_t sticky = static_cast<uint32_t>(a.scalars[EP_SCALAR_ERROR_BITS]);
    if (blockIdx.x > 0) {
        const IdxT *idx = static_cast<const IdxT *>(a.topk_idx);
        for (int b = tid; b < NB; b += kLayoutThreads) s_total[b] = 0;
        __syncthreads();
        for (int64_t i = tid; i < num_slots; i += kLayoutThreads) {
            const int64_t e = static_cast<int64_t>(idx[i]);
            if (e >= 0 && e < E) atomicAdd(&s_total[e], 1);
            else if (e != -1) atomicAdd(&s_total[E], 1);
        }
        __syncthreads();
        scan_experts(a, s_total, s_psum, s_wave, &s_fatal, false, sticky);
        if (s_fatal) return;
        for (int e = blockIdx.x - 1; e < E; e += gridDim.x - 1) {
            const int64_t end = s_psum[e + 1] < a.capacity ? s_psum[e + 1] : a.capacity;
            for (int64_t r = static_cast<int64_t>(s_psum[e]) + s_total[e] + tid; r < end;
                 r += kLayoutThreads)
                a.src_meta[r] = -1;
        }
        return;
    }
    int bucket[R];
    int rank[R];
    int32_t agg[kBucketsPerThread];
    rank_tile<IdxT, R>(a, 0, num_slots, tokens_per_tile, s_hist, s_tok, bucket, rank, agg);
#pragma unroll
    for (int q = 0; q < kBucketsPerThread; ++q) {
        const int b = tid + q * kLayoutThreads;
        if (b < NB) s_total[b] = agg[q];
    }
    __syncthreads();
    scan_experts(a, s_total, s_psum, s_wave, &s_fatal, true, sticky);
    const bool fatal = s_fatal != 0;
    if (!fatal) {
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int64_t i = wave_base + j * 64 + lane;
            if (i >= num_slots) continue;
            const int b = bucket[j];
            int32_t r = -1;
            if (b >= 0 && b < E) {
                r = s_psum[b] + s_hist[wave][b] + rank[j];
                a.src_meta[r] = static_cast<int32_t>(i);
            }
            a.dst[i] = r;
        }
    }
    number_rank_rows(a, 0, tokens_per_tile, s_tok, 0, s_wave);
    if (fatal || gridDim.x > 1) return;
    for (int e = wave; e < E; e += kLayoutWaves) {
        const int64_t end = s_psum[e + 1] < a.capacity ? s_psum[e + 1] : a.capacity;
        for (int64_t r = static_cast<int64_t>(s_psum[e]) + s_total[e] + lane; r < end; r += 64)
            a.src_meta[r] = -1;
    }
}

// ---------------------------------------------------------------- count + place
// Batches of at most kCountPlaceMaxTiles tiles.  layout_count: one block per
// tile ranks its slots (rank_tile), publishes the tile's counts as status
// words tagged with this call's epoch, and parks each slot's bucket and
// in-tile position in dst.  layout_place (after the kernel boundary, so every
// count is visible): one block per tile sums the counts of the tiles before it
// and of all tiles, scans the aligned totals into psum (every block the same
// way), writes its slots' final rows and source metadata and its tokens' rank
// rows; place_gap_blocks more blocks (same totals and scan) mark the experts'
// alignment gaps; tile 0 writes counts, psum and the scalars and finally moves
// the epoch on, so no later call can mistake these status words for its own.
// Nothing waits on another block.
#ifndef EP_LAYOUT_COUNT_PLACE_MAX_TILES
#define EP_LAYOUT_COUNT_PLACE_MAX_TILES 400
#endif
constexpr int kCountPlaceMaxTiles = EP_LAYOUT_COUNT_PLACE_MAX_TILES;

__device__ inline uint32_t park(int b, int pos) {
    return static_cast<uint32_t>(b + 1) | (static_cast<uint32_t>(pos) << 11);
}

template <typename IdxT, int R>
__global__ __launch_bounds__(kLayoutThreads) void layout_count_kernel(LayoutArgs a,
                                                                     int tokens_per_tile) {
    __shared__ int32_t s_hist[kLayoutWaves][kMaxBuckets];
    __shared__ uint8_t s_tok[kTileSlots];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = a.num_experts, NB = E + 2, K = a.num_topk;
    const int tile = blockIdx.x;
    const uint32_t epoch = static_cast<uint32_t>(*a.epoch);
    const int64_t num_slots = static_cast<int64_t>(a.num_tokens) * K;
    const int64_t tile_base = static_cast<int64_t>(tile) * tokens_per_tile * K;
    const int64_t tile_end_full = tile_base + static_cast<int64_t>(tokens_per_tile) * K;
    const int64_t tile_end = tile_end_full < num_slots ? tile_end_full : num_slots;
    const int64_t wave_base = tile_base + static_cast<int64_t>(wave) * (R * 64);
    int bucket[R];
    int rank[R];
    int32_t agg[kBucketsPerThread];
    rank_tile<IdxT, R>(a, tile_base, tile_end, tokens_per_tile, s_hist, s_tok, bucket, rank, agg);
    uint64_t *my_status = a.tile_status + static_cast<int64_t>(tile) * NB;
#pragma unroll
    for (int q = 0; q < kBucketsPerThread; ++q) {
        const int b = tid + q * kLayoutThreads;
        if (b < NB)
            store_status(&my_status[b],
                         pack_status(epoch, kFlagAggregate, static_cast<uint32_t>(agg[q])));
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t i = wave_base + j * 64 + lane;
        if (i < tile_end) {
            const int b = bucket[j];
            a.dst[i] = static_cast<int32_t>(b < 0 ? 0u : park(b, s_hist[wave][b] + rank[j]));
        }
    }
}

// Counts of buckets tid + q * kLayoutThreads (q < kBucketsPerThread) over
// every tile: the sum over tiles before `tile` into s_excl[b], over all
// tiles into s_total[b].  The words were written by an earlier kernel, so
// ordinary loads (which may hit in L2) see them; kCountWindow tiles of two
// buckets per round trip, all in flight together.  At 256 experts (258
// buckets: threads 0 and 1 hold two) 32 short tiles take one round trip
// instead of two and 128 long tiles four instead of eight; measured
// cache-cold, interleaved on one box: prefill 4096 x 8 layout 15.2 ->
// 14.3 us, 32768 x 8 25.0 -> 24.0 us.
constexpr int kCountWindow = 32;

__device__ void sum_tile_counts(const uint64_t *status, int NB, int num_tiles, int tile,
                                int32_t *s_excl, int32_t *s_total) {
    const int tid = threadIdx.x;
    for (int q = 0; q < kBucketsPerThread; q += 2) {
        const int b0 = tid + q * kLayoutThreads, b1 = b0 + kLayoutThreads;
        if (b0 >= NB) break;
        const bool two = b1 < NB;
        uint32_t ex0 = 0, tot0 = 0, ex1 = 0, tot1 = 0;
        for (int t0 = 0; t0 < num_tiles; t0 += kCountWindow) {
            uint32_t c0[kCountWindow], c1[kCountWindow];
#pragma unroll
            for (int w = 0; w < kCountWindow; ++w) {
                const uint32_t *row =
                    reinterpret_cast<const uint32_t *>(status + static_cast<int64_t>(t0 + w) * NB);
                c0[w] = t0 + w < num_tiles ? row[2 * b0] : 0u;
                c1[w] = t0 + w < num_tiles && two ? row[2 * b1] : 0u;
            }
#pragma unroll
            for (int w = 0; w < kCountWindow; ++w) {
                if (t0 + w < tile) {
                    ex0 += c0[w];
                    ex1 += c1[w];
                }
                tot0 += c0[w];
                tot1 += c1[w];
            }
        }
        s_excl[b0] = static_cast<int32_t>(ex0);
        s_total[b0] = static_cast<int32_t>(tot0);
        if (two) {
            s_excl[b1] = static_cast<int32_t>(ex1);
            s_total[b1] = static_cast<int32_t>(tot1);
        }
    }
}

template <typename IdxT, int R>
__global__ __launch_bounds__(kLayoutThreads) void layout_place_kernel(LayoutArgs a,
                                                                     int tokens_per_tile,
                                                                     int num_tiles,
                                                                     int gap_blocks) {
    __shared__ int32_t s_excl[kMaxBuckets];
    __shared__ int32_t s_total[kMaxBuckets];
    __shared__ int32_t s_psum[kMaxExperts + 1];
    __shared__ uint8_t s_tok[kTileSlots];
    __shared__ int64_t s_wave[kLayoutWaves];
    __shared__ int32_t s_fatal;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = a.num_experts, NB = E + 2, K = a.num_topk;
    const bool gap_block = static_cast<int>(blockIdx.x) >= num_tiles;
    const int tile = gap_block ? -1 : static_cast<int>(blockIdx.x);
    const int64_t num_slots = static_cast<int64_t>(a.num_tokens) * K;
    const int64_t tile_base = static_cast<int64_t>(gap_block ? 0 : tile) * tokens_per_tile * K;
    const int64_t tile_end_full = tile_base + static_cast<int64_t>(tokens_per_tile) * K;
    const int64_t tile_end = gap_block ? 0 : (tile_end_full < num_slots ? tile_end_full : num_slots);
    const int64_t wave_base = tile_base + static_cast<int64_t>(wave) * (R * 64);
    const uint32_t sticky = static_cast<uint32_t>(a.scalars[EP_SCALAR_ERROR_BITS]);

    // The tile's parked slots (independent of the counts: loads issued first).
    uint32_t parked[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t i = wave_base + j * 64 + lane;
        parked[j] = i < tile_end ? static_cast<uint32_t>(a.dst[i]) : 0u;
    }
    for (int i = tid; i < tokens_per_tile; i += kLayoutThreads) s_tok[i] = 0;

    // 1. Every tile's counts: this tile's exclusive offsets and the totals.
    sum_tile_counts(a.tile_status, NB, num_tiles, tile, s_excl, s_total);
    __syncthreads();

    // 2. Aligned exclusive scan over experts (identical in every block).
    scan_experts(a, s_total, s_psum, s_wave, &s_fatal, tile == 0, sticky);
    const bool fatal = s_fatal != 0;
    // Gap markers: of every gap_blocks-th expert from blockIdx.x - num_tiles
    // in the gap blocks, or, without gap blocks, of every num_tiles-th expert
    // from the tile's own index in the tile blocks (at the end).
    const int gap_first = gap_block ? static_cast<int>(blockIdx.x) - num_tiles : tile;
    const int gap_step = gap_block ? gap_blocks : num_tiles;
    auto mark_gaps = [&]() {
        for (int e = gap_first; e < E; e += gap_step) {
            const int64_t end = s_psum[e + 1] < a.capacity ? s_psum[e + 1] : a.capacity;
            for (int64_t r = static_cast<int64_t>(s_psum[e]) + s_total[e] + tid; r < end;
                 r += kLayoutThreads)
                a.src_meta[r] = -1;
        }
    };
    if (gap_block) {
        if (!fatal) mark_gaps();
        return;
    }

    // 3. Final rows and source metadata; flags of received tokens.
    const uint32_t k_magic = 0xFFFFFFFFu / static_cast<uint32_t>(K) + 1u;
    const uint32_t wave_slot0 = static_cast<uint32_t>(wave_base - tile_base);
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t i = wave_base + j * 64 + lane;
        if (i >= tile_end) continue;
        const int b = static_cast<int>(parked[j] & 0x7FFu) - 1;
        if (b >= 0 && b < E) {
            const uint32_t s = wave_slot0 + j * 64 + lane;
            s_tok[K == 1 ? s : __umulhi(s, k_magic)] = 1;
        }
        if (fatal) continue;
        int32_t r = -1;
        if (b >= 0 && b < E) {
            r = s_psum[b] + s_excl[b] + static_cast<int32_t>(parked[j] >> 11);
            a.src_meta[r] = static_cast<int32_t>(i);
        }
        a.dst[i] = r;
    }
    __syncthreads();

    // 4. Rank layout: the tile's received tokens after those of earlier tiles.
    number_rank_rows(a, static_cast<int64_t>(tile) * tokens_per_tile, tokens_per_tile, s_tok,
                     s_excl[E + 1], s_wave);
    if (gap_blocks == 0 && !fatal) mark_gaps();

    // 5. Tile 0 retires this call's status words.
    if (tile == 0 && tid == 0) {
        *a.ticket = 0;
        uint32_t next = static_cast<uint32_t>(*a.epoch) + 1u;
        if (next >= (1u << 30)) next = 1u;
        *a.epoch = static_cast<int32_t>(next);
    }
}

__global__ void handle_clear_kernel(int32_t *scalars, uint64_t *status, int64_t n) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = gid; i < n; i += stride) status[i] = 0;
    if (gid < EP_NUM_SCALARS) scalars[gid] = (gid == EP_SCALAR_EPOCH) ? 1 : 0;
}

// Header of the static scratch: int32 ticket, int32 epoch (1 after set-up).
__global__ void scratch_clear_kernel(uint64_t *words, int64_t n) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = gid; i < n; i += stride) words[i] = 0;
    if (gid == 0) {
        int32_t *header = reinterpret_cast<int32_t *>(words);
        header[1] = 1;
    }
}

// Scratch of ep_layout_noalloc: the layout scans' ticket, epoch and per-tile
// status words in a file-scope device array, so that call needs no
// workspace region of its own.  Each device holds its own copy (at its own
// address, found once per device with hipGetSymbolAddress); every
// ep_layout_noalloc call on a device shares it, so such calls that overlap
// on one device race.
static __device__ __align__(256) uint64_t scratch[kScratchBytes / 8];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t layout_scratch(hipStream_t stream, uint64_t **status, int32_t **ticket,
                          int32_t **epoch) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        ptr = g_scratch_ptr[dev];
        if (!ptr) {
            // Set-up, once per device with that device current: the array's
            // device address, then one clear (ticket 0, epoch 1, status
            // words 0) ordered before the first layout on this stream.
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!ptr) return hipErrorInvalidSymbol;
            scratch_clear_kernel<<<dim3(256), dim3(256), 0, stream>>>(
                static_cast<uint64_t *>(ptr), kScratchBytes / 8);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
            g_scratch_ptr[dev] = ptr;
        }
    }
    char *base = static_cast<char *>(ptr);
    *ticket = reinterpret_cast<int32_t *>(base);
    *epoch = reinterpret_cast<int32_t *>(base) + 1;
    *status = reinterpret_cast<uint64_t *>(base + kScratchHeaderBytes);
    return hipSuccess;
}

hipError_t launch_handle_clear(int32_t *scalars, uint64_t *tile_status, int64_t status_words,
                               hipStream_t stream) {
    int64_t blocks = (status_words + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 1024) blocks = 1024;
    handle_clear_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(scalars, tile_status,
                                                                           status_words);
    return hipGetLastError();
}

namespace {

// Extra blocks of layout_place that mark the alignment gaps, each taking
// every EP_LAYOUT_PLACE_GAP_BLOCKS-th expert (0: the tile blocks mark them
// after their rank rows).  Every such block reads all tiles' counts again,
// so fewer of them cost less; cache-cold, interleaved on one box, layout at
// prefill 4096 x 8 / 32768 x 8: one block per expert (256) 14.4 / 24.0 us,
// 64 blocks 13.9 / 23.2, 16 blocks 14.5 / 23.2, none 15.0 / 23.5.  (One
// block scan for both the expert totals and the rank rows instead of two:
// 14.0 / 23.5 us, not kept.)
#ifndef EP_LAYOUT_PLACE_GAP_BLOCKS
#define EP_LAYOUT_PLACE_GAP_BLOCKS 64
#endif
int place_gap_blocks(const LayoutArgs &a) {
    const int g = EP_LAYOUT_PLACE_GAP_BLOCKS;
    if (g < 0 || g > a.num_experts) return a.num_experts;
    return g;
}

template <typename IdxT, int R>
hipError_t launch_count_place(const LayoutArgs &a, hipStream_t stream, CallEvents ev) {
    const int tpt = layout_tokens_per_tile(a.num_topk, R);
    const int tiles = static_cast<int>(layout_tiles(a.num_tokens, a.num_topk, R));
    hipError_t e = launch_kernel(layout_count_kernel<IdxT, R>, dim3(tiles), dim3(kLayoutThreads),
                                 stream, ev.start, nullptr, a, tpt);
    if (e == hipSuccess)
        e = launch_kernel(layout_place_kernel<IdxT, R>, dim3(tiles + place_gap_blocks(a)),
                          dim3(kLayoutThreads), stream, nullptr, ev.stop, a, tpt, tiles,
                          place_gap_blocks(a));
    return e;
}

template <typename IdxT>
hipError_t launch_scan_finalize(const LayoutArgs &a, hipStream_t stream, CallEvents ev) {
    const int tpt = layout_tokens_per_tile(a.num_topk, kRoundsLarge);
    const int tiles = static_cast<int>(layout_tiles(a.num_tokens, a.num_topk, kRoundsLarge));
    const int64_t slots = static_cast<int64_t>(a.num_tokens) * a.num_topk;
    const int slot_blocks = static_cast<int>((slots + 255) / 256);
    const dim3 fin_blocks(static_cast<unsigned>(slot_blocks + a.num_experts));
    hipError_t e = launch_kernel(layout_scan_kernel<IdxT>, dim3(tiles), dim3(kLayoutThreads),
                                 stream, ev.start, nullptr, a, tpt, tiles);
    if (e == hipSuccess)
        e = launch_kernel(layout_finalize_kernel<IdxT>, fin_blocks, dim3(256), stream, nullptr,
                          ev.stop, a, slot_blocks);
    return e;
}

// Gap-marking blocks of the one-tile layout when there are alignment gaps.
#ifndef EP_LAYOUT_SINGLE_GAP_BLOCKS
#define EP_LAYOUT_SINGLE_GAP_BLOCKS 16
#endif

template <typename IdxT, int R>
hipError_t launch_single(const LayoutArgs &a, hipStream_t stream, CallEvents ev) {
    int gap_blocks = 0;
    if (a.alignment > 1)
        gap_blocks = a.num_experts < EP_LAYOUT_SINGLE_GAP_BLOCKS ? a.num_experts
                                                                 : EP_LAYOUT_SINGLE_GAP_BLOCKS;
    return launch_kernel(layout_single_kernel<IdxT, R>, dim3(1 + gap_blocks),
                         dim3(kLayoutThreads), stream, ev.start, ev.stop, a,
                         layout_tokens_per_tile(a.num_topk, R));
}

template <typename IdxT>
hipError_t launch_layout_idx(const LayoutArgs &a, hipStream_t stream, CallEvents ev) {
    if (layout_tiles(a.num_tokens, a.num_topk, kRoundsSmall) == 1)
        return launch_single<IdxT, kRoundsSmall>(a, stream, ev);
    if (layout_tiles(a.num_tokens, a.num_topk, kRoundsLarge) == 1)
        return launch_single<IdxT, kRoundsLarge>(a, stream, ev);
    if (layout_rounds(a.num_tokens, a.num_topk) == kRoundsSmall)
        return launch_count_place<IdxT, kRoundsSmall>(a, stream, ev);
    if (layout_tiles(a.num_tokens, a.num_topk, kRoundsLarge) <= kCountPlaceMaxTiles)
        return launch_count_place<IdxT, kRoundsLarge>(a, stream, ev);
    return launch_scan_finalize<IdxT>(a, stream, ev);
}

}  // namespace

hipError_t launch_layout(const LayoutArgs &a, hipStream_t stream, CallEvents ev) {
    return a.idx_is_i64 ? launch_layout_idx<int64_t>(a, stream, ev)
                        : launch_layout_idx<int32_t>(a, stream, ev);
}

}  // namespace ep
