/*
 * ep_ceilings.h - bandwidth ceilings for the benchmark (libep_ceilings.so).
 *
 * Plain gfx950 kernels that move the bytes of an access pattern and nothing
 * else, so that each layout / dispatch / combine call can be compared with
 * what the memory system gives for the same pattern.  The pattern that
 * matters is the one the pages name for the communication stage: one
 * copy / permute so that grouped GEMMs read contiguous expert ranges (DeepEP
 * notes ch.7 "V2: how dispatch builds expert inputs", s7.4); on one GPU it
 * is HBM traffic.  Not part of the layout / dispatch / combine interface
 * (include/ep.h); nothing in libep.so calls it.
 *
 * Conventions: pointers are device memory owned by the caller; sizes are in
 * bytes and must be multiples of 16 (16-byte vectors), pointers 16-byte
 * aligned.  Every call enqueues one kernel on `stream` and returns at once:
 * 0 on success, -1 for invalid arguments (nothing launched), else the
 * hipError_t of the launch.  `start` / `stop` may be NULL; when given, they
 * are attached to the kernel dispatch itself (recorded when it starts and
 * when it ends), so their interval is the kernel's execution only.
 */
#ifndef EP_CEILINGS_H
#define EP_CEILINGS_H

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * The sequential kernels take three tunables, so the benchmark can keep the
 * fastest setting as the ceiling: vec_per_thread (1, 2, 4, 8 or 16) 16-byte
 * vectors per thread per round, all requested before any is used (a block
 * of 256 threads covers 4096 * vec_per_thread bytes per round); blocks, the
 * grid (0 = one round per block, else at most that many blocks whose rounds
 * stride over the buffer); nontemporal (nonzero: streaming loads / stores).
 */

/* Words of `sink` that epc_read writes (-1 for invalid tunables). */
int64_t epc_read_sink_words(size_t bytes, int32_t vec_per_thread, int32_t blocks);

/* Load-only: read `bytes` of `src` once, in address order; one XOR-folded
 * word per wave goes to sink [epc_read_sink_words(...)].  Also used as the
 * cache flush. */
int epc_read(const void *src, size_t bytes, uint32_t *sink, int32_t vec_per_thread,
             int32_t blocks, int32_t nontemporal, hipStream_t stream,
             hipEvent_t start, hipEvent_t stop);

/* Store-only: write `bytes` of `dst` in address order with the 32-bit
 * `value` repeated. */
int epc_write(void *dst, size_t bytes, uint32_t value, int32_t vec_per_thread,
              int32_t blocks, int32_t nontemporal, hipStream_t stream,
              hipEvent_t start, hipEvent_t stop);

/* Device copy of `bytes`, loads and stores in address order (1:1). */
int epc_copy(void *dst, const void *src, size_t bytes, int32_t vec_per_thread,
             int32_t blocks, int32_t nontemporal, hipStream_t stream,
             hipEvent_t start, hipEvent_t stop);

/* The dispatch's store pattern alone: for each token t < tokens and each
 * 1 KB pass of a row (one wave), a constant is stored to that pass of row
 * slot_row[t*K + k] of dst [rows, row_bytes] for every k with
 * 0 <= slot_row[t*K + k] < rows (others skipped).  1 <= K <= 64.
 * nontemporal: nonzero for streaming stores (the dispatch's
 * EP_DISPATCH_STREAMING). */
int epc_row_store(void *dst, int64_t rows, int64_t row_bytes,
                  const int32_t *slot_row, int64_t tokens, int32_t K, int32_t nontemporal,
                  hipStream_t stream, hipEvent_t start, hipEvent_t stop);

/* The combine's traffic alone: out[t] (row_bytes, out holds tokens rows) =
 * XOR over k of in[slot_row[t*K + k]] (in holds `rows` rows; indices outside
 * [0, rows) read nothing), one thread per 16-byte column, non-temporal
 * loads and stores.  1 <= K <= 64. */
int epc_gather(void *out, const void *in, int64_t rows, int64_t row_bytes,
               const int32_t *slot_row, int64_t tokens, int32_t K,
               hipStream_t stream, hipEvent_t start, hipEvent_t stop);

/* A grid of `blocks` x `threads` that does nothing: the floor of a launch
 * timed by events on its dispatch (small calls are bound by it). */
int epc_empty(int32_t blocks, int32_t threads, hipStream_t stream, hipEvent_t start,
              hipEvent_t stop);

#ifdef __cplusplus
}
#endif

#endif /* EP_CEILINGS_H */
