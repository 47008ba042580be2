/*
 * ep.h - C ABI of the one-GPU MoE routing layout, dispatch and combine
 * library for AMD Instinct MI355X (gfx950).
 *
 * Sources: the DeepEP notes, chapter 7 "V2: how dispatch builds expert
 * inputs" [Ch7] and chapter 8 "V2: combine, handle and async overlap" [Ch8]
 * (bowenzhou.top/repos/deepep), the digest of vLLM pull request 52781
 * "DeepEP v2 combine made asynchronous" [vLLM], and the DeepEP README [README].
 *
 * What is computed, for one GPU's share of an expert-parallel MoE layer:
 *   layout   - from topk_idx [T, K] (-1 = empty slot), per-expert counts,
 *              the exclusive prefix sums of the counts aligned up to
 *              expert_alignment, the expanded row of every slot and the
 *              source slot of every expanded row.
 *   dispatch - copy every token row (bf16, or FP8 bytes plus 4-byte scale
 *              packs) into the expanded row of each of its slots; each
 *              expert owns one contiguous range whose start is a multiple
 *              of expert_alignment; alignment gaps can be zero-filled.
 *   combine  - for every token, sum its expert rows in slot order k = 0..K-1
 *              in fp32 as w[t,k] * (y[row] + bias[e]), add the per-token
 *              biases, and round to bf16.
 * and around them: the non-expanded ("rank") layout (each received token
 * once) with its dispatch and combine, the backward of combine and of
 * dispatch, and an FP8 quantiser (alone, or fused into the expanded or the
 * rank dispatch) with fp32 or packed UE8M0 scales.
 *
 * Memory ownership: the library never allocates, frees or keeps memory.  All
 * device buffers (workspace, inputs, outputs) belong to the caller and must
 * outlive the stream work that uses them.  The handle is a plain struct owned
 * by the caller; its device arrays point into the caller's workspace.
 *
 * Streams: every call except ep_handle_read_counts and ep_handle_import
 * only enqueues work on the given stream (0 = the null stream) and returns.
 * Ordering against other streams is the caller's job (events), which covers
 * the previous-event / compute-stream controls of [Ch8 §8.2].  Because only
 * those two calls synchronise, every other call can be captured in a HIP
 * graph (none records a memset; device state such as the layout's call tag
 * lives in the handle's workspace).
 *
 * Errors: a call returns a status.  Problems visible on the host (null
 * pointers, sizes, dtypes, alignment, workspace size) are reported before
 * anything is launched.  Problems only the device can see (capacity exceeded,
 * expert ids outside [-1, E)) set bits in the handle's device error word,
 * which ep_handle_read_counts turns into EP_ERR_CAPACITY / EP_ERR_INVALID_ID
 * (or EP_ERR_TIMEOUT if the layout scan's bounded wait ever gave up; that
 * bit is sticky: every later layout on the handle keeps it until
 * ep_handle_init sets the handle up again).  After a capacity or timeout
 * error, dispatch and combine on that handle write nothing.  Calls on one
 * handle must be ordered on one stream; overlapping calls on the same
 * handle race.
 */
#ifndef EP_H
#define EP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ep_status {
    EP_OK = 0,
    EP_ERR_NULL = 1,          /* a required pointer is NULL                    */
    EP_ERR_SHAPE = 2,         /* a size is out of range or inconsistent        */
    EP_ERR_DTYPE = 3,         /* element type not accepted by this call        */
    EP_ERR_UNSUPPORTED = 4,   /* valid for the method, beyond this library's   */
                              /* limits (K > 64, E > 1024, capacity >= 2^31, */
                              /* more than 256 scale packs per token), or a   */
                              /* dispatch flag bit this library does not know */
    EP_ERR_MISALIGNED = 5,    /* pointer or row size not 16-byte aligned       */
    EP_ERR_WORKSPACE = 6,     /* workspace NULL or smaller than required       */
    EP_ERR_NOT_LAID_OUT = 7,  /* dispatch / combine before a layout            */
    EP_ERR_CAPACITY = 8,      /* device: psum[E] > capacity                    */
    EP_ERR_INVALID_ID = 9,    /* device: an id outside [-1, E) was seen        */
    EP_ERR_HIP = 10,          /* a HIP runtime call or launch failed           */
    EP_ERR_TIMEOUT = 11       /* device: the layout scan's bounded wait ended  */
                              /* without its predecessor's count (layout void) */
} ep_status;

typedef enum ep_dtype {
    EP_BF16 = 0,
    EP_FP8_E4M3 = 1,          /* OCP E4M3FN bytes; copied, never interpreted   */
    EP_F32 = 2,
    EP_I32 = 3,
    EP_I64 = 4
} ep_dtype;

/* Scale-factor formats written by the FP8 quantiser. */
typedef enum ep_sf_format {
    EP_SF_F32 = 0,            /* one binary32 scale per 128-channel block       */
    EP_SF_UE8M0 = 1           /* one exponent byte per block, four per 4-byte   */
                              /* pack, lowest block in the low byte            */
} ep_sf_format;

/* Device error word bits (scalars[EP_SCALAR_ERROR_BITS]). */
#define EP_ERRBIT_CAPACITY 1u
#define EP_ERRBIT_INVALID_ID 2u
#define EP_ERRBIT_SCAN_TIMEOUT 4u
/* Bits after which dispatch and combine on the handle write nothing. */
#define EP_ERRBIT_FATAL (EP_ERRBIT_CAPACITY | EP_ERRBIT_SCAN_TIMEOUT)

/* Indices into the handle's device scalars array. */
#define EP_SCALAR_NUM_RECV_TOKENS 0   /* tokens with >= 1 valid slot          */
#define EP_SCALAR_ERROR_BITS 1
#define EP_SCALAR_INVALID_COUNT 2     /* slots with an id outside [-1, E)     */
#define EP_SCALAR_EPOCH 3             /* internal: layout call tag            */
#define EP_SCALAR_TICKET 4            /* internal: tile ticket counter        */
#define EP_SCALAR_NUM_EXPANDED 5      /* psum[E]                              */
#define EP_NUM_SCALARS 8

/*
 * Routing state that combine and cached re-dispatch reuse [Ch7 §7.5: the
 * handle keeps counts, prefix sums, alignment, destination slots and source
 * metadata; a re-dispatch with an old handle takes no topk_idx and must keep
 * expert count, alignment and capacity].  Plain data: the caller may copy
 * it; every copy refers to the same workspace.  Fields are set by
 * ep_handle_init / ep_layout and must not be edited by the caller.
 */
typedef struct ep_handle {
    int32_t max_tokens;         /* T bound fixed at init                        */
    int32_t num_tokens;         /* T of the last layout                         */
    int32_t num_topk;           /* K                                            */
    int32_t num_experts;        /* E                                            */
    int32_t expert_alignment;   /* A                                            */
    int32_t laid_out;           /* 1 after ep_layout / ep_handle_import         */
    int64_t capacity;           /* rows of every expanded buffer                */
    int32_t *counts;            /* device [E] unaligned per-expert counts       */
    int32_t *psum;              /* device [E+1] exclusive scan of aligned counts*/
    int32_t *dst_slot;          /* device [max_tokens*K] row of slot t*K+k, -1  */
    int32_t *src_meta;          /* device [capacity] slot t*K+k of a row, -1 on */
                                /* gap rows, unspecified at or past psum[E]     */
    int32_t *scalars;           /* device [EP_NUM_SCALARS]                      */
    uint64_t *tile_status;      /* device scratch: per-tile counts of a layout  */
    const void *topk_idx;       /* BORROWED device [T, K] ids of the last layout*/
    int32_t topk_idx_dtype;     /* EP_I32 or EP_I64                             */
    int32_t status_tiles;       /* tiles the scratch is sized for               */
    int32_t *recv_row;          /* device [max_tokens] rank-layout row of token */
                                /* t (tokens with a valid slot, in token order),*/
                                /* -1 if the token has no valid slot            */
    int32_t *recv_src;          /* device [max_tokens] token of each rank row;  */
                                /* entries past num_recv_tokens unspecified     */
} ep_handle;

/* Size of ep_handle in bytes, so bindings can check their struct layout. */
size_t ep_handle_sizeof(void);

/*
 * Worst-case expanded rows at one rank when counts are not read back
 * [Ch7 §7.2, allocation without CPU sync]: T*min(K,E) + (A-1)*E rounded up
 * to a multiple of A.  Returns -1 if an argument is <= 0 (T may be 0).
 * With duplicate experts inside a token and K > E, size by T*K + (A-1)*E.
 */
int64_t ep_capacity_bound(int32_t num_tokens, int32_t num_topk,
                          int32_t num_experts, int32_t expert_alignment);

/* Bytes of device workspace a handle with these sizes needs (0 if invalid). */
size_t ep_workspace_bytes(int32_t max_tokens, int32_t num_topk,
                          int32_t num_experts, int32_t expert_alignment,
                          int64_t capacity);

/*
 * Set up a handle in a caller-owned device workspace of ws_bytes bytes
 * (256-byte aligned, at least ep_workspace_bytes).  Clears the layout scan's
 * scratch with one small kernel on `stream`.  1 <= K <= 64,
 * 1 <= E <= 1024, A >= 1, 0 <= max_tokens, max_tokens*K < 2^31,
 * 0 <= capacity < 2^31.
 */
ep_status ep_handle_init(ep_handle *h, int32_t max_tokens, int32_t num_topk,
                         int32_t num_experts, int32_t expert_alignment,
                         int64_t capacity, void *workspace, size_t ws_bytes,
                         hipStream_t stream);

/*
 * Routing layout [Ch7 §7.1 input contract; §7.2 counts, source metadata and
 * slot index come out of dispatch; §7.3 expanded layout aligned per expert].
 *   topk_idx  device [num_tokens, K], EP_I64 or EP_I32, -1 = empty slot.
 *             Borrowed by the handle: it must stay alive and unmodified
 *             while the handle is used with a bias (combine reads expert ids).
 *   num_tokens  <= max_tokens.
 *   cumulative_stats  NULL or device int32 [E]; counts are added to it
 *             (the per-expert receive statistics of [Ch7 §7.2]).
 * Order inside an expert segment: ascending slot index t*K+k.  Ids outside
 * [-1, E) are treated as empty and flagged.  Writes counts, psum, dst_slot,
 * src_meta (gap rows -1), the rank layout (recv_row, recv_src: tokens with a
 * valid slot in token order [Ch7 §7.4]) and the scalars; all on `stream`.
 */
ep_status ep_layout(ep_handle *h, const void *topk_idx, ep_dtype idx_dtype,
                    int32_t num_tokens, int32_t *cumulative_stats,
                    hipStream_t stream);

/*
 * ep_layout for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, checks, kernels and outputs as ep_layout; the layout
 * scans' scratch (tile ticket, call epoch, per-tile status words) lives in
 * a static device array of the library, EP_LAYOUT_SCRATCH_BYTES (1 MiB) per
 * device, held until the process ends, instead of in the handle's
 * workspace.  The first call on a device finds that array's address and
 * enqueues one clear kernel on `stream`; no call allocates or frees.
 * Returns EP_ERR_WORKSPACE, with nothing launched, when the batch needs
 * more status words than the array holds: (number of tiles) * (E + 2) >
 * (1 MiB - 256) / 8, with 128 tokens per tile at K = 8 up to 64 tiles
 * (65536 slots) and 256 tokens per tile beyond (e.g. E = 256: up to
 * 507 tiles, 129792 tokens at K = 8).  Every ep_layout_noalloc call on a
 * device shares the array: calls that overlap on one device (other streams,
 * other threads) race and may produce wrong layouts; calls ordered on one
 * stream are safe, and the array keeps the last call's status words.
 */
#define EP_LAYOUT_SCRATCH_BYTES (1 << 20)
ep_status ep_layout_noalloc(ep_handle *h, const void *topk_idx, ep_dtype idx_dtype,
                            int32_t num_tokens, int32_t *cumulative_stats,
                            hipStream_t stream);

/*
 * The only blocking call besides import [Ch7 §7.2: with CPU sync the host
 * waits for the receive counts and then sizes outputs exactly].  Waits for
 * `stream`, then copies to any non-NULL host pointer: counts [E], psum [E+1],
 * num_expanded (= psum[E]), num_recv_tokens, error_bits, invalid_count.
 * Returns EP_ERR_TIMEOUT, EP_ERR_CAPACITY or EP_ERR_INVALID_ID (in that order
 * of precedence) when the device set the bit (outputs are still filled),
 * else EP_OK.
 */
ep_status ep_handle_read_counts(const ep_handle *h, int32_t *counts,
                                int32_t *psum, int64_t *num_expanded,
                                int32_t *num_recv_tokens, uint32_t *error_bits,
                                int32_t *invalid_count, hipStream_t stream);

/*
 * Install a layout computed elsewhere (host arrays: counts [E], psum [E+1],
 * dst_slot [num_tokens*K], src_meta [psum[E]]) and the device topk_idx it
 * belongs to.  Synchronous (host buffers may be reused on return).  Meant
 * for interop and for checking dispatch/combine against a reference layout.
 * Validated on the host before anything is copied: psum[0] = 0, each
 * expert's run fits its segment, every dst_slot lies in [-1, psum[E]), and
 * src_meta is the inverse of dst_slot (every run row names a slot that
 * points back at it, every gap row is -1) - else EP_ERR_SHAPE; psum[E] >
 * capacity gives EP_ERR_CAPACITY.  After the copy, one kernel on `stream`
 * numbers the rank rows from dst_slot (tokens with a slot row >= 0, in token
 * order [Ch7 §7.4]) and counts them; if that count differs from
 * num_recv_tokens the call returns EP_ERR_SHAPE and leaves the handle not
 * laid out.
 */
ep_status ep_handle_import(ep_handle *h, const void *topk_idx, ep_dtype idx_dtype,
                           int32_t num_tokens, const int32_t *counts,
                           const int32_t *psum, const int32_t *dst_slot,
                           const int32_t *src_meta, int32_t num_recv_tokens,
                           hipStream_t stream);

/*
 * Dispatch copy epilogue into the expert-expanded layout [Ch7 §7.1 (bf16 x,
 * or FP8 data plus scale factors; top-k weights optional), §7.3 (copy
 * epilogue with per-expert alignment, optional zero padding of the gaps,
 * scale factors with their own token and hidden strides, received weights),
 * §7.4 (contiguous aligned expert ranges for a grouped GEMM)].
 *   x        device [num_tokens, hidden]: bf16 (hidden % 8 == 0) or FP8
 *            bytes (hidden % 128 == 0); 16-byte aligned.
 *   sf       FP8 only (NULL for bf16): the token's scale factors as 4-byte
 *            packs [Ch7 §7.3 names the pack count and both strides]; pack
 *            (t, j), j < num_sf_packs, at sf[t*sf_token_stride +
 *            j*sf_hidden_stride] (strides in packs).  Packs are copied as
 *            bits: one fp32 per 128 channels, or four UE8M0 exponent bytes.
 *   num_sf_packs  FP8 only: packs per token, 1..256; 0 means hidden/128
 *            (one fp32 per 128-channel block).  Must be 0 for bf16.
 *   topk_weights  NULL or device fp32 [num_tokens, K].
 *   out_x    device [capacity, hidden] of x's type, 16-byte aligned.
 *   out_sf   FP8 only: pack (r, j) at out_sf[r*out_sf_token_stride +
 *            j*out_sf_hidden_stride]; a column-major buffer whose token
 *            stride is 1 and whose pack stride is ep_tma_aligned_rows(rows)
 *            is the grouped-GEMM scale layout.
 *   out_w    NULL or device fp32 [capacity]: weight of the row's slot
 *            (1.0 when topk_weights is NULL).
 *   flags    0, or EP_DISPATCH_ZERO_PADDING and/or EP_DISPATCH_STREAMING
 *            (other bits: EP_ERR_UNSUPPORTED).  EP_DISPATCH_ZERO_PADDING
 *            [Ch7 §7.3, do_zero_padding]: gap rows get zero bytes, zero
 *            scales, weight 0.  EP_DISPATCH_STREAMING: the rows of out_x
 *            are written with non-temporal stores, which go on to HBM
 *            during the call; without it they are written through the
 *            caches and may stay dirty in the last-level cache (MALL) for
 *            a consumer that reads them next, and reach HBM later.  The
 *            bytes written are the same either way.
 * With no tokens in the layout, x and sf may be NULL, and so may out_x and
 * out_sf unless zero padding is asked for and capacity > 0 (an imported
 * layout can have gap rows and no tokens).
 * Rows at or past psum[E], and gap rows without zero padding, are not
 * written.  Reuses the handle, so a cached re-dispatch is just another call.
 */
#define EP_DISPATCH_ZERO_PADDING 1
#define EP_DISPATCH_STREAMING 2
ep_status ep_dispatch(const ep_handle *h, const void *x, ep_dtype x_dtype,
                      int32_t hidden, const void *sf, int64_t sf_token_stride,
                      int64_t sf_hidden_stride, int32_t num_sf_packs,
                      const float *topk_weights, void *out_x, void *out_sf,
                      int64_t out_sf_token_stride, int64_t out_sf_hidden_stride,
                      float *out_w, int32_t flags, hipStream_t stream);

/*
 * Uncached dispatch: ep_layout on topk_idx, then ep_dispatch of x, in one
 * call with the same arguments and the same outputs as those two calls [Ch7
 * §7.2: the dispatch kernel also produces the counts, the source metadata
 * and the slot index].  The layout's kernels and the copy are enqueued
 * back to back on `stream` after one host-side check of both argument sets:
 * errors are those of the two calls, and nothing is launched unless both
 * argument sets are valid.
 */
ep_status ep_layout_dispatch(ep_handle *h, const void *topk_idx, ep_dtype idx_dtype,
                             int32_t num_tokens, int32_t *cumulative_stats,
                             const void *x, ep_dtype x_dtype, int32_t hidden,
                             const void *sf, int64_t sf_token_stride,
                             int64_t sf_hidden_stride, int32_t num_sf_packs,
                             const float *topk_weights, void *out_x, void *out_sf,
                             int64_t out_sf_token_stride, int64_t out_sf_hidden_stride,
                             float *out_w, int32_t flags, hipStream_t stream);

/*
 * Rows of a column-major scale buffer aligned for the tensor-memory loads of
 * a grouped GEMM [Ch7 §7.3: the FP8 scales may use a column-major stride
 * aligned for TMA]: `rows` rounded up to a whole 16 bytes of 4-byte packs,
 * i.e. to a multiple of 4.  Returns -1 for rows < 0.
 */
int64_t ep_tma_aligned_rows(int64_t rows);

/*
 * FP8 quantiser: the producer of dispatch's FP8 input [Ch7 §7.1: FP8 data
 * travels with per-block scale factors; §7.3: the scale factors are 4-byte
 * packs with their own strides].  The pages give no recipe; this one is the
 * per-128-channel recipe of the benchmark inputs:
 *   amax = largest |x| of the block (NaN skipped); s = max(amax, 1e-12)/448
 *   (binary32); EP_SF_F32 stores s, EP_SF_UE8M0 stores the exponent byte of
 *   s rounded up to a power of two; the divisor is the stored scale's value;
 *   code = E4M3FN nearest to clamp(x / divisor, -448, 448) (binary32
 *   division), ties to even; a NaN quotient gives 0x7F.
 *   x        device bf16 [num_tokens, hidden], hidden % 128 == 0, 16-byte
 *            aligned.
 *   out_q    device [num_tokens, hidden] E4M3FN codes, 16-byte aligned.
 *   out_sf   device 4-byte packs, pack (t, j) at out_sf[t*token_stride +
 *            j*hidden_stride], j < ep_sf_packs(hidden, fmt).
 */
int32_t ep_sf_packs(int32_t hidden, ep_sf_format fmt);   /* -1 if invalid */
ep_status ep_quantize_fp8(const void *x, int32_t num_tokens, int32_t hidden,
                          ep_sf_format fmt, void *out_q, void *out_sf,
                          int64_t out_sf_token_stride, int64_t out_sf_hidden_stride,
                          hipStream_t stream);

/*
 * Quantising dispatch: ep_quantize_fp8 of bf16 x fused with ep_dispatch of
 * the codes and packs (same layout, weights, zero-padding and NULL rules), so x is
 * read once in bf16 and every routed row is written once in FP8 [Ch7 §7.3,
 * §7.4].  out_x is [capacity, hidden] codes; out_sf is [capacity,
 * ep_sf_packs(hidden, fmt)] packs with the given strides.
 */
ep_status ep_dispatch_quant(const ep_handle *h, const void *x, int32_t hidden,
                            ep_sf_format fmt, const float *topk_weights, void *out_x,
                            void *out_sf, int64_t out_sf_token_stride,
                            int64_t out_sf_hidden_stride, float *out_w,
                            int32_t zero_padding, hipStream_t stream);

/*
 * Combine [Ch8 §8.1: reduce along the handle back to the source, with
 * optional fused bias and gate-weight reduction; bf16 x and fp32 weights],
 * [vLLM implementation breakdown: the combine input must be bf16 and the
 * weights may be None].
 *   y        device bf16 [capacity, hidden], hidden % 8 == 0, 16-byte
 *            aligned; only rows that hold a slot are read.
 *   topk_weights  NULL (weight 1) or device fp32 [num_tokens, K].
 *   bias     NULL or device bf16 [E, hidden]: expert e's output bias, added
 *            to the expert row before weighting.
 *   bias_0, bias_1  NULL or device bf16 [num_tokens, hidden]: per-token
 *            biases added after the reduction, bias_0 first [Ch8 §8.1].
 *   out      device bf16 [num_tokens, hidden].
 * out[t][h] = bf16_rne(((sum over valid k in order of w[t,k]*(y[r][h]+b[e][h]))
 *                       + b0[t][h]) + b1[t][h])
 * in fp32 from +0.0 with separately rounded multiply and add; a token with
 * no valid slot gets +0.0 (plus its per-token biases).
 */
ep_status ep_combine(const ep_handle *h, const void *y, ep_dtype y_dtype,
                     int32_t hidden, const float *topk_weights,
                     const void *bias, const void *bias_0, const void *bias_1,
                     void *out, hipStream_t stream);

/*
 * Dispatch into the non-expanded ("rank") layout [Ch7 §7.4: each received
 * token once, [received_tokens, hidden] plus top-k metadata; §7.3: the
 * epilogue also writes the received top-k ids and weights].  Row
 * recv_row[t] of out_x (bf16 or FP8 bytes, [max_tokens, hidden]) gets x[t];
 * FP8 scale packs as in ep_dispatch; out_topk_idx (NULL or [max_tokens, K], the
 * dtype of the layout's topk_idx) gets the token's ids with -1 for empty or
 * invalid slots; out_topk_weights (NULL or fp32 [max_tokens, K]) its weights
 * with 0 for those slots (1 for valid slots when topk_weights is NULL).
 * Rows at or past num_recv_tokens are not written; with no tokens in the
 * layout every buffer may be NULL.
 */
ep_status ep_dispatch_rank(const ep_handle *h, const void *x, ep_dtype x_dtype,
                           int32_t hidden, const void *sf, int64_t sf_token_stride,
                           int64_t sf_hidden_stride, int32_t num_sf_packs,
                           const float *topk_weights, void *out_x, void *out_sf,
                           int64_t out_sf_token_stride, int64_t out_sf_hidden_stride,
                           void *out_topk_idx, float *out_topk_weights,
                           hipStream_t stream);

/*
 * Quantising rank dispatch: ep_quantize_fp8 of bf16 x fused with
 * ep_dispatch_rank of the codes and packs [Ch7 §7.4 rank layout, §7.3 FP8
 * data with scale packs and the received top-k metadata].  Row recv_row[t]
 * of out_x ([max_tokens, hidden] E4M3FN codes, 16-byte aligned) gets token
 * t's codes and row recv_row[t] of out_sf ([max_tokens,
 * ep_sf_packs(hidden, fmt)] packs, any strides) its packs; out_topk_idx and
 * out_topk_weights (NULL or as in ep_dispatch_rank) get the received top-k
 * metadata.  hidden % 128 == 0.  Rows at or past num_recv_tokens are not
 * written; with no tokens in the layout every buffer may be NULL.
 */
ep_status ep_dispatch_rank_quant(const ep_handle *h, const void *x, int32_t hidden,
                                 ep_sf_format fmt, const float *topk_weights, void *out_x,
                                 void *out_sf, int64_t out_sf_token_stride,
                                 int64_t out_sf_hidden_stride, void *out_topk_idx,
                                 float *out_topk_weights, hipStream_t stream);

/*
 * Combine from the rank layout [Ch8 §8.1: reduce back to the source token,
 * optionally adding bias_0 and bias_1].  At one rank every received token has
 * one row of x (bf16 [max_tokens, hidden], already reduced over its experts):
 * out[t][h] = bf16_rne(fl32(fl32(v + b0[t][h]) + b1[t][h])), v = the row's
 * value or +0.0 for a token with no valid slot; NULL biases are skipped.
 */
ep_status ep_combine_rank(const ep_handle *h, const void *x, int32_t hidden,
                          const void *bias_0, const void *bias_1, void *out,
                          hipStream_t stream);

/*
 * Backward of combine [README, training example: the backward of combine is
 * a dispatch of the output gradient, and the combined top-k weights carry the
 * weights' gradient; forward as in ep_combine].  With
 * out[t] = sum_k w[t,k] * (y[r] + b[e]) and g = d loss / d out:
 *   grad_y            NULL or bf16 [capacity, hidden]: routed row r = dst[t,k]
 *                     gets bf16_rne(fl32(w[t,k] * g[t])) (g[t] without
 *                     weights); other rows are not written.
 *   grad_topk_weights NULL or fp32 [T, K]: sum_h g[t][h] * (y[r][h] + b[e][h]),
 *                     0 for an empty slot (needs y; bias may be NULL).
 *   grad_bias         NULL or fp32 [E, hidden]: sum over expert e's rows of
 *                     w * g[t] (every expert written, 0 if it has no row).
 * Both sums are accumulated in binary64 from exact terms and rounded once to
 * binary32.  grad_out is bf16 [T, hidden]; topk_weights / bias as given to
 * ep_combine.  One row pass plus one bias pass (when grad_bias) on `stream`.
 */
ep_status ep_combine_backward(const ep_handle *h, const void *grad_out, int32_t hidden,
                              const float *topk_weights, const void *y, const void *bias,
                              void *grad_y, float *grad_topk_weights, float *grad_bias,
                              hipStream_t stream);

/*
 * Backward of dispatch [README, training example: the backward of dispatch
 * is a combine of the gradient rows, returning the gradient of the received
 * top-k weights as well].
 *   grad_out_x        bf16 [capacity, hidden]: gradient of out_x (for an FP8
 *                     dispatch the gradient is bf16).
 *   grad_out_w        NULL or fp32 [capacity]: gradient of out_w.
 *   grad_x            NULL or bf16 [T, hidden]: the combine of grad_out_x with
 *                     no weights and no bias (slot order, binary32, RNE).
 *   grad_topk_weights NULL or fp32 [T, K]: grad_out_w[dst[t,k]], 0 for an
 *                     empty slot (0 everywhere when grad_out_w is NULL).
 */
ep_status ep_dispatch_backward(const ep_handle *h, const void *grad_out_x, int32_t hidden,
                               const float *grad_out_w, void *grad_x, float *grad_topk_weights,
                               hipStream_t stream);

/*
 * Profiling hook (the tracing the pages leave to CUDA events, [Ch8 §8.2]):
 * the next layout, dispatch, combine or backward call made on this host
 * thread stamps `start` when its first kernel begins and `stop` when its
 * last kernel ends.  The events ride on the kernel dispatches themselves
 * (AMD's hipExtLaunchKernel), so the interval holds kernel execution only,
 * not queueing or launch latency.  Either may be NULL; both must have been
 * created by the caller on the current device.  The hook applies to exactly
 * one call (consumed even if that call fails validation); a call that
 * launches nothing stamps nothing.
 */
ep_status ep_time_next_call(hipEvent_t start, hipEvent_t stop);

/* Static text for a status code. */
const char *ep_status_str(ep_status s);

#ifdef __cplusplus
}
#endif

#endif /* EP_H */
