/*
 * ep_oracle.c - CPU oracle for MoE routing layout, dispatch copy and combine.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * statement of what the GPU path computes.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg load it; the product path never
 * does.  It shares no code, header, table or helper with the HIP library.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC
 * (x86-64 SSE arithmetic: every float operation below is one IEEE-754
 * binary32 operation rounded to nearest even; nothing is fused or reassociated).
 *
 * Sources (web pages; each function cites the section it follows):
 *   [Ch7]    DeepEP source notes, chapter 7 "V2: how dispatch builds expert
 *            inputs" (bowenzhou.top/repos/deepep/07-v2-dispatch)
 *   [Ch8]    DeepEP source notes, chapter 8 "V2: combine, handle and async
 *            overlap" (bowenzhou.top/repos/deepep/08-v2-combine-events)
 *   [vLLM]   digest of vLLM pull request 52781, "DeepEP v2 combine made
 *            asynchronous" (prhub.com.cn/vllm-project/vllm/pull/52781)
 *   [README] DeepEP README, Chinese rendering (gittoolsai.com)
 *
 * Readings where the pages leave a step open (plainest reading consistent
 * with the rest; the same list is kept with the design notes):
 *   R1  rows inside an expert segment are ordered by ascending flattened slot
 *       index i = t*K + k (a stable counting sort); one rank means one source.
 *   R2  an expert with no routed slot gets an empty segment.
 *   R3  psum is exclusive with E+1 entries over aligned counts; counts are the
 *       unaligned per-expert counts.
 *   R4  source metadata is one int32 per expanded row holding t*K + k, and -1
 *       on alignment-gap rows; rows at or past psum[E] are not written.
 *   R5  ids outside [-1, E) are treated as empty slots and counted as invalid.
 *   R6  duplicate experts inside one token are not merged; each slot gets its
 *       own row, ordered by k.
 *   R7  a token whose slots are all empty combines to +0.0 and does not count
 *       towards num_recv_tokens.
 *   R8  zero padding clears gap rows only (x bytes, scale entries, weight).
 *   R9  bias is the expert's output bias [E, H], added to the expert row
 *       before the weight is applied: out = sum_k w_k * (y_k + b[e_k]).
 *   R10 missing top-k weights mean weight 1 (the product is skipped).
 *   R11 combine accumulates in binary32, in slot order k = 0..K-1, starting at
 *       +0.0, with separately rounded multiply and add; the result is rounded
 *       to bf16 to nearest even (NaN becomes the quiet NaN 0x7FC0).
 *   R12 num_recv_tokens is the number of tokens with at least one valid slot.
 *   R17-R22 (rank layout, per-token biases, gradients) are stated with the
 *       functions that use them below.
 *   R23 the FP8 quantiser (which the pages do not give) follows the
 *       per-128-channel recipe of the workload inputs; see
 *       oracle_quantize_fp8.
 *
 * Where no reading is needed the definition is the pages' own.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/*
 * Threads of the token loops of oracle_dispatch and of the combines (the
 * benchmark's all-cores leg; 1 by default).  Tokens are independent: each
 * writes only its own slot rows or output row, so any thread count gives
 * the same bytes as one thread.  Every other function is single-threaded.
 */
static int g_threads = 1;

void oracle_set_threads(int threads)
{
    g_threads = threads > 1 ? threads : 1;
}

/* Error codes returned by oracle_layout. */
#define ORACLE_OK 0
#define ORACLE_ERR_CAPACITY 1
#define ORACLE_ERR_ARGS 2

/*
 * Worst-case number of expanded rows at one rank when the receive counts are
 * not read back by the CPU [Ch7 §7.2, the no-CPU-sync sizing]: each token can
 * land on at most min(K, E) local experts, each expert segment can waste up to
 * A-1 rows of alignment, and the total is rounded up to a multiple of A.
 */
int64_t oracle_capacity_bound(int64_t T, int64_t K, int64_t E, int64_t A)
{
    int64_t per_token = K < E ? K : E;
    int64_t n = T * per_token + (A - 1) * E;
    return (n + A - 1) / A * A;
}

/*
 * Routing layout [Ch7 §7.1 (input contract, -1 means no selection),
 * §7.2 (counts, source metadata and slot index built with the dispatch),
 * §7.3 (expert-expanded layout, expert_alignment), §7.5 (handle fields:
 * unaligned counts, per-expert prefix sums, destination slots, source
 * metadata)].
 *
 * topk_idx [T*K] row-major int64.  Outputs:
 *   counts[E]          unaligned per-expert counts
 *   psum[E+1]          exclusive scan of counts aligned up to A (R3)
 *   dst[T*K]           expanded row of slot i, -1 for empty slots
 *   src_meta[capacity] slot index of each filled row, -1 on gap rows (R4)
 *   scalars[3]         {num_recv_tokens, invalid_count, num_expanded}
 * On capacity overflow only counts, psum and scalars are written.
 */
int oracle_layout(int64_t T, int64_t K, int64_t E, int64_t A, int64_t capacity,
                  const int64_t *topk_idx, int32_t *counts, int32_t *psum,
                  int32_t *dst, int32_t *src_meta, int64_t *scalars)
{
    if (T < 0 || K <= 0 || E <= 0 || A <= 0 || capacity < 0)
        return ORACLE_ERR_ARGS;

    int64_t invalid = 0, num_recv = 0;
    for (int64_t e = 0; e < E; ++e)
        counts[e] = 0;

    /* Count valid slots per expert and tokens with any valid slot. */
    for (int64_t t = 0; t < T; ++t) {
        int any = 0;
        for (int64_t k = 0; k < K; ++k) {
            int64_t e = topk_idx[t * K + k];
            if (e == -1)
                continue;
            if (e < 0 || e >= E) {          /* R5 */
                ++invalid;
                continue;
            }
            counts[e] += 1;
            any = 1;
        }
        num_recv += any;                    /* R12 */
    }

    /* Aligned exclusive prefix sum over experts (R2, R3). */
    int64_t run = 0;
    psum[0] = 0;
    for (int64_t e = 0; e < E; ++e) {
        int64_t aligned = (counts[e] + A - 1) / A * A;
        run += aligned;
        if (run > INT32_MAX)
            return ORACLE_ERR_ARGS;
        psum[e + 1] = (int32_t)run;
    }
    scalars[0] = num_recv;
    scalars[1] = invalid;
    scalars[2] = run;
    if (run > capacity)
        return ORACLE_ERR_CAPACITY;

    /* Place slots in ascending slot order (R1): the next free row of the
     * expert's segment. */
    int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    if (!fill)
        return ORACLE_ERR_ARGS;
    for (int64_t i = 0; i < T * K; ++i) {
        int64_t e = topk_idx[i];
        if (e < 0 || e >= E) {
            dst[i] = -1;
            continue;
        }
        int32_t row = psum[e] + fill[e];
        fill[e] += 1;
        dst[i] = row;
        src_meta[row] = (int32_t)i;
    }
    free(fill);

    /* Alignment gaps: rows [psum[e] + counts[e], psum[e+1]) hold no token. */
    for (int64_t e = 0; e < E; ++e)
        for (int64_t r = (int64_t)psum[e] + counts[e]; r < psum[e + 1]; ++r)
            src_meta[r] = -1;
    return ORACLE_OK;
}

/*
 * Dispatch copy epilogue into the expert-expanded layout [Ch7 §7.1 (x is a
 * bf16 matrix or FP8 data plus scale factors; weights optional), §7.3 (copy
 * epilogue writes received rows, scale factors with their own token/hidden
 * strides and per-row top-k weights; zero padding clears alignment gaps),
 * §7.4 (each expert owns one contiguous, aligned range)].
 *
 * x          [T, row_bytes] raw bytes (bf16: 2H bytes, FP8: H bytes)
 * sf         FP8 scale factors as 4-byte packs (one fp32, or four UE8M0
 *            exponent bytes; the pack count is an argument of the pages'
 *            epilogue), pack (t, j) at sf[t*sf_ts + j*sf_hs], j < num_sf;
 *            copied as bits; NULL when num_sf == 0
 * w          [T*K] top-k weights or NULL (R10: weight 1)
 * out_x      [capacity, row_bytes]
 * out_sf     element (r, j) at out_sf[r*o_ts + j*o_hs]; NULL if num_sf == 0
 * out_w      [capacity] per-row weight or NULL
 * Rows that are neither routed nor (with zero padding) gap rows are left as
 * they were.
 */
void oracle_dispatch(int64_t T, int64_t K, int64_t E, int64_t row_bytes,
                     const uint8_t *x, int64_t num_sf, const uint32_t *sf,
                     int64_t sf_ts, int64_t sf_hs, const float *w,
                     const int32_t *counts, const int32_t *psum,
                     const int32_t *dst, uint8_t *out_x, uint32_t *out_sf,
                     int64_t o_ts, int64_t o_hs, float *out_w, int zero_padding)
{
#pragma omp parallel for num_threads(g_threads) if (g_threads > 1) schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t r = dst[t * K + k];
            if (r < 0)
                continue;
            memcpy(out_x + r * row_bytes, x + t * row_bytes, (size_t)row_bytes);
            for (int64_t j = 0; j < num_sf; ++j)
                out_sf[r * o_ts + j * o_hs] = sf[t * sf_ts + j * sf_hs];
            if (out_w)
                out_w[r] = w ? w[t * K + k] : 1.0f;
        }
    }
    if (!zero_padding)
        return;
#pragma omp parallel for num_threads(g_threads) if (g_threads > 1) schedule(static)
    for (int64_t e = 0; e < E; ++e) {
        for (int64_t r = (int64_t)psum[e] + counts[e]; r < psum[e + 1]; ++r) {
            memset(out_x + r * row_bytes, 0, (size_t)row_bytes);
            for (int64_t j = 0; j < num_sf; ++j)
                out_sf[r * o_ts + j * o_hs] = 0;
            if (out_w)
                out_w[r] = 0.0f;
        }
    }
}

/* bf16 bit pattern -> binary32: the bf16 bits are the high half (exact). */
static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary32 -> bf16 by round to nearest, ties to even (R11). */
static uint16_t f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return 0x7FC0;
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/*
 * Combine: follow the handle back to token order and reduce the expert
 * outputs [Ch8 §8.1 (combine reads the handle's source metadata and
 * reduces back to the source; bias and gate-weight reduction can be fused;
 * the kernel takes bf16 x and fp32 top-k weights), vLLM digest "Implementation
 * breakdown" (combine input must be bf16; top-k weights may be passed as
 * None)].  Readings R7, R9, R10, R11.
 *
 * y    [rows, H] bf16 bits, row r at y + r*H
 * w    [T*K] fp32 or NULL; bias [E, H] bf16 bits or NULL
 * out  [T, H] bf16 bits
 */
static void combine_tokens(int64_t T, int64_t K, int64_t H, const uint16_t *y,
                           const float *w, const uint16_t *bias,
                           const int64_t *topk_idx, const int32_t *dst,
                           const uint16_t *b0, const uint16_t *b1, uint16_t *out)
{
#pragma omp parallel for num_threads(g_threads) if (g_threads > 1) schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int64_t k = 0; k < K; ++k) {
                int64_t r = dst[t * K + k];
                if (r < 0)
                    continue;
                float v = bf16_to_f32(y[r * H + h]);
                if (bias) {
                    int64_t e = topk_idx[t * K + k];
                    v = v + bf16_to_f32(bias[e * H + h]);
                }
                float p = w ? w[t * K + k] * v : v;
                acc = acc + p;
            }
            if (b0)
                acc = acc + bf16_to_f32(b0[t * H + h]);
            if (b1)
                acc = acc + bf16_to_f32(b1[t * H + h]);
            out[t * H + h] = f32_to_bf16(acc);
        }
    }
}

void oracle_combine(int64_t T, int64_t K, int64_t H, const uint16_t *y,
                    const float *w, const uint16_t *bias,
                    const int64_t *topk_idx, const int32_t *dst, uint16_t *out)
{
    combine_tokens(T, K, H, y, w, bias, topk_idx, dst, NULL, NULL, out);
}

/*
 * The same weighted sum in binary64, without the final rounding to bf16.
 * Used only to bound the binary32 result of oracle_combine in the tests; it
 * is not a parity target.  Terms are the binary64 values of the same inputs.
 */
void oracle_combine_f64(int64_t T, int64_t K, int64_t H, const uint16_t *y,
                        const float *w, const uint16_t *bias,
                        const int64_t *topk_idx, const int32_t *dst,
                        double *out, double *abs_terms)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < H; ++h) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t r = dst[t * K + k];
                if (r < 0)
                    continue;
                double v = (double)bf16_to_f32(y[r * H + h]);
                if (bias)
                    v += (double)bf16_to_f32(bias[topk_idx[t * K + k] * H + h]);
                double p = w ? (double)w[t * K + k] * v : v;
                acc += p;
                mag += p < 0 ? -p : p;
            }
            out[t * H + h] = acc;
            abs_terms[t * H + h] = mag;
        }
    }
}

/*
 * Backward of combine [README, training example: the backward of combine is
 * a dispatch of the gradient and the combined top-k weights carry the
 * weights' gradient; the forward is the combine above].  With
 * out[t] = sum_k w[t,k] * (y[r] + b[e]) (r = dst[t,k], e = topk_idx[t,k]) and
 * g = d loss / d out (bf16 [T, H]):
 *   grad_y[r][h]    = bf16(fl32(w[t,k] * g[t][h]))     (g itself if w is NULL)
 *   grad_w[t,k]     = sum_h g[t][h] * (y[r][h] + b[e][h])   (binary64, no
 *                     rounding of the terms: the reference value), 0 for an
 *                     empty slot
 *   grad_bias[e][h] = sum over the rows of expert e of w * g[t][h]
 *                     (binary64; each product of a binary32 weight and a
 *                     bf16 value is exact in binary64)
 * grad_w and grad_bias are reference values: binary64 sums of exact terms,
 * so their evaluation order changes them only by binary64 rounding.  Any
 * output pointer may be NULL.  Rows of grad_y that hold no slot are not
 * written.
 */
void oracle_combine_backward(int64_t T, int64_t K, int64_t E, int64_t H,
                             const uint16_t *g, const float *w,
                             const uint16_t *y, const uint16_t *bias,
                             const int64_t *topk_idx, const int32_t *dst,
                             const int32_t *counts, const int32_t *psum,
                             const int32_t *src_meta, uint16_t *grad_y,
                             double *grad_w, double *grad_bias)
{
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t r = dst[t * K + k];
            if (grad_w)
                grad_w[t * K + k] = 0.0;
            if (r < 0)
                continue;
            int64_t e = topk_idx[t * K + k];
            double acc = 0.0;
            for (int64_t h = 0; h < H; ++h) {
                float gv = bf16_to_f32(g[t * H + h]);
                if (grad_y) {
                    float s = w ? w[t * K + k] * gv : gv;
                    grad_y[r * H + h] = f32_to_bf16(s);
                }
                if (grad_w) {
                    double v = (double)bf16_to_f32(y[r * H + h]);
                    if (bias)
                        v += (double)bf16_to_f32(bias[e * H + h]);
                    acc += (double)gv * v;
                }
            }
            if (grad_w)
                grad_w[t * K + k] = acc;
        }
    }
    if (!grad_bias)
        return;
    for (int64_t e = 0; e < E; ++e) {
        for (int64_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int64_t r = psum[e]; r < (int64_t)psum[e] + counts[e]; ++r) {
                int64_t i = src_meta[r];
                int64_t t = i / K;
                double gv = (double)bf16_to_f32(g[t * H + h]);
                acc += w ? (double)w[i] * gv : gv;
            }
            grad_bias[e * H + h] = acc;
        }
    }
}

/*
 * Backward of dispatch [README, training example: the backward of dispatch
 * is a combine of the gradient rows, returning the gradient of the
 * dispatched top-k weights too].  With go = d loss / d out_x (bf16
 * [capacity, H]) and gw = d loss / d out_w ([capacity], may be NULL):
 *   grad_x[t]   = the combine of go with no weights and no bias
 *   grad_w[t,k] = gw[dst[t,k]], 0 for an empty slot
 */
void oracle_dispatch_backward(int64_t T, int64_t K, int64_t H,
                              const uint16_t *go, const float *gw,
                              const int64_t *topk_idx, const int32_t *dst,
                              uint16_t *grad_x, float *grad_w)
{
    if (grad_x)
        oracle_combine(T, K, H, go, NULL, NULL, topk_idx, dst, grad_x);
    if (!grad_w)
        return;
    for (int64_t i = 0; i < T * K; ++i)
        grad_w[i] = (dst[i] >= 0 && gw) ? gw[dst[i]] : 0.0f;
}

/*
 * Non-expanded ("rank") layout [Ch7 §7.4: the normal layout keeps each
 * received token once, [received_tokens, hidden] plus top-k metadata;
 * §7.5: the handle keeps the received-token count].  At one rank a token is
 * received when it has at least one valid slot (R12); received tokens keep
 * their order.  recv_row[t] is its row (-1 if not received); recv_src[row]
 * is the token of each row.  Returns the number of received tokens.
 */
int64_t oracle_rank_layout(int64_t T, int64_t K, int64_t E,
                           const int64_t *topk_idx, int32_t *recv_row,
                           int32_t *recv_src)
{
    int64_t rows = 0;
    for (int64_t t = 0; t < T; ++t) {
        int any = 0;
        for (int64_t k = 0; k < K; ++k) {
            int64_t e = topk_idx[t * K + k];
            if (e >= 0 && e < E)
                any = 1;
        }
        if (any) {
            recv_row[t] = (int32_t)rows;
            recv_src[rows] = (int32_t)t;
            ++rows;
        } else {
            recv_row[t] = -1;
        }
    }
    return rows;
}

/*
 * Dispatch into the rank layout [Ch7 §7.3: the epilogue writes the received
 * rows, their scale factors and the received top-k ids and weights].  Row
 * recv_row[t] gets the bytes of x[t], its scales, the token's top-k ids
 * (-1 for an empty or invalid slot) and weights (0 for such a slot; 1 for a
 * valid slot when w is NULL).  Rows of tokens that are not received do not
 * exist; nothing else is written.
 */
void oracle_dispatch_rank(int64_t T, int64_t K, int64_t E, int64_t row_bytes,
                          const uint8_t *x, int64_t num_sf, const uint32_t *sf,
                          int64_t sf_ts, int64_t sf_hs, const float *w,
                          const int64_t *topk_idx, const int32_t *recv_row,
                          uint8_t *out_x, uint32_t *out_sf, int64_t o_ts,
                          int64_t o_hs, int64_t *out_idx, float *out_w)
{
    for (int64_t t = 0; t < T; ++t) {
        int64_t r = recv_row[t];
        if (r < 0)
            continue;
        memcpy(&out_x[r * row_bytes], &x[t * row_bytes], (size_t)row_bytes);
        for (int64_t j = 0; j < num_sf; ++j)
            out_sf[r * o_ts + o_hs * j] = sf[t * sf_ts + sf_hs * j];
        for (int64_t k = 0; k < K; ++k) {
            int64_t e = topk_idx[t * K + k];
            int valid = e >= 0 && e < E;
            if (out_idx)
                out_idx[r * K + k] = valid ? e : -1;
            if (out_w)
                out_w[r * K + k] = valid ? (w ? w[t * K + k] : 1.0f) : 0.0f;
        }
    }
}

/*
 * Combine from the rank layout with the two per-token biases [Ch8 §8.1: the
 * combine takes bias_0 and bias_1 and reduces back to the source token].  At
 * one rank each received token has exactly one row, already reduced over its
 * experts, so out[t][h] = bf16(fl32(fl32(v + b0[t][h]) + b1[t][h])) with
 * v = x[recv_row[t]][h], or +0.0 for a token that was not received.  Either
 * bias may be NULL (its add is skipped).
 */
void oracle_combine_rank(int64_t T, int64_t H, const uint16_t *x,
                         const int32_t *recv_row, const uint16_t *b0,
                         const uint16_t *b1, uint16_t *out)
{
    for (int64_t t = 0; t < T; ++t) {
        int64_t r = recv_row[t];
        for (int64_t h = 0; h < H; ++h) {
            float acc = r >= 0 ? bf16_to_f32(x[r * H + h]) : 0.0f;
            if (b0)
                acc = acc + bf16_to_f32(b0[t * H + h]);
            if (b1)
                acc = acc + bf16_to_f32(b1[t * H + h]);
            out[t * H + h] = f32_to_bf16(acc);
        }
    }
}

/*
 * The expanded combine with the per-token biases added after the slot
 * reduction (R9 for the expert bias; bias_0 then bias_1 per token):
 *   out[t][h] = bf16(fl32(fl32(acc + b0[t][h]) + b1[t][h]))
 * where acc is oracle_combine's binary32 slot-order sum.
 */
void oracle_combine_token_bias(int64_t T, int64_t K, int64_t H,
                               const uint16_t *y, const float *w,
                               const uint16_t *bias, const int64_t *topk_idx,
                               const int32_t *dst, const uint16_t *b0,
                               const uint16_t *b1, uint16_t *out)
{
    combine_tokens(T, K, H, y, w, bias, topk_idx, dst, b0, b1, out);
}

/*
 * FP8 quantisation of bf16 rows, the producer of dispatch's FP8 input
 * [Ch7 §7.1: FP8 data travels with per-block scale factors; §7.3: the
 * epilogue takes the number of 4-byte scale packs].  The pages give no
 * quantiser; the reading used (R23) is the per-128-channel recipe of the
 * workload inputs, plus a power-of-two (UE8M0) variant:
 *   amax  = largest |x| of the block (NaN entries skipped), binary32
 *   s     = max(amax, 1e-12f) / 448, one binary32 division
 *   F32   : the block's pack is the binary32 s; divisor = s
 *   UE8M0 : s rounded up to a power of two 2^(e-127); the block's byte is e,
 *           four blocks per pack, the lowest block in the low byte (a last
 *           partial pack is zero-filled); divisor = 2^(e-127)
 *   code  = E4M3FN nearest to clamp(x / divisor, -448, 448) (binary32
 *           division), ties to the even code; a NaN quotient gives 0x7F.
 * E4M3FN: sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, code 0x7F (and 0xFF) NaN, largest finite 448.
 */
#define ORACLE_SF_F32 0
#define ORACLE_SF_UE8M0 1

/* exact value of 2^n for |n| < 200 */
static double pow2(int n)
{
    double v = 1.0;
    for (; n > 0; --n)
        v *= 2.0;
    for (; n < 0; ++n)
        v *= 0.5;
    return v;
}

/* magnitude of the E4M3FN code c, 0 <= c <= 126 */
static double e4m3_magnitude(int c)
{
    int e = c >> 3, m = c & 7;
    return e == 0 ? m * pow2(-9) : (8 + m) * pow2(e - 10);
}

static uint32_t f32_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

static float bits_f32(uint32_t u)
{
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary32 -> E4M3FN: clamp to +-448, nearest magnitude, ties to even code */
static uint8_t e4m3_from_f32(float v)
{
    if (v != v)
        return 0x7F;
    uint8_t sign = (f32_bits(v) >> 31) ? 0x80 : 0x00;
    double a = v < 0 ? -(double)v : (double)v;
    if (a > 448.0)
        a = 448.0;
    int lo = 0;                           /* largest code whose value <= a */
    while (lo < 126 && e4m3_magnitude(lo + 1) <= a)
        ++lo;
    int code = lo;
    if (lo < 126) {
        double dlo = a - e4m3_magnitude(lo), dhi = e4m3_magnitude(lo + 1) - a;
        if (dhi < dlo || (dhi == dlo && ((lo + 1) & 1) == 0))
            code = lo + 1;
    }
    return (uint8_t)(sign | code);
}

/* Codes of n binary32 values (exported for pinning the conversion). */
void oracle_f32_to_e4m3(int64_t n, const float *in, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = e4m3_from_f32(in[i]);
}

/* Scale packs per row: H/128 for F32, ceil(H/512) for UE8M0. */
int64_t oracle_sf_packs(int64_t H, int format)
{
    int64_t blocks = H / 128;
    return format == ORACLE_SF_UE8M0 ? (blocks + 3) / 4 : blocks;
}

/*
 * x bf16 [T, H] (H % 128 == 0) -> q E4M3FN codes [T, H] and scale packs
 * sf[t*s_ts + p*s_hs], p < oracle_sf_packs(H, format).
 */
void oracle_quantize_fp8(int64_t T, int64_t H, const uint16_t *x, int format,
                         uint8_t *q, uint32_t *sf, int64_t s_ts, int64_t s_hs)
{
    int64_t packs = oracle_sf_packs(H, format);
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t p = 0; p < packs; ++p)
            sf[t * s_ts + p * s_hs] = 0;
        for (int64_t j = 0; j < H / 128; ++j) {
            const uint16_t *blk = x + t * H + j * 128;
            float amax = 0.0f;
            for (int i = 0; i < 128; ++i) {
                float a = bits_f32(f32_bits(bf16_to_f32(blk[i])) & 0x7FFFFFFFu);
                if (a > amax)
                    amax = a;
            }
            float s = (amax > 1e-12f ? amax : 1e-12f) / 448.0f;
            float divisor = s;
            if (format == ORACLE_SF_UE8M0) {
                uint32_t e = (f32_bits(s) >> 23) & 0xFF;
                if (f32_bits(s) & 0x7FFFFFu)
                    ++e;                  /* round up to the next power of two */
                divisor = bits_f32(e << 23);
                sf[t * s_ts + (j / 4) * s_hs] |= e << (8 * (j % 4));
            } else {
                sf[t * s_ts + j * s_hs] = f32_bits(s);
            }
            for (int i = 0; i < 128; ++i)
                q[t * H + j * 128 + i] = e4m3_from_f32(bf16_to_f32(blk[i]) / divisor);
        }
    }
}

/*
 * Quantising dispatch: the quantiser above followed by the dispatch copy of
 * the codes and scale packs into the expanded layout (same weights and zero
 * padding rules as oracle_dispatch).
 */
void oracle_dispatch_quant(int64_t T, int64_t K, int64_t E, int64_t H,
                           const uint16_t *x, int format, const float *w,
                           const int32_t *counts, const int32_t *psum,
                           const int32_t *dst, uint8_t *out_x, uint32_t *out_sf,
                           int64_t o_ts, int64_t o_hs, float *out_w,
                           int zero_padding)
{
    int64_t packs = oracle_sf_packs(H, format);
    uint8_t *q = malloc((size_t)(T * H > 0 ? T * H : 1));
    uint32_t *sf = malloc((size_t)(T * packs > 0 ? T * packs : 1) * sizeof *sf);
    if (!q || !sf) {
        free(q);
        free(sf);
        return;
    }
    oracle_quantize_fp8(T, H, x, format, q, sf, packs, 1);
    oracle_dispatch(T, K, E, H, q, packs, sf, packs, 1, w, counts, psum, dst,
                    out_x, out_sf, o_ts, o_hs, out_w, zero_padding);
    free(q);
    free(sf);
}
