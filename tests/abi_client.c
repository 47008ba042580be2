/*
 * A plain C client of libep.so: no torch and no Python in the path.  It reads
 * a routing and payloads from binary files, runs ep_layout, ep_dispatch (bf16
 * rows, top-k weights, zero padding, streaming stores) and ep_combine
 * (weights and an expert bias) through the C ABI on a stream of its own,
 * with buffers from hipMalloc, and writes the layout and every output back
 * to files.
 *
 * ep_client_run(DIR, T, K, E, A, H)
 *   reads  DIR/topk_idx.bin (int64 [T,K]), x.bin (bf16 bits [T,H]),
 *          w.bin (fp32 [T,K]), y.bin (bf16 bits [capacity,H]),
 *          bias.bin (bf16 bits [E,H]),
 *   writes DIR/counts.bin, psum.bin, dst.bin, src_meta.bin (int32),
 *          out_x.bin (bf16 bits [capacity,H], untouched rows 0xA5),
 *          out_w.bin (fp32 [capacity]), out.bin (bf16 bits [T,H]),
 *          scalars.txt (num_expanded num_recv_tokens error_bits invalid),
 *   with capacity = ep_capacity_bound(T, K, E, A); returns 0, or 1 after
 *   printing what failed, or 2 for bad sizes.  Built as a shared object it
 *   is called in-process (tests/test_abi_client.py); built as a program,
 *   `abi_client DIR T K E A H` runs the same function.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ep.h"

#define HIP_TRY(call)                                                             \
    do {                                                                          \
        hipError_t e_ = (call);                                                   \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));     \
            goto done;                                                            \
        }                                                                         \
    } while (0)

#define EP_TRY(call)                                                              \
    do {                                                                          \
        ep_status s_ = (call);                                                    \
        if (s_ != EP_OK) {                                                        \
            fprintf(stderr, "%s failed: %s\n", #call, ep_status_str(s_));         \
            goto done;                                                            \
        }                                                                         \
    } while (0)

static int file_path(char *buf, size_t n, const char *dir, const char *name) {
    return snprintf(buf, n, "%s/%s", dir, name) < (int)n;
}

/* Read exactly n bytes of DIR/name into a new device buffer (NULL on error). */
static void *load(const char *dir, const char *name, size_t n) {
    char p[4096];
    void *host = malloc(n ? n : 1), *dev = NULL;
    FILE *f = file_path(p, sizeof(p), dir, name) ? fopen(p, "rb") : NULL;
    int ok = host && f && fread(host, 1, n, f) == n;
    if (f) fclose(f);
    if (ok && hipMalloc(&dev, n ? n : 16) != hipSuccess) {
        dev = NULL;
        ok = 0;
    }
    if (ok && hipMemcpy(dev, host, n, hipMemcpyHostToDevice) != hipSuccess) ok = 0;
    free(host);
    if (!ok) {
        fprintf(stderr, "cannot load %zu bytes of %s/%s\n", n, dir, name);
        if (dev) hipFree(dev);
        return NULL;
    }
    return dev;
}

/* Copy n bytes of a device buffer to DIR/name; 0 on success. */
static int save(const char *dir, const char *name, const void *dev, size_t n) {
    char p[4096];
    void *host = malloc(n ? n : 1);
    int ok = host && hipMemcpy(host, dev, n, hipMemcpyDeviceToHost) == hipSuccess;
    FILE *f = ok && file_path(p, sizeof(p), dir, name) ? fopen(p, "wb") : NULL;
    ok = ok && f && fwrite(host, 1, n, f) == n;
    if (f) fclose(f);
    free(host);
    if (!ok) fprintf(stderr, "cannot save %s/%s\n", dir, name);
    return ok ? 0 : 1;
}

int ep_client_run(const char *dir, int32_t T, int32_t K, int32_t E, int32_t A, int32_t H) {
    const int64_t cap = ep_capacity_bound(T, K, E, A);
    if (cap < 0 || H <= 0) {
        fprintf(stderr, "bad sizes\n");
        return 2;
    }
    if (ep_handle_sizeof() != sizeof(ep_handle)) {
        fprintf(stderr, "ep_handle layout mismatch\n");
        return 1;
    }
    const size_t slots = (size_t)T * K, rows = (size_t)cap;
    int rc = 1;
    int stream_made = 0;
    hipStream_t stream;
    void *idx = NULL, *x = NULL, *y = NULL, *bias = NULL, *out_x = NULL, *out = NULL, *ws = NULL;
    float *w = NULL, *out_w = NULL;
    ep_handle h;
    int64_t num_expanded = 0;
    int32_t num_recv = 0, invalid = 0;
    uint32_t bits = 0;
    size_t ws_bytes;
    char p[4096];
    FILE *f;

    if (!(idx = load(dir, "topk_idx.bin", 8 * slots))) goto done;
    if (!(x = load(dir, "x.bin", 2 * (size_t)T * H))) goto done;
    if (!(w = (float *)load(dir, "w.bin", 4 * slots))) goto done;
    if (!(y = load(dir, "y.bin", 2 * rows * H))) goto done;
    if (!(bias = load(dir, "bias.bin", 2 * (size_t)E * H))) goto done;
    HIP_TRY(hipMalloc(&out_x, 2 * rows * H + 16));
    HIP_TRY(hipMalloc((void **)&out_w, 4 * rows + 16));
    HIP_TRY(hipMalloc(&out, 2 * (size_t)T * H + 16));
    ws_bytes = ep_workspace_bytes(T, K, E, A, cap);
    if (ws_bytes == 0) {
        fprintf(stderr, "ep_workspace_bytes rejected the sizes\n");
        goto done;
    }
    HIP_TRY(hipMalloc(&ws, ws_bytes));                  /* 256-byte aligned */
    HIP_TRY(hipStreamCreateWithFlags(&stream, hipStreamNonBlocking));
    stream_made = 1;
    /* Poison on the same stream: a non-blocking stream is not ordered after
     * work on the null stream. */
    HIP_TRY(hipMemsetAsync(out_x, 0xA5, 2 * rows * H, stream));
    HIP_TRY(hipMemsetAsync(out_w, 0xA5, 4 * rows, stream));

    EP_TRY(ep_handle_init(&h, T, K, E, A, cap, ws, ws_bytes, stream));
    EP_TRY(ep_layout(&h, idx, EP_I64, T, NULL, stream));
    /* zero padding, rows stored with streaming (non-temporal) stores */
    EP_TRY(ep_dispatch(&h, x, EP_BF16, H, NULL, 0, 0, 0, w, out_x, NULL, 0, 0, out_w,
                       EP_DISPATCH_ZERO_PADDING | EP_DISPATCH_STREAMING, stream));
    EP_TRY(ep_combine(&h, y, EP_BF16, H, w, bias, NULL, NULL, out, stream));
    EP_TRY(ep_handle_read_counts(&h, NULL, NULL, &num_expanded, &num_recv, &bits, &invalid,
                                 stream));
    HIP_TRY(hipStreamSynchronize(stream));

    if (save(dir, "counts.bin", h.counts, 4 * (size_t)E) ||
        save(dir, "psum.bin", h.psum, 4 * (size_t)(E + 1)) ||
        save(dir, "dst.bin", h.dst_slot, 4 * slots) ||
        save(dir, "src_meta.bin", h.src_meta, 4 * (size_t)num_expanded) ||
        save(dir, "out_x.bin", out_x, 2 * rows * H) || save(dir, "out_w.bin", out_w, 4 * rows) ||
        save(dir, "out.bin", out, 2 * (size_t)T * H))
        goto done;
    f = file_path(p, sizeof(p), dir, "scalars.txt") ? fopen(p, "w") : NULL;
    if (!f) goto done;
    fprintf(f, "%lld %d %u %d\n", (long long)num_expanded, num_recv, bits, invalid);
    fclose(f);
    rc = 0;

done:
    if (stream_made) hipStreamDestroy(stream);
    hipFree(idx);
    hipFree(x);
    hipFree(w);
    hipFree(y);
    hipFree(bias);
    hipFree(out_x);
    hipFree(out_w);
    hipFree(out);
    hipFree(ws);
    return rc;
}

int main(int argc, char **argv) {
    if (argc != 7) {
        fprintf(stderr, "usage: %s DIR T K E A H\n", argv[0]);
        return 2;
    }
    return ep_client_run(argv[1], atoi(argv[2]), atoi(argv[3]), atoi(argv[4]), atoi(argv[5]),
                         atoi(argv[6]));
}
