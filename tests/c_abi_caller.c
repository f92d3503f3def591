/*
 * c_abi_caller.c -- one spec_mixed_accept call from plain C.
 *
 * The verify library's boundary is a C ABI: plain pointers and sizes, no
 * Python or torch types.  This program uses nothing else: the HIP runtime's
 * C API for device memory and a stream, and include/specverify.h.  It
 * reads a call's inputs from a file, runs the call on device buffers it
 * allocates itself, and writes the outputs to a file, for a test to compare
 * with the Python binding's results and with the oracle.
 *
 * Usage: c_abi_caller IN OUT
 *
 * IN (little-endian): int32 b, K, V, dtype, has_lengths; the target logits
 * [b, K+1, V] and draft logits [b, K, V] (dense, elements of the dtype);
 * draft tokens [b, K] int32; temperatures [b] double; draft lengths [b]
 * int32 when has_lengths; seeds [b] uint64.
 * OUT: int32 status (the call's return code), then n_accepted [b] int32,
 * tokens [b, K+1] int32, p_draft [b, K] float, q_draft [b, K] float,
 * target_argmax [b, K+1] int32.
 *
 * Exit status: 0 when the call returned SPEC_OK, 1 when it returned an
 * error (written to OUT), 2 on an I/O or HIP runtime failure.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "specverify.h"

#define HIP_CHECK(call)                                                                   \
    do {                                                                                  \
        hipError_t e_ = (call);                                                           \
        if (e_ != hipSuccess) {                                                           \
            fprintf(stderr, "c_abi_caller: %s failed: %s\n", #call, hipGetErrorString(e_)); \
            return 2;                                                                     \
        }                                                                                 \
    } while (0)

/* Reads n bytes into a new host buffer (NULL on a short read). */
static void *read_block(FILE *f, size_t n) {
    void *p = malloc(n ? n : 1);
    if (p && n && fread(p, 1, n, f) != n) {
        free(p);
        return NULL;
    }
    return p;
}

/* A device copy of n host bytes. */
static hipError_t to_device(void **dst, const void *src, size_t n) {
    hipError_t e = hipMalloc(dst, n ? n : 1);
    if (e != hipSuccess) return e;
    return n ? hipMemcpy(*dst, src, n, hipMemcpyHostToDevice) : hipSuccess;
}

int main(int argc, char **argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
        return 2;
    }
    FILE *in = fopen(argv[1], "rb");
    if (!in) {
        fprintf(stderr, "c_abi_caller: cannot open %s\n", argv[1]);
        return 2;
    }
    int32_t hdr[5];
    if (fread(hdr, sizeof(int32_t), 5, in) != 5) {
        fprintf(stderr, "c_abi_caller: short header\n");
        return 2;
    }
    const int b = hdr[0], K = hdr[1], V = hdr[2], dtype = hdr[3], has_len = hdr[4];
    if (b < 1 || K < 1 || V < 1 || (dtype != SPEC_F32 && dtype != SPEC_BF16)) {
        fprintf(stderr, "c_abi_caller: bad header\n");
        return 2;
    }
    const size_t es = dtype == SPEC_BF16 ? 2 : 4;
    const size_t n_t = (size_t)b * (K + 1) * V * es, n_d = (size_t)b * K * V * es;
    const size_t n_x = (size_t)b * K * sizeof(int32_t), n_T = (size_t)b * sizeof(double);
    const size_t n_len = has_len ? (size_t)b * sizeof(int32_t) : 0, n_s = (size_t)b * sizeof(uint64_t);
    void *h_t = read_block(in, n_t), *h_d = read_block(in, n_d), *h_x = read_block(in, n_x);
    void *h_T = read_block(in, n_T), *h_len = read_block(in, n_len), *h_s = read_block(in, n_s);
    fclose(in);
    if (!h_t || !h_d || !h_x || !h_T || !h_len || !h_s) {
        fprintf(stderr, "c_abi_caller: short input\n");
        return 2;
    }

    void *d_t, *d_d, *d_x, *d_T, *d_len = NULL, *d_s;
    HIP_CHECK(to_device(&d_t, h_t, n_t));
    HIP_CHECK(to_device(&d_d, h_d, n_d));
    HIP_CHECK(to_device(&d_x, h_x, n_x));
    HIP_CHECK(to_device(&d_T, h_T, n_T));
    if (has_len) HIP_CHECK(to_device(&d_len, h_len, n_len));
    HIP_CHECK(to_device(&d_s, h_s, n_s));

    const size_t n_n = (size_t)b * sizeof(int32_t), n_tok = (size_t)b * (K + 1) * sizeof(int32_t);
    const size_t n_pq = (size_t)b * K * sizeof(float);
    void *d_n, *d_tok, *d_p, *d_q, *d_am, *d_ws;
    HIP_CHECK(hipMalloc(&d_n, n_n));
    HIP_CHECK(hipMalloc(&d_tok, n_tok));
    HIP_CHECK(hipMalloc(&d_p, n_pq));
    HIP_CHECK(hipMalloc(&d_q, n_pq));
    HIP_CHECK(hipMalloc(&d_am, n_tok));
    const size_t ws_bytes = spec_mixed_workspace_bytes(b, K, V, dtype);
    if (ws_bytes == 0) {
        fprintf(stderr, "c_abi_caller: the sizes are outside what the library accepts\n");
        return 2;
    }
    HIP_CHECK(hipMalloc(&d_ws, ws_bytes));              /* hipMalloc memory is 256-byte aligned */
    hipStream_t st;
    HIP_CHECK(hipStreamCreate(&st));

    const int status = spec_mixed_accept(d_t, d_d, dtype, (int64_t)(K + 1) * V, V, (int64_t)K * V, V,
                                         (const int32_t *)d_x, b, K, V, (const double *)d_T,
                                         (const int32_t *)d_len, (const uint64_t *)d_s, (int32_t *)d_n,
                                         (int32_t *)d_tok, (float *)d_p, (float *)d_q, (int32_t *)d_am, d_ws,
                                         ws_bytes, (void *)st);
    HIP_CHECK(hipStreamSynchronize(st));

    void *h_n = malloc(n_n), *h_tok = malloc(n_tok), *h_p = malloc(n_pq), *h_q = malloc(n_pq), *h_am = malloc(n_tok);
    if (!h_n || !h_tok || !h_p || !h_q || !h_am) return 2;
    HIP_CHECK(hipMemcpy(h_n, d_n, n_n, hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(h_tok, d_tok, n_tok, hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(h_p, d_p, n_pq, hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(h_q, d_q, n_pq, hipMemcpyDeviceToHost));
    HIP_CHECK(hipMemcpy(h_am, d_am, n_tok, hipMemcpyDeviceToHost));

    FILE *out = fopen(argv[2], "wb");
    if (!out) {
        fprintf(stderr, "c_abi_caller: cannot open %s\n", argv[2]);
        return 2;
    }
    const int32_t st32 = status;
    int ok = fwrite(&st32, sizeof st32, 1, out) == 1;
    ok = ok && fwrite(h_n, 1, n_n, out) == n_n && fwrite(h_tok, 1, n_tok, out) == n_tok;
    ok = ok && fwrite(h_p, 1, n_pq, out) == n_pq && fwrite(h_q, 1, n_pq, out) == n_pq;
    ok = ok && fwrite(h_am, 1, n_tok, out) == n_tok;
    ok = (fclose(out) == 0) && ok;
    if (!ok) {
        fprintf(stderr, "c_abi_caller: cannot write %s\n", argv[2]);
        return 2;
    }

    HIP_CHECK(hipStreamDestroy(st));
    void *dev[] = {d_t, d_d, d_x, d_T, d_len, d_s, d_n, d_tok, d_p, d_q, d_am, d_ws};
    for (size_t i = 0; i < sizeof dev / sizeof dev[0]; ++i)
        if (dev[i]) HIP_CHECK(hipFree(dev[i]));
    void *host[] = {h_t, h_d, h_x, h_T, h_len, h_s, h_n, h_tok, h_p, h_q, h_am};
    for (size_t i = 0; i < sizeof host / sizeof host[0]; ++i) free(host[i]);
    if (status != SPEC_OK) fprintf(stderr, "c_abi_caller: %s\n", spec_status_string(status));
    return status == SPEC_OK ? 0 : 1;
}
