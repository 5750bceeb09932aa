/*
 * sage_c_consumer.c -- a plain C program that uses the library through its
 * C ABI only (include/sage_mi355x.h): HIP runtime calls for device memory,
 * the library for the computation.  No C++, no Python, no torch.
 *
 * Usage:
 *   sage_c_consumer errors
 *       host-side validation only (no device is touched): invalid calls must
 *       return the documented status codes and a non-empty message
 *   sage_c_consumer run IN OUT B N H
 *       IN: Q, K, V as BF16 bits, each contiguous [B][N][H][128]; the
 *       one-call sage_attn_fwd with sm_scale = 1/sqrt(128) on the default
 *       stream; OUT: O as BF16 bits [B][N][H][128]
 *   sage_c_consumer run2 IN OUT B N H
 *       the same through the two calls: sage_quantized_carve,
 *       sage_quantize_qkv, then sage_attn_fwd_quantized
 * Prints "ok" and exits 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

#include <hip/hip_runtime_api.h>

#include "sage_mi355x.h"

#define FAIL(...) do { fprintf(stderr, __VA_ARGS__); fprintf(stderr, "\n"); return 1; } while (0)
#define HIPCHK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) FAIL("%s: %s", #x, hipGetErrorString(e_)); } while (0)

static int expect(sage_status got, sage_status want, const char* what)
{
    if (got != want) {
        fprintf(stderr, "%s: status %d (%s), expected %d\n", what, (int)got, sage_status_string(got), (int)want);
        return 1;
    }
    if (want != SAGE_OK && strlen(sage_last_error_message()) == 0) {
        fprintf(stderr, "%s: empty error message\n", what);
        return 1;
    }
    return 0;
}

static int errors_only(void)
{
    int bad = 0;
    sage_shape good = {1, 200, 2, 128}, d64 = {1, 200, 2, 64};
    size_t need = sage_workspace_bytes(good);
    if (need == 0 || sage_workspace_bytes(d64) != 0) FAIL("sage_workspace_bytes");
    sage_quantized qz;
    /* fake, never dereferenced device addresses: validation is host-only */
    void* ws = (void*)(uintptr_t)0x7f0000000000ull;
    bad |= expect(sage_quantized_carve(good, ws, need, &qz), SAGE_OK, "carve");
    bad |= expect(sage_quantized_carve(good, ws, need - 1, &qz), SAGE_ERR_WORKSPACE, "carve small");
    bad |= expect(sage_quantized_carve(d64, ws, need, &qz), SAGE_ERR_INVALID_ARGUMENT, "carve D=64");
    sage_bf16_in in = {(const void*)(uintptr_t)0x7e0000000000ull, 200 * 2 * 128, 2 * 128, 128};
    sage_bf16_in odd = in;
    odd.stride_n = 250;
    sage_bf16_out out = {(void*)(uintptr_t)0x7d0000000000ull, 200 * 2 * 128, 2 * 128, 128};
    bad |= expect(sage_quantize_qkv(NULL, &in, &in, &qz, NULL), SAGE_ERR_INVALID_ARGUMENT, "quantize NULL q");
    bad |= expect(sage_quantize_qkv(&in, &odd, &in, &qz, NULL), SAGE_ERR_UNSUPPORTED, "quantize odd stride");
    bad |= expect(sage_attn_fwd_quantized(&qz, NAN, &out, NULL), SAGE_ERR_INVALID_ARGUMENT, "mainloop NaN scale");
    bad |= expect(sage_attn_fwd(&in, &in, &in, good, 0.088f, &out, ws, need - 256, NULL), SAGE_ERR_WORKSPACE,
                  "one-call small workspace");
    sage_range r = {150, 51, 0, 2};
    bad |= expect(sage_attn_fwd_quantized_range(&qz, 0.088f, &r, &out, NULL), SAGE_ERR_INVALID_ARGUMENT,
                  "range past N");
    sage_norm_rope nr = {NULL, NULL, NULL, NULL, 1e-6f};
    bad |= expect(sage_quantize_qkv_norm_rope(&in, &in, &in, &nr, &qz, NULL), SAGE_ERR_INVALID_ARGUMENT,
                  "norm_rope NULL tables");
    if (bad) return 1;
    printf("ok\n");
    return 0;
}

static int run(const char* in_path, const char* out_path, int B, int N, int H, int two_calls)
{
    const size_t elems = (size_t)B * N * H * 128, bytes = elems * 2;
    uint16_t* host = (uint16_t*)malloc(3 * bytes);
    if (!host) FAIL("host allocation");
    FILE* f = fopen(in_path, "rb");
    if (!f || fread(host, 1, 3 * bytes, f) != 3 * bytes) FAIL("cannot read %s", in_path);
    fclose(f);
    sage_shape s = {B, N, H, 128};
    const size_t need = sage_workspace_bytes(s);
    if (need == 0) FAIL("invalid shape");
    void *q, *k, *v, *o, *ws;
    HIPCHK(hipMalloc(&q, bytes));
    HIPCHK(hipMalloc(&k, bytes));
    HIPCHK(hipMalloc(&v, bytes));
    HIPCHK(hipMalloc(&o, bytes));
    HIPCHK(hipMalloc(&ws, need));            /* hipMalloc returns 256-byte aligned memory */
    HIPCHK(hipMemcpy(q, host, bytes, hipMemcpyHostToDevice));
    HIPCHK(hipMemcpy(k, host + elems, bytes, hipMemcpyHostToDevice));
    HIPCHK(hipMemcpy(v, host + 2 * elems, bytes, hipMemcpyHostToDevice));
    const int64_t sb = (int64_t)N * H * 128, sn = (int64_t)H * 128, sh = 128;
    sage_bf16_in qi = {q, sb, sn, sh}, ki = {k, sb, sn, sh}, vi = {v, sb, sn, sh};
    sage_bf16_out oo = {o, sb, sn, sh};
    const float sm_scale = (float)(1.0 / sqrt(128.0));
    if (two_calls) {
        sage_quantized qz;
        sage_status st = sage_quantized_carve(s, ws, need, &qz);
        if (st != SAGE_OK) FAIL("sage_quantized_carve: %s: %s", sage_status_string(st), sage_last_error_message());
        st = sage_quantize_qkv(&qi, &ki, &vi, &qz, NULL);
        if (st != SAGE_OK) FAIL("sage_quantize_qkv: %s: %s", sage_status_string(st), sage_last_error_message());
        st = sage_attn_fwd_quantized(&qz, sm_scale, &oo, NULL);
        if (st != SAGE_OK)
            FAIL("sage_attn_fwd_quantized: %s: %s", sage_status_string(st), sage_last_error_message());
    } else {
        sage_status st = sage_attn_fwd(&qi, &ki, &vi, s, sm_scale, &oo, ws, need, NULL);
        if (st != SAGE_OK) FAIL("sage_attn_fwd: %s: %s", sage_status_string(st), sage_last_error_message());
    }
    HIPCHK(hipDeviceSynchronize());
    HIPCHK(hipMemcpy(host, o, bytes, hipMemcpyDeviceToHost));
    f = fopen(out_path, "wb");
    if (!f || fwrite(host, 1, bytes, f) != bytes) FAIL("cannot write %s", out_path);
    fclose(f);
    HIPCHK(hipFree(q));
    HIPCHK(hipFree(k));
    HIPCHK(hipFree(v));
    HIPCHK(hipFree(o));
    HIPCHK(hipFree(ws));
    free(host);
    printf("ok\n");
    return 0;
}

int main(int argc, char** argv)
{
    if (argc == 2 && strcmp(argv[1], "errors") == 0) return errors_only();
    if (argc == 7 && (strcmp(argv[1], "run") == 0 || strcmp(argv[1], "run2") == 0))
        return run(argv[2], argv[3], atoi(argv[4]), atoi(argv[5]), atoi(argv[6]), strcmp(argv[1], "run2") == 0);
    fprintf(stderr, "usage: %s errors | run IN OUT B N H | run2 IN OUT B N H\n", argv[0]);
    return 2;
}
