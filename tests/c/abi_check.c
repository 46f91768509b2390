/*
 * The library's C ABI called from plain C: device buffers from the HIP
 * runtime API (hipMalloc / hipMemcpy), no Python, no torch.  Every output is
 * compared, byte for byte, with the oracle's C functions on the same inputs
 * (test infrastructure: this program links the oracle library).  Exit 0
 * when everything matches.
 *
 * Definitions: C = A x B with int32 sums and packed int4 operands (INT4 GEMM
 * article, www.cf-1.com/news/6060138, §2.1, §3.2); the Q31 requantize and
 * the NHWC conv (MCU conv front-end article, news.rkmt.cn/news/16638, §2.1,
 * §2.3, §3.1).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "qgemm.h"

/* the oracle's C entry points (oracle/qgemm_oracle.c) */
int orc_gemm_s8s8_requant(const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb,
                          const int32_t *bias, const int32_t *mult, const int32_t *shift,
                          int8_t *C, int64_t ldc, int64_t N, int64_t K,
                          const int64_t *rows, int64_t nrows);
int orc_gemm_w4a8_requant(const int8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                          const int32_t *bias, const int32_t *mult, const int32_t *shift,
                          int8_t *C, int64_t ldc, int64_t N, int64_t K,
                          const int64_t *rows, int64_t nrows);
int orc_conv2d_nhwc_s8_requant(const int8_t *X, const int8_t *Wt, const int32_t *bias,
                               const int32_t *mult, const int32_t *shift, int8_t *Y,
                               int64_t batch, int64_t H, int64_t W, int64_t C_in, int64_t C_out,
                               int64_t KH, int64_t KW, int64_t sh, int64_t sw, int64_t ph,
                               int64_t pw, const int64_t *pix, int64_t npix);

static uint64_t state = 0x9E3779B97F4A7C15ull;

static uint32_t next32(void) /* xorshift64* */
{
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (uint32_t)((state * 0x2545F4914F6CDD1Dull) >> 32);
}

static int32_t uniform(int64_t lo, int64_t hi) /* [lo, hi] */
{
    return (int32_t)(lo + (int64_t)(next32() % (uint64_t)(hi - lo + 1)));
}

static void fill_i8(int8_t *p, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        p[i] = (int8_t)uniform(-128, 127);
}

static void fill_params(int32_t *bias, int32_t *mult, int32_t *shift, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        bias[i] = uniform(-32768, 32768);
        mult[i] = uniform(1 << 30, 2147483647);
        shift[i] = uniform(36, 44); /* mostly unsaturated at these K */
    }
}

#define HIP_OK(x)                                                            \
    do {                                                                     \
        if ((x) != hipSuccess) {                                             \
            fprintf(stderr, "%s:%d: %s failed\n", __FILE__, __LINE__, #x); \
            exit(2);                                                         \
        }                                                                    \
    } while (0)

static void *to_device(const void *h, size_t n)
{
    void *d = NULL;
    HIP_OK(hipMalloc(&d, n));
    HIP_OK(hipMemcpy(d, h, n, hipMemcpyHostToDevice));
    return d;
}

static int64_t *all_rows(int64_t n)
{
    int64_t *r = (int64_t *)malloc((size_t)n * sizeof *r);
    for (int64_t i = 0; i < n; ++i)
        r[i] = i;
    return r;
}

static int compare(const char *what, const int8_t *got, const int8_t *want, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        if (got[i] != want[i]) {
            printf("%s: output %zu differs (%d vs %d)\n", what, i, got[i], want[i]);
            return 1;
        }
    printf("%s: %zu outputs match\n", what, n);
    return 0;
}

/* int8 x int8 (w4 = 0) or int8 x packed int4 (w4 = 1) GEMM, requantized */
static int gemm_case(int64_t M, int64_t N, int64_t K, int w4)
{
    const size_t bbytes = (size_t)(w4 ? N * K / 2 : N * K);
    int8_t *A = malloc((size_t)(M * K)), *B = malloc(bbytes);
    int32_t *bias = malloc((size_t)N * 4), *mult = malloc((size_t)N * 4), *shift = malloc((size_t)N * 4);
    int8_t *C = malloc((size_t)(M * N)), *W = malloc((size_t)(M * N));
    fill_i8(A, (size_t)(M * K));
    fill_i8(B, bbytes);
    fill_params(bias, mult, shift, N);
    void *dA = to_device(A, (size_t)(M * K)), *dB = to_device(B, bbytes);
    void *dbias = to_device(bias, (size_t)N * 4), *dmult = to_device(mult, (size_t)N * 4);
    void *dshift = to_device(shift, (size_t)N * 4);
    void *dC = NULL;
    HIP_OK(hipMalloc(&dC, (size_t)(M * N)));
    qg_status st = w4 ? qgemm_w4a8_requant(dA, K, dB, K, dbias, dmult, dshift, dC, N, M, N, K, NULL)
                      : qgemm_s8s8_requant(dA, K, dB, K, dbias, dmult, dshift, dC, N, M, N, K, NULL);
    if (st != QG_OK) {
        printf("gemm %lld x %lld x %lld: %s\n", (long long)M, (long long)N, (long long)K,
               qg_status_string(st));
        return 1;
    }
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(C, dC, (size_t)(M * N), hipMemcpyDeviceToHost));
    int64_t *rows = all_rows(M);
    int ost = w4 ? orc_gemm_w4a8_requant(A, K, (const uint8_t *)B, K, bias, mult, shift, W, N, N, K, rows, M)
                 : orc_gemm_s8s8_requant(A, K, B, K, bias, mult, shift, W, N, N, K, rows, M);
    char what[96];
    snprintf(what, sizeof what, "%s %lldx%lldx%lld", w4 ? "w4a8" : "s8s8", (long long)M,
             (long long)N, (long long)K);
    int bad = ost != 0 ? (printf("%s: oracle status %d\n", what, ost), 1)
                       : compare(what, C, W, (size_t)(M * N));
    hipFree(dA), hipFree(dB), hipFree(dbias), hipFree(dmult), hipFree(dshift), hipFree(dC);
    free(A), free(B), free(bias), free(mult), free(shift), free(C), free(W), free(rows);
    return bad;
}

static int conv_case(int b, int H, int Wd, int ci, int co, int k, int s, int pad)
{
    const int Ho = (H + 2 * pad - k) / s + 1, Wo = (Wd + 2 * pad - k) / s + 1;
    const size_t nx = (size_t)b * H * Wd * ci, nw = (size_t)co * k * k * ci;
    const size_t ny = (size_t)b * Ho * Wo * co;
    int8_t *X = malloc(nx), *Wt = malloc(nw), *Y = malloc(ny), *R = malloc(ny);
    int32_t *bias = malloc((size_t)co * 4), *mult = malloc((size_t)co * 4), *shift = malloc((size_t)co * 4);
    fill_i8(X, nx);
    fill_i8(Wt, nw);
    fill_params(bias, mult, shift, co);
    void *dX = to_device(X, nx), *dW = to_device(Wt, nw);
    void *dbias = to_device(bias, (size_t)co * 4), *dmult = to_device(mult, (size_t)co * 4);
    void *dshift = to_device(shift, (size_t)co * 4);
    void *dY = NULL;
    HIP_OK(hipMalloc(&dY, ny));
    qg_status st = qconv2d_nhwc_s8_requant(dX, dW, dbias, dmult, dshift, dY, b, H, Wd, ci, co, k, k,
                                           s, s, pad, pad, NULL);
    char what[96];
    snprintf(what, sizeof what, "conv %dx%dx%dx%d->%d k%d s%d p%d", b, H, Wd, ci, co, k, s, pad);
    if (st != QG_OK) {
        printf("%s: %s\n", what, qg_status_string(st));
        return 1;
    }
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(Y, dY, ny, hipMemcpyDeviceToHost));
    int64_t *pix = all_rows((int64_t)b * Ho * Wo);
    int ost = orc_conv2d_nhwc_s8_requant(X, Wt, bias, mult, shift, R, b, H, Wd, ci, co, k, k, s, s,
                                         pad, pad, pix, (int64_t)b * Ho * Wo);
    int bad = ost != 0 ? (printf("%s: oracle status %d\n", what, ost), 1) : compare(what, Y, R, ny);
    hipFree(dX), hipFree(dW), hipFree(dbias), hipFree(dmult), hipFree(dshift), hipFree(dY);
    free(X), free(Wt), free(Y), free(R), free(bias), free(mult), free(shift), free(pix);
    return bad;
}

int main(void)
{
    int bad = 0;
    bad |= gemm_case(300, 260, 64, 0);    /* tile kernel */
    bad |= gemm_case(2048, 4096, 256, 0); /* persistent ring kernel (128 tiles) */
    bad |= gemm_case(16, 1024, 1024, 1);  /* skinny weight stream */
    bad |= gemm_case(40, 520, 4096, 1);   /* skinny, two token blocks */
    bad |= gemm_case(300, 260, 128, 1);   /* tile kernel, int4 weights */
    bad |= conv_case(2, 14, 15, 64, 64, 3, 1, 1);  /* LDS-band conv */
    bad |= conv_case(1, 13, 17, 32, 48, 3, 2, 1);  /* implicit-im2col conv */
    /* a rejected call: nothing is launched, and the status has a text */
    qg_status st = qgemm_s8s8_requant(NULL, 16, NULL, 16, NULL, NULL, NULL, NULL, 16, 1, 1, 16, NULL);
    if (st != QG_ERR_NULLPTR || qg_status_string(st) == NULL) {
        printf("null pointers: status %d\n", (int)st);
        bad = 1;
    }
    printf("c abi: %s\n", bad ? "MISMATCH" : "every output matches the oracle");
    return bad;
}
