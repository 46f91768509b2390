/*
 * qgemm_oracle.c -- plain CPU oracle for the quantized GEMM / conv path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It
 * shares no code, header or table with the HIP library and includes no HIP
 * header.
 *
 * Sources of the definitions (web pages; section numbers are the pages' own):
 *   [INT4-GEMM]  "DeepGEMM" INT4 GEMM article, www.cf-1.com/news/6060138
 *                  §2.1 (two signed nibbles per byte), §3.2 (C = A*B with
 *                  packed INT4 in, INT32 out), §4.3 (B stored column-major).
 *   [MCU-CONV]   smart-speaker MCU conv front-end article,
 *                news.rkmt.cn/news/16638
 *                  §2.1 (output geometry and MAC count), §2.3 (Q31
 *                  requantize: 64-bit product, add half an LSB, arithmetic
 *                  shift, saturate; symmetric zero point 0; padding equals
 *                  the zero point), §3.1 (NHWC activations, weights
 *                  [out][kh][kw][in]), §3.2 (conv as C = A x B over an
 *                  im2col matrix), §3.3 (bias enters the requantize step;
 *                  the depthwise conv: one input channel per output
 *                  channel, weights [kh][kw][c]).
 *
 *   [FLATQUANT]  Ascend FlatQuant operator article, www.zwxr.cn/news/277566
 *                  «per-token 模式» (per-token INT4 scale from max|x|).
 *   [VOYAGER]    Voyager quantization article, www.dpshk.com/news/2695434
 *                  §1.1 (Q = round(x / scale) + zero_point).
 *
 * Readings where the pages are silent or contradict themselves:
 *   - packed INT4: element 2i is the LOW nibble of byte i, element 2i+1 the
 *     high nibble; codes are 4-bit two's complement (0x8 = -8).
 *   - bias is added to the int32 accumulator before the Q31 multiply.
 *   - the page's ">>" of a negative product is an arithmetic (flooring)
 *     shift, so the requantize rounds exact halves up (toward +infinity).
 *   - requant domain: acc + bias fits int32, mult in [0, 2^31-1],
 *     shift in [1, 63]; outside it the oracle reports ORC_E_DOMAIN/RANGE
 *     instead of producing a value.
 *   - GEMM layouts: A is [M][lda] row-major, B is [N][ldb] (K contiguous,
 *     i.e. column-major K x N); packed operands count lda/ldb in nibbles.
 *   - conv: NHWC input, OHWI weights, dilation 1, one group, symmetric
 *     padding filled with the input zero point (0 unless given), floor
 *     output-size formula.
 *   - asymmetric forms: one zero point per tensor for each operand and for
 *     the output, in [-128, 127]; the output zero point is added to the
 *     shifted value before the int8 saturation.
 *
 * Every entry point can compute a subset of output rows (GEMM) or output
 * pixels (conv) so that full-size problems can be checked on samples; the
 * selected results are written compactly, row r of the output holding the
 * r-th requested row/pixel.  OpenMP only spreads independent output rows
 * over threads; every dot product is summed in one thread, in k order.
 */
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORC_OK 0
#define ORC_E_RANGE 1   /* an int32 intermediate does not fit in int32 */
#define ORC_E_DOMAIN 2  /* shift or multiplier outside the stated domain */

/* ---- O1: packed INT4 element access ([INT4-GEMM] §2.1, §3.2) ---- */
int orc_int4_at(const uint8_t *row, int64_t i)
{
    uint8_t byte = row[i / 2];
    int code = (i % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
    return code < 8 ? code : code - 16;
}

/* ---- O3: Q31 requantize ([MCU-CONV] §2.3, bias per §3.3) ----
 * The output code is the product x * M of x = acc + bias and the Q31
 * multiplier, scaled down by 2^shift and rounded to the nearest integer; the
 * page rounds by adding half an LSB before an arithmetic (flooring) shift,
 * so a value exactly halfway between two integers goes up, toward +infinity.
 * The code is then saturated to the int8 range.  Below, the rounding is
 * stated through the quotient and remainder of a floor division, in 128-bit
 * integers, so that no intermediate can overflow for any shift in [1, 63]. */

/* Nearest integer to t / 2^s, exact halves rounded up. */
static __int128 round_half_up_pow2(__int128 t, int s)
{
    const __int128 unit = (__int128)1 << s;
    __int128 q = t / unit, r = t % unit;   /* C division truncates toward 0 */
    if (r < 0) {                           /* make q the floor, 0 <= r < unit */
        q -= 1;
        r += unit;
    }
    return 2 * r >= unit ? q + 1 : q;      /* a remainder of half or more rounds up */
}

/* v limited to [lo, hi]. */
static int8_t saturate(__int128 v, int32_t lo, int32_t hi)
{
    if (v < lo)
        return (int8_t)lo;
    if (v > hi)
        return (int8_t)hi;
    return (int8_t)v;
}

int orc_requant(int64_t acc, int32_t bias, int32_t mult, int32_t shift, int8_t *out)
{
    const int64_t x = acc + bias;
    if (x < INT32_MIN || x > INT32_MAX)
        return ORC_E_RANGE;
    if (shift < 1 || shift > 63 || mult < 0)
        return ORC_E_DOMAIN;
    *out = saturate(round_half_up_pow2((__int128)x * mult, shift), -128, 127);
    return ORC_OK;
}

/* The requantize over arrays of cases (test convenience: one call instead
 * of one per case); status is the OR of the cases' statuses. */
int orc_requant_many(const int64_t *acc, const int32_t *bias, const int32_t *mult,
                     const int32_t *shift, int8_t *out, int64_t n)
{
    int status = ORC_OK;
    for (int64_t i = 0; i < n; ++i)
        status |= orc_requant(acc[i], bias[i], mult[i], shift[i], &out[i]);
    return status;
}

/* ---- O2: plain dot products over K, int64 sums ---- */
static int64_t dot_s8_s8(const int8_t *a, const int8_t *b, int64_t K)
{
    int64_t acc = 0;
    for (int64_t k = 0; k < K; ++k)
        acc += (int64_t)a[k] * (int64_t)b[k];
    return acc;
}

static int64_t dot_s4_s4(const uint8_t *a, const uint8_t *b, int64_t K)
{
    int64_t acc = 0;
    for (int64_t k = 0; k < K; ++k)
        acc += (int64_t)orc_int4_at(a, k) * (int64_t)orc_int4_at(b, k);
    return acc;
}

static int64_t dot_s8_s4(const int8_t *a, const uint8_t *b, int64_t K)
{
    int64_t acc = 0;
    for (int64_t k = 0; k < K; ++k)
        acc += (int64_t)a[k] * (int64_t)orc_int4_at(b, k);
    return acc;
}

/* kinds of operand: 8 = int8 bytes, 4 = packed signed int4 (ld in nibbles) */
static int64_t dot_any(int ka, const void *A, int64_t lda, int64_t m,
                       int kb, const void *B, int64_t ldb, int64_t n, int64_t K)
{
    if (ka == 8 && kb == 8)
        return dot_s8_s8((const int8_t *)A + m * lda, (const int8_t *)B + n * ldb, K);
    if (ka == 4 && kb == 4)
        return dot_s4_s4((const uint8_t *)A + m * (lda / 2), (const uint8_t *)B + n * (ldb / 2), K);
    /* ka == 8 && kb == 4 */
    return dot_s8_s4((const int8_t *)A + m * lda, (const uint8_t *)B + n * (ldb / 2), K);
}

/*
 * Raw accumulators acc[r][n] = sum_k A[m_r][k] * B[n][k] as int64
 * ([INT4-GEMM] §3.2 with C zeroed first; [MCU-CONV] §3.2).
 * rows == NULL means rows 0..nrows-1.  out is [nrows][N].
 */
int orc_gemm_acc(int ka, const void *A, int64_t lda, int kb, const void *B, int64_t ldb,
                 int64_t N, int64_t K, const int64_t *rows, int64_t nrows, int64_t *out)
{
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t m = rows ? rows[r] : r;
        for (int64_t n = 0; n < N; ++n)
            out[r * N + n] = dot_any(ka, A, lda, m, kb, B, ldb, n, K);
    }
    return ORC_OK;
}

/* GEMM followed by the per-output-channel requantize; out is [nrows][ldc]. */
static int gemm_requant(int ka, const void *A, int64_t lda, int kb, const void *B, int64_t ldb,
                        const int32_t *bias, const int32_t *mult, const int32_t *shift,
                        int8_t *C, int64_t ldc, int64_t N, int64_t K,
                        const int64_t *rows, int64_t nrows)
{
    int status = ORC_OK;
    #pragma omp parallel for schedule(dynamic, 1) reduction(| : status)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t m = rows ? rows[r] : r;
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc = dot_any(ka, A, lda, m, kb, B, ldb, n, K);
            if (acc < INT32_MIN || acc > INT32_MAX)
                status |= ORC_E_RANGE;
            int8_t y = 0;
            status |= orc_requant(acc, bias ? bias[n] : 0, mult[n], shift[n], &y);
            C[r * ldc + n] = y;
        }
    }
    return status;
}

/* int8 x int8 -> int32 -> requantized int8 */
int orc_gemm_s8s8_requant(const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb,
                          const int32_t *bias, const int32_t *mult, const int32_t *shift,
                          int8_t *C, int64_t ldc, int64_t N, int64_t K,
                          const int64_t *rows, int64_t nrows)
{
    return gemm_requant(8, A, lda, 8, B, ldb, bias, mult, shift, C, ldc, N, K, rows, nrows);
}

/* int8 activations x packed int4 weights -> requantized int8 */
int orc_gemm_w4a8_requant(const int8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                          const int32_t *bias, const int32_t *mult, const int32_t *shift,
                          int8_t *C, int64_t ldc, int64_t N, int64_t K,
                          const int64_t *rows, int64_t nrows)
{
    return gemm_requant(8, A, lda, 4, B, ldb, bias, mult, shift, C, ldc, N, K, rows, nrows);
}

/* packed int4 x packed int4 -> raw int32 ([INT4-GEMM] §3.2) */
int orc_gemm_s4s4_i32(const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                      int32_t *C, int64_t ldc, int64_t N, int64_t K,
                      const int64_t *rows, int64_t nrows)
{
    int status = ORC_OK;
    #pragma omp parallel for schedule(dynamic, 1) reduction(| : status)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t m = rows ? rows[r] : r;
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc = dot_any(4, A, lda, m, 4, B, ldb, n, K);
            if (acc < INT32_MIN || acc > INT32_MAX)
                status |= ORC_E_RANGE;
            C[r * ldc + n] = (int32_t)acc;
        }
    }
    return status;
}

/* ---- O4/O5: NHWC conv geometry and MAC count ([MCU-CONV] §2.1) ---- */
int64_t orc_conv_out_size(int64_t in, int64_t k, int64_t stride, int64_t pad)
{
    int64_t span = in + 2 * pad - k;
    if (span < 0)
        return 0;
    return span / stride + 1;
}

/* MACs = out_w * out_h * out_c * in_c * k_w * k_h (per image), taps over
 * padding included, times the batch. */
int64_t orc_conv_macs(int64_t batch, int64_t H, int64_t W, int64_t C_in, int64_t C_out,
                      int64_t KH, int64_t KW, int64_t sh, int64_t sw, int64_t ph, int64_t pw)
{
    int64_t Ho = orc_conv_out_size(H, KH, sh, ph);
    int64_t Wo = orc_conv_out_size(W, KW, sw, pw);
    return batch * Ho * Wo * C_out * C_in * KH * KW;
}

/* Accumulator of one output element: the sum over taps and input channels,
 * with positions outside the image contributing the zero point 0. */
static int64_t conv_acc_at(const int8_t *X, const int8_t *Wt,
                           int64_t H, int64_t W, int64_t C_in,
                           int64_t KH, int64_t KW, int64_t sh, int64_t sw,
                           int64_t ph, int64_t pw,
                           int64_t b, int64_t oh, int64_t ow, int64_t oc)
{
    int64_t acc = 0;
    for (int64_t kh = 0; kh < KH; ++kh) {
        for (int64_t kw = 0; kw < KW; ++kw) {
            int64_t ih = oh * sh - ph + kh;
            int64_t iw = ow * sw - pw + kw;
            if (ih < 0 || ih >= H || iw < 0 || iw >= W)
                continue; /* padded tap: input value is the zero point 0 */
            for (int64_t ci = 0; ci < C_in; ++ci) {
                int64_t x = X[((b * H + ih) * W + iw) * C_in + ci];
                int64_t w = Wt[((oc * KH + kh) * KW + kw) * C_in + ci];
                acc += x * w;
            }
        }
    }
    return acc;
}

/* Raw conv accumulators for the selected output pixels; out is [npix][C_out].
 * Pixel index p = (b * H_out + oh) * W_out + ow.  pix == NULL means 0..npix-1. */
int orc_conv2d_acc(const int8_t *X, const int8_t *Wt,
                   int64_t batch, int64_t H, int64_t W, int64_t C_in, int64_t C_out,
                   int64_t KH, int64_t KW, int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                   const int64_t *pix, int64_t npix, int64_t *out)
{
    int64_t Ho = orc_conv_out_size(H, KH, sh, ph);
    int64_t Wo = orc_conv_out_size(W, KW, sw, pw);
    (void)batch;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < npix; ++r) {
        int64_t p = pix ? pix[r] : r;
        int64_t b = p / (Ho * Wo);
        int64_t oh = (p / Wo) % Ho;
        int64_t ow = p % Wo;
        for (int64_t oc = 0; oc < C_out; ++oc)
            out[r * C_out + oc] = conv_acc_at(X, Wt, H, W, C_in, KH, KW, sh, sw, ph, pw,
                                              b, oh, ow, oc);
    }
    return ORC_OK;
}

/* Conv followed by the per-output-channel requantize; Y is [npix][C_out]. */
int orc_conv2d_nhwc_s8_requant(const int8_t *X, const int8_t *Wt,
                               const int32_t *bias, const int32_t *mult, const int32_t *shift,
                               int8_t *Y,
                               int64_t batch, int64_t H, int64_t W, int64_t C_in, int64_t C_out,
                               int64_t KH, int64_t KW, int64_t sh, int64_t sw,
                               int64_t ph, int64_t pw,
                               const int64_t *pix, int64_t npix)
{
    int64_t Ho = orc_conv_out_size(H, KH, sh, ph);
    int64_t Wo = orc_conv_out_size(W, KW, sw, pw);
    int status = ORC_OK;
    (void)batch;
    #pragma omp parallel for schedule(dynamic, 16) reduction(| : status)
    for (int64_t r = 0; r < npix; ++r) {
        int64_t p = pix ? pix[r] : r;
        int64_t b = p / (Ho * Wo);
        int64_t oh = (p / Wo) % Ho;
        int64_t ow = p % Wo;
        for (int64_t oc = 0; oc < C_out; ++oc) {
            int64_t acc = conv_acc_at(X, Wt, H, W, C_in, KH, KW, sh, sw, ph, pw, b, oh, ow, oc);
            if (acc < INT32_MIN || acc > INT32_MAX)
                status |= ORC_E_RANGE;
            int8_t y = 0;
            status |= orc_requant(acc, bias ? bias[oc] : 0, mult[oc], shift[oc], &y);
            Y[r * C_out + oc] = y;
        }
    }
    return status;
}

/* ---- depthwise NHWC conv ([MCU-CONV] §3.3): every channel is convolved
 * on its own, input channel c feeding only output channel c; the weights are
 * [KH][KW][C], tap-major with the channels innermost, as that section's
 * per-channel kernel walks them; positions outside the image are the zero
 * point 0 ([MCU-CONV] §2.3). ---- */

/* MACs = out_w * out_h * C * k_w * k_h per image: the [MCU-CONV] §2.1
 * count with one input channel per output channel. */
int64_t orc_dwconv_macs(int64_t batch, int64_t H, int64_t W, int64_t C, int64_t KH, int64_t KW,
                        int64_t sh, int64_t sw, int64_t ph, int64_t pw)
{
    int64_t Ho = orc_conv_out_size(H, KH, sh, ph);
    int64_t Wo = orc_conv_out_size(W, KW, sw, pw);
    return batch * Ho * Wo * C * KH * KW;
}

static int64_t dwconv_acc_at(const int8_t *X, const int8_t *Wt,
                             int64_t H, int64_t W, int64_t C,
                             int64_t KH, int64_t KW, int64_t sh, int64_t sw,
                             int64_t ph, int64_t pw,
                             int64_t b, int64_t oh, int64_t ow, int64_t c)
{
    int64_t acc = 0;
    for (int64_t kh = 0; kh < KH; ++kh) {
        const int64_t ih = oh * sh + kh - ph;
        for (int64_t kw = 0; kw < KW; ++kw) {
            const int64_t iw = ow * sw + kw - pw;
            if (ih < 0 || ih >= H || iw < 0 || iw >= W)
                continue; /* padded tap: input value is the zero point 0 */
            const int64_t x = X[((b * H + ih) * W + iw) * C + c];
            const int64_t w = Wt[(kh * KW + kw) * C + c];
            acc += x * w;
        }
    }
    return acc;
}

/* Raw depthwise accumulators of the selected output pixels; out is
 * [npix][C].  Pixel index p = (b * H_out + oh) * W_out + ow; pix == NULL
 * means 0..npix-1. */
int orc_dwconv2d_acc(const int8_t *X, const int8_t *Wt,
                     int64_t batch, int64_t H, int64_t W, int64_t C,
                     int64_t KH, int64_t KW, int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                     const int64_t *pix, int64_t npix, int64_t *out)
{
    int64_t Ho = orc_conv_out_size(H, KH, sh, ph);
    int64_t Wo = orc_conv_out_size(W, KW, sw, pw);
    (void)batch;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < npix; ++r) {
        int64_t p = pix ? pix[r] : r;
        int64_t b = p / (Ho * Wo);
        int64_t oh = (p / Wo) % Ho;
        int64_t ow = p % Wo;
        for (int64_t c = 0; c < C; ++c)
            out[r * C + c] = dwconv_acc_at(X, Wt, H, W, C, KH, KW, sh, sw, ph, pw, b, oh, ow, c);
    }
    return ORC_OK;
}

/* Depthwise conv followed by the per-channel requantize; Y is [npix][C]. */
int orc_dwconv2d_nhwc_s8_requant(const int8_t *X, const int8_t *Wt,
                                 const int32_t *bias, const int32_t *mult,
                                 const int32_t *shift, int8_t *Y,
                                 int64_t batch, int64_t H, int64_t W, int64_t C,
                                 int64_t KH, int64_t KW, int64_t sh, int64_t sw,
                                 int64_t ph, int64_t pw, const int64_t *pix, int64_t npix)
{
    int64_t Ho = orc_conv_out_size(H, KH, sh, ph);
    int64_t Wo = orc_conv_out_size(W, KW, sw, pw);
    int status = ORC_OK;
    (void)batch;
    #pragma omp parallel for schedule(dynamic, 16) reduction(| : status)
    for (int64_t r = 0; r < npix; ++r) {
        int64_t p = pix ? pix[r] : r;
        int64_t b = p / (Ho * Wo);
        int64_t oh = (p / Wo) % Ho;
        int64_t ow = p % Wo;
        for (int64_t c = 0; c < C; ++c) {
            int64_t acc = dwconv_acc_at(X, Wt, H, W, C, KH, KW, sh, sw, ph, pw, b, oh, ow, c);
            int8_t y = 0;
            status |= orc_requant(acc, bias ? bias[c] : 0, mult[c], shift[c], &y);
            Y[r * C + c] = y;
        }
    }
    return status;
}

/* ---- asymmetric quantization.  [VOYAGER] §1.1: a code Q stands for the
 * real value (Q - zero_point) * scale.  [INT4-GEMM] §4.1: both GEMM operands
 * carry a zero point, and the product picks up a compensation term.
 * [MCU-CONV] §2.3: the padding of an asymmetric input is its zero point;
 * §3.3: the requantize adds the output zero point.  Zero points are per
 * tensor, in the int8 code range.  The product of two dequantized operands
 * is scale_a * scale_b * (A - za) * (B - zb), so the integer accumulator is
 * sum_k (A[m][k] - za) * (B[n][k] - zb), written out below term by term. ---- */

/* Q31 requantize with an output zero point and a fused activation: the
 * rounded value (as in orc_requant) plus out_zero, clamped to
 * [act_min, act_max] inside the int8 range.  [VOYAGER] §3.1 fuses the activation into the GEMM and requantize
 * (Conv -> DQ -> ReLU -> Q becomes one operator); on codes with zero point
 * out_zero, ReLU is the clamp at act_min = out_zero, and (-128, 127) is the
 * plain int8 saturation. */
int orc_requant_zp(int64_t acc, int32_t bias, int32_t mult, int32_t shift, int32_t out_zero,
                   int32_t act_min, int32_t act_max, int8_t *out)
{
    const int64_t x = acc + bias;
    if (x < INT32_MIN || x > INT32_MAX)
        return ORC_E_RANGE;
    if (shift < 1 || shift > 63 || mult < 0 || out_zero < -128 || out_zero > 127)
        return ORC_E_DOMAIN;
    if (act_min < -128 || act_max > 127 || act_min > act_max)
        return ORC_E_DOMAIN;
    const __int128 y = round_half_up_pow2((__int128)x * mult, shift);
    *out = saturate(y + out_zero, act_min, act_max);  /* zero point, then the clamp */
    return ORC_OK;
}

static int zero_point_ok(int32_t z)
{
    return z >= -128 && z <= 127;
}

static int64_t dot_s8_s8_zp(const int8_t *a, const int8_t *b, int64_t K, int64_t za, int64_t zb)
{
    int64_t acc = 0;
    for (int64_t k = 0; k < K; ++k)
        acc += ((int64_t)a[k] - za) * ((int64_t)b[k] - zb);
    return acc;
}

/* acc[r][n] = sum_k (A[m_r][k] - a_zero) * (B[n][k] - b_zero) as int64. */
int orc_gemm_s8s8_acc_zp(const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb,
                         int32_t a_zero, int32_t b_zero, int64_t N, int64_t K,
                         const int64_t *rows, int64_t nrows, int64_t *out)
{
    if (!zero_point_ok(a_zero) || !zero_point_ok(b_zero))
        return ORC_E_DOMAIN;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t m = rows ? rows[r] : r;
        for (int64_t n = 0; n < N; ++n)
            out[r * N + n] = dot_s8_s8_zp(A + m * lda, B + n * ldb, K, a_zero, b_zero);
    }
    return ORC_OK;
}

/* asymmetric int8 x int8 -> requantized int8 with an output zero point */
int orc_gemm_s8s8_requant_zp(const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb,
                             const int32_t *bias, const int32_t *mult, const int32_t *shift,
                             int32_t a_zero, int32_t b_zero, int32_t out_zero,
                             int32_t act_min, int32_t act_max,
                             int8_t *C, int64_t ldc, int64_t N, int64_t K,
                             const int64_t *rows, int64_t nrows)
{
    if (!zero_point_ok(a_zero) || !zero_point_ok(b_zero))
        return ORC_E_DOMAIN;
    int status = ORC_OK;
    #pragma omp parallel for schedule(dynamic, 1) reduction(| : status)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t m = rows ? rows[r] : r;
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc = dot_s8_s8_zp(A + m * lda, B + n * ldb, K, a_zero, b_zero);
            int8_t y = 0;
            status |= orc_requant_zp(acc, bias ? bias[n] : 0, mult[n], shift[n], out_zero,
                                     act_min, act_max, &y);
            C[r * ldc + n] = y;
        }
    }
    return status;
}

/* One output element of the asymmetric conv: positions outside the image
 * hold the input zero point, so they contribute (za - za) * (w - zb) = 0. */
static int64_t conv_acc_zp_at(const int8_t *X, const int8_t *Wt,
                              int64_t H, int64_t W, int64_t C_in,
                              int64_t KH, int64_t KW, int64_t sh, int64_t sw,
                              int64_t ph, int64_t pw, int64_t za, int64_t zb,
                              int64_t b, int64_t oh, int64_t ow, int64_t oc)
{
    const int8_t *wrow = Wt + oc * KH * KW * C_in;  /* OHWI row of channel oc */
    int64_t acc = 0;
    for (int64_t kh = 0; kh < KH; ++kh) {
        for (int64_t kw = 0; kw < KW; ++kw) {
            const int64_t y = kh + oh * sh - ph;
            const int64_t xx = kw + ow * sw - pw;
            const int inside = y >= 0 && y < H && xx >= 0 && xx < W;
            for (int64_t ci = 0; ci < C_in; ++ci) {
                int64_t x = inside ? X[((b * H + y) * W + xx) * C_in + ci] : za;
                int64_t w = wrow[(kh * KW + kw) * C_in + ci];
                acc += (x - za) * (w - zb);
            }
        }
    }
    return acc;
}

int orc_conv2d_acc_zp(const int8_t *X, const int8_t *Wt,
                      int64_t batch, int64_t H, int64_t W, int64_t C_in, int64_t C_out,
                      int64_t KH, int64_t KW, int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                      int32_t a_zero, int32_t b_zero,
                      const int64_t *pix, int64_t npix, int64_t *out)
{
    int64_t Ho = orc_conv_out_size(H, KH, sh, ph);
    int64_t Wo = orc_conv_out_size(W, KW, sw, pw);
    (void)batch;
    if (!zero_point_ok(a_zero) || !zero_point_ok(b_zero))
        return ORC_E_DOMAIN;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < npix; ++r) {
        int64_t p = pix ? pix[r] : r;
        int64_t b = p / (Ho * Wo);
        int64_t oh = (p / Wo) % Ho;
        int64_t ow = p % Wo;
        for (int64_t oc = 0; oc < C_out; ++oc)
            out[r * C_out + oc] = conv_acc_zp_at(X, Wt, H, W, C_in, KH, KW, sh, sw, ph, pw,
                                                 a_zero, b_zero, b, oh, ow, oc);
    }
    return ORC_OK;
}

int orc_conv2d_nhwc_s8_requant_zp(const int8_t *X, const int8_t *Wt,
                                  const int32_t *bias, const int32_t *mult,
                                  const int32_t *shift, int32_t a_zero, int32_t b_zero,
                                  int32_t out_zero, int32_t act_min, int32_t act_max, int8_t *Y,
                                  int64_t batch, int64_t H, int64_t W, int64_t C_in,
                                  int64_t C_out, int64_t KH, int64_t KW, int64_t sh,
                                  int64_t sw, int64_t ph, int64_t pw,
                                  const int64_t *pix, int64_t npix)
{
    int64_t Ho = orc_conv_out_size(H, KH, sh, ph);
    int64_t Wo = orc_conv_out_size(W, KW, sw, pw);
    int status = ORC_OK;
    (void)batch;
    if (!zero_point_ok(a_zero) || !zero_point_ok(b_zero))
        return ORC_E_DOMAIN;
    #pragma omp parallel for schedule(dynamic, 16) reduction(| : status)
    for (int64_t r = 0; r < npix; ++r) {
        int64_t p = pix ? pix[r] : r;
        int64_t b = p / (Ho * Wo);
        int64_t oh = (p / Wo) % Ho;
        int64_t ow = p % Wo;
        for (int64_t oc = 0; oc < C_out; ++oc) {
            int64_t acc = conv_acc_zp_at(X, Wt, H, W, C_in, KH, KW, sh, sw, ph, pw,
                                         a_zero, b_zero, b, oh, ow, oc);
            int8_t y = 0;
            status |= orc_requant_zp(acc, bias ? bias[oc] : 0, mult[oc], shift[oc], out_zero,
                                     act_min, act_max, &y);
            Y[r * C_out + oc] = y;
        }
    }
    return status;
}

/* The depthwise form: channel c alone, weights [kh][kw][c]. */
static int64_t dwconv_acc_zp_at(const int8_t *X, const int8_t *Wt,
                                int64_t H, int64_t W, int64_t C,
                                int64_t KH, int64_t KW, int64_t sh, int64_t sw,
                                int64_t ph, int64_t pw, int64_t za, int64_t zb,
                                int64_t b, int64_t oh, int64_t ow, int64_t c)
{
    int64_t acc = 0;
    for (int64_t t = 0; t < KH * KW; ++t) {      /* taps in [kh][kw] order */
        const int64_t kh = t / KW, kw = t % KW;
        const int64_t y = kh + oh * sh - ph;
        const int64_t xx = kw + ow * sw - pw;
        const int inside = y >= 0 && y < H && xx >= 0 && xx < W;
        const int64_t x = inside ? X[(((b * H) + y) * W + xx) * C + c] : za;
        const int64_t w = Wt[t * C + c];
        acc += (x - za) * (w - zb);
    }
    return acc;
}

int orc_dwconv2d_acc_zp(const int8_t *X, const int8_t *Wt,
                        int64_t batch, int64_t H, int64_t W, int64_t C,
                        int64_t KH, int64_t KW, int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                        int32_t a_zero, int32_t b_zero,
                        const int64_t *pix, int64_t npix, int64_t *out)
{
    int64_t Ho = orc_conv_out_size(H, KH, sh, ph);
    int64_t Wo = orc_conv_out_size(W, KW, sw, pw);
    (void)batch;
    if (!zero_point_ok(a_zero) || !zero_point_ok(b_zero))
        return ORC_E_DOMAIN;
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < npix; ++r) {
        int64_t p = pix ? pix[r] : r;
        int64_t b = p / (Ho * Wo);
        int64_t oh = (p / Wo) % Ho;
        int64_t ow = p % Wo;
        for (int64_t c = 0; c < C; ++c)
            out[r * C + c] = dwconv_acc_zp_at(X, Wt, H, W, C, KH, KW, sh, sw, ph, pw,
                                              a_zero, b_zero, b, oh, ow, c);
    }
    return ORC_OK;
}

int orc_dwconv2d_nhwc_s8_requant_zp(const int8_t *X, const int8_t *Wt,
                                    const int32_t *bias, const int32_t *mult,
                                    const int32_t *shift, int32_t a_zero, int32_t b_zero,
                                    int32_t out_zero, int32_t act_min, int32_t act_max,
                                    int8_t *Y,
                                    int64_t batch, int64_t H, int64_t W, int64_t C,
                                    int64_t KH, int64_t KW, int64_t sh, int64_t sw,
                                    int64_t ph, int64_t pw, const int64_t *pix, int64_t npix)
{
    int64_t Ho = orc_conv_out_size(H, KH, sh, ph);
    int64_t Wo = orc_conv_out_size(W, KW, sw, pw);
    int status = ORC_OK;
    (void)batch;
    if (!zero_point_ok(a_zero) || !zero_point_ok(b_zero))
        return ORC_E_DOMAIN;
    #pragma omp parallel for schedule(dynamic, 16) reduction(| : status)
    for (int64_t r = 0; r < npix; ++r) {
        int64_t p = pix ? pix[r] : r;
        int64_t b = p / (Ho * Wo);
        int64_t oh = (p / Wo) % Ho;
        int64_t ow = p % Wo;
        for (int64_t c = 0; c < C; ++c) {
            int64_t acc = dwconv_acc_zp_at(X, Wt, H, W, C, KH, KW, sh, sw, ph, pw,
                                           a_zero, b_zero, b, oh, ow, c);
            int8_t y = 0;
            status |= orc_requant_zp(acc, bias ? bias[c] : 0, mult[c], shift[c], out_zero,
                                     act_min, act_max, &y);
            Y[r * C + c] = y;
        }
    }
    return status;
}

/* ---- MSB-first INT4 packing ([INT4-GEMM] §3.2 names it as the order some
 * NPUs expect; the conversion script of its §4.1 packs the first element of
 * each pair into the high nibble): element 2i is the HIGH nibble of byte i,
 * element 2i+1 the low one; codes stay 4-bit two's complement. ---- */
int orc_int4_at_msb(const uint8_t *row, int64_t i)
{
    const int byte = row[i / 2];
    const int code = (i % 2 == 0) ? (byte >> 4) : (byte & 0x0F);
    return code >= 8 ? code - 16 : code;
}

/* packed int4 x packed int4 -> raw int32, both operands MSB-first */
int orc_gemm_s4s4_i32_msb(const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                          int32_t *C, int64_t ldc, int64_t N, int64_t K,
                          const int64_t *rows, int64_t nrows)
{
    int status = ORC_OK;
    #pragma omp parallel for schedule(dynamic, 1) reduction(| : status)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t m = rows ? rows[r] : r;
        const uint8_t *a = A + m * (lda / 2);
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t *b = B + n * (ldb / 2);
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)orc_int4_at_msb(a, k) * (int64_t)orc_int4_at_msb(b, k);
            if (acc < INT32_MIN || acc > INT32_MAX)
                status |= ORC_E_RANGE;
            C[r * ldc + n] = (int32_t)acc;
        }
    }
    return status;
}

/* int8 activations x MSB-first packed int4 weights -> requantized int8 */
int orc_gemm_w4a8_requant_msb(const int8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                              const int32_t *bias, const int32_t *mult, const int32_t *shift,
                              int8_t *C, int64_t ldc, int64_t N, int64_t K,
                              const int64_t *rows, int64_t nrows)
{
    int status = ORC_OK;
    #pragma omp parallel for schedule(dynamic, 1) reduction(| : status)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t m = rows ? rows[r] : r;
        const int8_t *a = A + m * lda;
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t *b = B + n * (ldb / 2);
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k)
                acc += (int64_t)a[k] * (int64_t)orc_int4_at_msb(b, k);
            if (acc < INT32_MIN || acc > INT32_MAX)
                status |= ORC_E_RANGE;
            int8_t y = 0;
            status |= orc_requant(acc, bias ? bias[n] : 0, mult[n], shift[n], &y);
            C[r * ldc + n] = y;
        }
    }
    return status;
}

/* ---- INT4 x INT4 with a binary16 output ([INT4-GEMM] §6: a variant of
 * the GEMM whose C is FP16, converted from the int32 accumulator).  The
 * accumulator goes to binary32 (exact: |acc| < 2^24 under the int4 K
 * bound), is multiplied by the optional per-row and per-column scales in
 * that order, each product rounded to binary32, and is rounded to binary16
 * to nearest, ties to even; magnitudes from 65520 up become infinities.
 * Without scales this is the page's plain conversion of the accumulator. ---- */

/* binary32 -> binary16, round to nearest, ties to even (bit patterns). */
uint16_t orc_f32_to_f16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a >= 0x7F800000u)                       /* infinity or NaN */
        return (uint16_t)(sign | (a > 0x7F800000u ? 0x7E00u : 0x7C00u));
    if (a >= 0x477FF000u)                       /* >= 65520: rounds past 65504 */
        return (uint16_t)(sign | 0x7C00u);
    const int e = (int)(a >> 23) - 127;         /* unbiased exponent */
    const uint32_t full = (a & 0x7FFFFFu) | 0x800000u;  /* 24-bit significand */
    int shift;                                  /* significand bits to drop */
    uint32_t base;                              /* exponent field of the result */
    if (e >= -14) {                             /* normal binary16 */
        shift = 13;
        base = (uint32_t)(e + 15) << 10;
    } else {                                    /* subnormal: units of 2^-24 */
        if (e < -25)
            return sign;                        /* below half the smallest step */
        shift = -e - 1;                         /* 14 .. 24 */
        base = 0;
    }
    uint32_t h = (full >> shift) & (e >= -14 ? 0x3FFu : 0xFFFFFFu);
    const uint32_t rem = full & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1);
    uint32_t r = base + h;
    if (rem > half || (rem == half && (r & 1u)))
        r += 1;                                 /* a carry moves into the exponent */
    return (uint16_t)(sign | r);
}

int orc_gemm_s4s4_f16(const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                      const float *scale_a, const float *scale_b, uint16_t *C, int64_t ldc,
                      int64_t N, int64_t K, const int64_t *rows, int64_t nrows)
{
    int status = ORC_OK;
    #pragma omp parallel for schedule(dynamic, 1) reduction(| : status)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t m = rows ? rows[r] : r;
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc = dot_any(4, A, lda, m, 4, B, ldb, n, K);
            if (acc <= -(1 << 24) || acc >= (1 << 24))
                status |= ORC_E_RANGE;
            float t = (float)acc;
            if (scale_a)
                t = t * scale_a[m];
            if (scale_b)
                t = t * scale_b[n];
            C[r * ldc + n] = orc_f32_to_f16(t);
        }
    }
    return status;
}

/* ---- per-token activation quantizer ([FLATQUANT] «per-token 模式»:
 * per token, scale = max|x| / (qmax / clip_ratio), codes = x / scale;
 * [VOYAGER] §1.1: Q = round(x / scale) + zero_point with round-half-away
 * rounding, zero point 0 here).  qmax is 7 for int4 (as the page states)
 * and 127 for int8.  The codes are decided in IEEE binary32, the precision
 * the GPU kernel computes in: the divisions are correctly rounded float
 * divisions, then the quotient is rounded half away from zero and clamped
 * to [-qmax, qmax].  A token whose values are all zero gets scale 0 and
 * codes 0.  Inputs must be finite. ---- */

/* binary16 / bfloat16 bit patterns to float (both convert exactly). */
float orc_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) << 31;
    int32_t e = (h >> 10) & 0x1F;
    uint32_t m = h & 0x3FF;
    float v;
    if (e == 0) {
        v = (float)m * (1.0f / 16777216.0f); /* m * 2^-24, exact */
    } else if (e == 31) {
        union { uint32_t u; float f; } inf = {0x7F800000u | (m << 13)};
        v = inf.f;
    } else {
        union { uint32_t u; float f; } x = {((uint32_t)(e - 15 + 127) << 23) | (m << 13)};
        v = x.f;
    }
    return sign ? -v : v;
}

float orc_bf16_to_f32(uint16_t b)
{
    union { uint32_t u; float f; } x = {(uint32_t)b << 16};
    return x.f;
}

/* round half away from zero of a binary32 value, as an integer */
static int64_t round_half_away(float q)
{
    float a = q < 0 ? -q : q;
    if (a >= 2147483648.0f)               /* clamps to +-qmax anyway; keeps the cast defined */
        a = 2147483648.0f;
    float f = (float)(int64_t)a;          /* floor of a */
    int64_t r = (int64_t)f + ((a - f) >= 0.5f ? 1 : 0);
    return q < 0 ? -r : r;
}

/* dtype: 0 = binary32, 1 = binary16, 2 = bfloat16; X is [M][ldx] elements.
 * bits 8: Q is int8 [M][ldq]; bits 4: Q is packed int4 [M][ldq/2 bytes]
 * (element 2i in the low nibble of byte i).  scale is [M]. */
int orc_quant_per_token(const void *X, int dtype, int64_t ldx, int64_t M, int64_t K,
                        float clip_ratio, int bits, void *Q, int64_t ldq, float *scale)
{
    const float qmax = bits == 4 ? 7.0f : 127.0f;
    if ((bits != 4 && bits != 8) || !(clip_ratio > 0.0f))
        return ORC_E_DOMAIN;
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = dtype == 0 ? ((const float *)X)[m * ldx + k]
                    : dtype == 1 ? orc_f16_to_f32(((const uint16_t *)X)[m * ldx + k])
                                 : orc_bf16_to_f32(((const uint16_t *)X)[m * ldx + k]);
            float a = v < 0 ? -v : v;
            if (a > amax)
                amax = a;
        }
        const float sc = amax / (qmax / clip_ratio);
        scale[m] = sc;
        for (int64_t k = 0; k < K; ++k) {
            int64_t q = 0;
            if (sc > 0.0f) {
                float v = dtype == 0 ? ((const float *)X)[m * ldx + k]
                        : dtype == 1 ? orc_f16_to_f32(((const uint16_t *)X)[m * ldx + k])
                                     : orc_bf16_to_f32(((const uint16_t *)X)[m * ldx + k]);
                q = round_half_away(v / sc);
                if (q > (int64_t)qmax)
                    q = (int64_t)qmax;
                if (q < -(int64_t)qmax)
                    q = -(int64_t)qmax;
            }
            if (bits == 8) {
                ((int8_t *)Q)[m * ldq + k] = (int8_t)q;
            } else {
                uint8_t *byte = (uint8_t *)Q + m * (ldq / 2) + k / 2;
                uint8_t nib = (uint8_t)(q & 0xF);
                if (k % 2 == 0)
                    *byte = (uint8_t)((*byte & 0xF0) | nib);
                else
                    *byte = (uint8_t)((*byte & 0x0F) | (nib << 4));
            }
        }
    }
    return ORC_OK;
}

/* ---- threading controls, so a caller can state the cores it used ---- */
void orc_set_threads(int n)
{
    if (n > 0)
        omp_set_num_threads(n);
}

int orc_max_threads(void)
{
    return omp_get_max_threads();
}
