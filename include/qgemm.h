/*
 * qgemm.h -- C ABI of the MI355X (gfx950) quantized GEMM / conv library.
 *
 * The computation: low-bit integer matrix products with INT32 accumulation,
 * and a fused per-output-channel fixed-point requantize back to INT8.
 *
 * Definitions followed (web pages; section numbers are the pages' own):
 *   - INT4 operands are signed 4-bit two's complement, two per byte
 *     ("DeepGEMM" INT4 GEMM article, www.cf-1.com/news/6060138, §2.1).
 *     Element 2i is the LOW nibble of byte i, element 2i+1 the high nibble.
 *   - C = A * B with INT4 or INT8 inputs and INT32 accumulation (same
 *     article, §3.2); B is stored column-major, i.e. as [N][K] with K
 *     contiguous (same article, §4.3).
 *   - Requantize (MCU conv front-end article, news.rkmt.cn/news/16638,
 *     §2.3, with the bias of §3.3):
 *         x = acc + bias[n]                       (int32)
 *         t = x * mult[n]                         (int64)
 *         t = t + 2^(shift[n] - 1)                (half an LSB)
 *         y = t >> shift[n]                       (arithmetic shift)
 *         out = min(127, max(-128, y))            (int8)
 *     Symmetric quantization: zero point 0, so there is no zero-point
 *     argument and conv padding reads 0 (same article, §2.3).
 *   - Conv: NHWC activations, OHWI weights [C_out][KH][KW][C_in] (same
 *     article, §3.1), computed as an implicit GEMM over the im2col matrix
 *     of §3.2 with K index (kh * KW + kw) * C_in + ci; output size
 *     floor((H + 2*pad - KH) / stride) + 1 (same article, §2.1).
 *
 * Conventions shared by every entry point:
 *   - Every pointer is DEVICE memory owned by the caller.  The library never
 *     allocates, frees or synchronizes.  It keeps no mutable state, except
 *     the per-GPU scratch array of qgemm_s8s8_requant_zp_noalloc.
 *   - stream: a hipStream_t (NULL = default stream).  A call validates its
 *     arguments on the host, enqueues its kernels on `stream` and returns;
 *     the result is ready when the stream reaches that point.  A fault in a
 *     kernel surfaces at the caller's next synchronization.
 *   - Leading dimensions are in ELEMENTS.  For packed int4 operands they
 *     count nibbles and must be even; the byte stride is ld / 2.
 *   - Alignment: every base pointer must be 16-byte aligned, and the row
 *     strides of the operands (lda, ldb in bytes) multiples of 16 bytes.
 *     The output row stride ldc may be any value >= N; when ldc is a
 *     multiple of 4 the kernels store four results per instruction.
 *   - Outputs must not overlap inputs.
 *   - Results are deterministic: integer sums are exact, so repeated calls
 *     give identical bytes.
 *   - Device-resident preconditions, not checked by the library:
 *     shift[n] in [1, 63]; mult[n] in [0, 2^31 - 1]; acc + bias[n] fits in
 *     int32.  Outside them the output bytes are unspecified (no fault).
 *
 * Status codes (checked in this order; every argument check happens on the
 * host before any HIP call, so it is testable without a GPU):
 *   QG_ERR_NULLPTR   a required pointer is NULL (bias may be NULL = zero)
 *   QG_ERR_INVALID   a size, stride or alignment rule is broken
 *   QG_ERR_NO_DEVICE no HIP device is current, or it is not gfx950
 *   QG_ERR_LAUNCH    the kernel launch reported an error
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QG_OK = 0,
    QG_ERR_NULLPTR = 1,
    QG_ERR_INVALID = 2,
    QG_ERR_NO_DEVICE = 3,
    QG_ERR_LAUNCH = 4
} qg_status;

/* Largest K accepted by the int4 entry points.  The library computes on
 * 16x-scaled nibbles; this bound keeps the scaled int32 sums exact:
 * s4s4: 256 * 64 * K < 2^31;  w4a8: 16 * 128 * 8 * K < 2^31 (|a| <= 128). */
#define QG_S4S4_MAX_K 131040
#define QG_W4A8_MAX_K 131040

/* Input element types of qquant_per_token. */
#define QG_DT_F32 0
#define QG_DT_F16 1
#define QG_DT_BF16 2

/*
 * qgemm_s8s8_requant -- C[m][n] = requant(sum_k A[m][k] * B[n][k]).
 *   A     int8  [M][lda], row-major, lda >= K
 *   B     int8  [N][ldb] (column-major K x N), ldb >= K
 *   bias  int32 [N] or NULL;  mult int32 [N] (Q31);  shift int32 [N]
 *   C     int8  [M][ldc], ldc >= N
 *   M, N, K >= 1; K % 16 == 0 (16-byte rows); lda, ldb % 16 == 0.
 * MCU conv front-end article §2.3 (requantize), §3.2 (C = A x B);
 * INT4 GEMM article §4.3 (B column-major).
 */
qg_status qgemm_s8s8_requant(const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb,
                             const int32_t *bias, const int32_t *mult, const int32_t *shift,
                             int8_t *C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                             void *stream);

/*
 * qgemm_s4s4_i32 -- C[m][n] = sum_k A[m][k] * B[n][k], raw int32, no requant.
 *   A     packed int4 [M][lda/2 bytes], lda >= K (nibbles)
 *   B     packed int4 [N][ldb/2 bytes], ldb >= K
 *   C     int32 [M][ldc], ldc >= N
 *   M, N >= 1; K >= 1, K % 32 == 0 (16-byte packed rows), K <= QG_S4S4_MAX_K;
 *   lda, ldb % 32 == 0 (nibbles).
 * INT4 GEMM article §2.1 (packing), §3.2 (C = A*B into a zeroed C).
 */
qg_status qgemm_s4s4_i32(const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                         int32_t *C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                         void *stream);

/*
 * qgemm_s4s4_f16 -- packed int4 x packed int4 with a binary16 output:
 *   C[m][n] = fp16(fp32(acc) * scale_a[m] * scale_b[n]),
 *   acc = sum_k A[m][k] * B[n][k] (exact in binary32 under the K bound), the
 *   products taken in that order, each rounded to binary32, the result
 *   rounded to binary16 to nearest, ties to even (65520 and up become
 *   infinities).  scale_a [M] and scale_b [N] are optional (NULL = 1): with
 *   neither, C is the accumulator converted to FP16, as the INT4 GEMM
 *   article's §6 variant does; with them, C is the dequantized product
 *   (per-token activation scales, per-channel weight scales).
 *   C     binary16 bit patterns [M][ldc], ldc >= N
 *   A, B, lda, ldb, M, N, K as for qgemm_s4s4_i32; scale_a / scale_b
 *   16-byte aligned when given.
 */
qg_status qgemm_s4s4_f16(const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                         const float *scale_a, const float *scale_b, uint16_t *C, int64_t ldc,
                         int64_t M, int64_t N, int64_t K, void *stream);

/*
 * qgemm_w4a8_requant -- int8 activations x packed int4 weights, requantized.
 *   A     int8  [M][lda], lda >= K
 *   B     packed int4 [N][ldb/2 bytes], ldb >= K (nibbles)
 *   bias/mult/shift as for qgemm_s8s8_requant
 *   C     int8  [M][ldc], ldc >= N
 *   M, N >= 1; K % 32 == 0, K <= QG_W4A8_MAX_K; lda % 16 == 0, ldb % 32 == 0.
 * Small M (a few tokens) runs a weight-streaming kernel; larger M runs the
 * tiled kernel.  Same definitions as above.
 */
qg_status qgemm_w4a8_requant(const int8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                             const int32_t *bias, const int32_t *mult, const int32_t *shift,
                             int8_t *C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                             void *stream);

/*
 * qgemm_w4a8_requant_msb -- qgemm_w4a8_requant with the int4 weights packed
 * high nibble first: element 2i of a row in the high nibble of byte i, 2i+1
 * in the low one (INT4 GEMM article §3.2 names this order as the one some
 * NPUs use; its §4.1 conversion script packs that way).  Same arguments and
 * rules as qgemm_w4a8_requant.  (qgemm_s4s4_i32 needs no such variant: with
 * both operands in the same order the sum over K is the same either way.)
 */
qg_status qgemm_w4a8_requant_msb(const int8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                                 const int32_t *bias, const int32_t *mult,
                                 const int32_t *shift, int8_t *C, int64_t ldc, int64_t M,
                                 int64_t N, int64_t K, void *stream);

/*
 * qconv2d_nhwc_s8_requant -- int8 NHWC conv, zero-point-0 padding, requant.
 *   X     int8 [batch][H][Wd][C_in]  (NHWC, dense)
 *   W     int8 [C_out][KH][KW][C_in] (OHWI, dense)
 *   bias/mult/shift int32 [C_out] (bias may be NULL)
 *   Y     int8 [batch][H_out][W_out][C_out] (NHWC, dense)
 *   H_out = (H + 2*pad_h - KH) / stride_h + 1, W_out likewise; both >= 1.
 *   batch, H, Wd, KH, KW, stride >= 1; pad >= 0; C_in % 16 == 0 and
 *   C_out % 16 == 0 (pad channels with zeros, as the MCU article's §3.1
 *   pads input channels); dilation 1, one group.
 * MCU conv front-end article §2.1, §2.3, §3.1, §3.2; 3x3 taps walked as
 * shifted 1x1 products (Groq TSP ResNet50 article, www.pwwt.cn/news/1982903,
 * §2.1).
 */
qg_status qconv2d_nhwc_s8_requant(const int8_t *X, const int8_t *W,
                                  const int32_t *bias, const int32_t *mult,
                                  const int32_t *shift, int8_t *Y,
                                  int32_t batch, int32_t H, int32_t Wd, int32_t C_in,
                                  int32_t C_out, int32_t KH, int32_t KW,
                                  int32_t stride_h, int32_t stride_w,
                                  int32_t pad_h, int32_t pad_w, void *stream);

/*
 * qdwconv2d_nhwc_s8_requant -- depthwise int8 NHWC conv, zero-point-0
 * padding, requant: output channel c is the conv of input channel c alone.
 *   X     int8 [batch][H][Wd][C]  (NHWC, dense)
 *   W     int8 [KH][KW][C]        (tap-major, channels innermost, dense)
 *   bias/mult/shift int32 [C] (bias may be NULL)
 *   Y     int8 [batch][H_out][W_out][C] (NHWC, dense)
 *   H_out, W_out as for qconv2d_nhwc_s8_requant; both >= 1.
 *   batch, H, Wd, C, KH, KW, stride >= 1; pad >= 0; C % 16 == 0.
 * MCU conv front-end article §3.3 (one input channel per output channel,
 * weights indexed [kh][kw][c], border filled with the zero point), §2.3
 * (requantize).  3x3 with equal strides 1 or 2 runs on the int8 matrix
 * cores; other shapes run a direct kernel.
 */
qg_status qdwconv2d_nhwc_s8_requant(const int8_t *X, const int8_t *W,
                                    const int32_t *bias, const int32_t *mult,
                                    const int32_t *shift, int8_t *Y,
                                    int32_t batch, int32_t H, int32_t Wd, int32_t C,
                                    int32_t KH, int32_t KW, int32_t stride_h, int32_t stride_w,
                                    int32_t pad_h, int32_t pad_w, void *stream);

/*
 * qquant_per_token -- symmetric per-token quantization of float activations.
 *   X      [M][ldx] elements of dtype: QG_DT_F32 (binary32), QG_DT_F16
 *          (binary16) or QG_DT_BF16 (bfloat16); finite values
 *   Q      bits 8: int8 [M][ldq]; bits 4: packed int4 [M][ldq/2 bytes],
 *          element 2i in the low nibble of byte i
 *   scale  float32 [M], written: scale[m] = max_k |X[m][k]| / (qmax / clip)
 *   qmax = 127 (bits 8) or 7 (bits 4); Q[m][k] = X[m][k] / scale[m] in
 *   binary32, rounded half away from zero and clamped to [-qmax, qmax];
 *   a token of zeros gets scale 0 and codes 0.  All arithmetic is IEEE
 *   binary32 (half inputs are widened exactly first).
 *   M >= 1; 16 <= K, K % 16 == 0; ldx >= K with ldx % 8 == 0 (ldx % 4 == 0
 *   for binary32); ldq >= K, ldq % 16 == 0; 0 < clip <= 1; X, Q 16-byte
 *   aligned, scale 4-byte aligned.
 * Ascend FlatQuant operator article (www.zwxr.cn/news/277566), per-token
 * mode (the scale, clip_ratio, int4 range); Voyager quantization article
 * (www.dpshk.com/news/2695434) §1.1 (round half away from zero, zero point
 * 0); INT4 GEMM article §2.1 (nibble order).  The codes feed the A operand
 * of the GEMMs above.
 */
qg_status qquant_per_token(const void *X, int32_t dtype, int64_t ldx, void *Q, int64_t ldq,
                           float *scale, int64_t M, int64_t K, float clip, int32_t bits,
                           void *stream);

/*
 * Asymmetric (zero-point) forms with a fused activation clamp.  A code Q
 * stands for (Q - zero_point) * scale (Voyager quantization article,
 * www.dpshk.com/news/2695434, §1.1), so with per-tensor zero points a_zero
 * (activations), b_zero (weights) and out_zero (output), all in [-128, 127]:
 *   acc = sum_k (A[m][k] - a_zero) * (B[n][k] - b_zero)        (GEMM)
 *   acc = sum over taps and input channels of (X - a_zero) * (W - b_zero),
 *         positions outside the image holding a_zero             (convs)
 *   out = (((acc + bias) * mult + 2^(shift-1)) >> shift) + out_zero,
 *         saturated to [act_min, act_max] (the zero point added first)
 * with -128 <= act_min <= act_max <= 127: (-128, 127) is the plain int8
 * saturation and (out_zero, 127) a fused ReLU (the Voyager article's §3.1
 * fuses GEMM + bias + activation into one operator).
 * (INT4 GEMM article §4.1 for zero points on both operands; MCU conv
 * front-end article §2.3 for padding with the input zero point and §3.3 for
 * the output zero point.)  Layouts, strides, alignment and the other
 * requirements are those of the symmetric call of the same name.
 * Precondition: acc + bias fits in int32.
 *
 * Each call takes a caller-owned device workspace of at least the bytes its
 * *_workspace_size function returns for the same shape (16-byte aligned);
 * the library writes per-row / per-column compensation sums there on the
 * call's stream, ahead of the main kernel, and keeps nothing between calls.
 * Calls that share a workspace must be ordered (one stream).  The size
 * functions return 0 for shapes the call rejects.  Errors as above;
 * QG_ERR_NULLPTR for a NULL workspace, QG_ERR_INVALID for a zero point or
 * clamp bound out of range or a workspace that is too small or misaligned.
 */
size_t qgemm_s8s8_requant_zp_workspace_size(int64_t M, int64_t N);
qg_status qgemm_s8s8_requant_zp(const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb,
                                const int32_t *bias, const int32_t *mult, const int32_t *shift,
                                int32_t a_zero, int32_t b_zero, int32_t out_zero,
                                int32_t act_min, int32_t act_max, int8_t *C, int64_t ldc,
                                int64_t M, int64_t N, int64_t K, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * qgemm_s8s8_requant_zp_noalloc -- qgemm_s8s8_requant_zp without a
 * workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments (less workspace / workspace_bytes), result
 * and errors as qgemm_s8s8_requant_zp.  The compensation sums live in a
 * 1 MiB array inside the library, one per GPU, held until the process ends:
 * the call allocates nothing, and returns QG_ERR_INVALID when
 * 4 * (ceil(M / 64) + ceil(N / 64)) * 64 > 1048576 (about M + N <= 262,000).
 * Every call on one GPU shares that array: calls that may overlap on the
 * same GPU (other streams, other host threads) race and must be ordered by
 * the caller.  QG_ERR_LAUNCH also covers a failure to find the array's
 * address on the current device.
 */
qg_status qgemm_s8s8_requant_zp_noalloc(const int8_t *A, int64_t lda, const int8_t *B,
                                        int64_t ldb, const int32_t *bias, const int32_t *mult,
                                        const int32_t *shift, int32_t a_zero, int32_t b_zero,
                                        int32_t out_zero, int32_t act_min, int32_t act_max,
                                        int8_t *C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                        void *stream);

size_t qconv2d_nhwc_s8_requant_zp_workspace_size(int32_t batch, int32_t H, int32_t Wd,
                                                 int32_t C_out, int32_t KH, int32_t KW,
                                                 int32_t stride_h, int32_t stride_w,
                                                 int32_t pad_h, int32_t pad_w);
qg_status qconv2d_nhwc_s8_requant_zp(const int8_t *X, const int8_t *W, const int32_t *bias,
                                     const int32_t *mult, const int32_t *shift, int32_t a_zero,
                                     int32_t b_zero, int32_t out_zero, int32_t act_min,
                                     int32_t act_max, int8_t *Y, int32_t batch,
                                     int32_t H, int32_t Wd, int32_t C_in, int32_t C_out,
                                     int32_t KH, int32_t KW, int32_t stride_h, int32_t stride_w,
                                     int32_t pad_h, int32_t pad_w, void *workspace,
                                     size_t workspace_bytes, void *stream);

size_t qdwconv2d_nhwc_s8_requant_zp_workspace_size(int32_t C);
qg_status qdwconv2d_nhwc_s8_requant_zp(const int8_t *X, const int8_t *W, const int32_t *bias,
                                       const int32_t *mult, const int32_t *shift,
                                       int32_t a_zero, int32_t b_zero, int32_t out_zero,
                                       int32_t act_min, int32_t act_max,
                                       int8_t *Y, int32_t batch, int32_t H, int32_t Wd,
                                       int32_t C, int32_t KH, int32_t KW, int32_t stride_h,
                                       int32_t stride_w, int32_t pad_h, int32_t pad_w,
                                       void *workspace, size_t workspace_bytes, void *stream);

/* Human-readable name of a status code (static string, never NULL). */
const char *qg_status_string(qg_status s);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int qg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
