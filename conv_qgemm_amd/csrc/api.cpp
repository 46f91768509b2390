// api.cpp -- the C ABI of libqgemm (declared in include/qgemm.h).
//
// Each entry point (1) checks every argument on the host, before any HIP
// call, (2) checks that the current device is a gfx950, (3) launches its
// kernels on the caller's stream and returns without synchronizing.
// Status codes and the validate-then-execute split follow the convention of
// the aclnnFlatQuantV2 guide (www.zwxr.cn/news/277566, its error-code and
// two-phase-call sections); no workspace is needed, so the two phases are
// one call.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "../../include/qgemm.h"
#include "launch.hpp"

namespace {

constexpr int kMaxDevices = 64;
constexpr int64_t kMaxDim = (int64_t)1 << 30;
constexpr int64_t kMaxGrid = (int64_t)1 << 24;
// per-device facts, filled once: architecture verdict (0 unknown, 1 gfx950,
// 2 other) and compute-unit count
std::atomic<int> g_arch_ok[kMaxDevices];
std::atomic<int> g_cus[kMaxDevices];

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

qg_status check_device(int *cus)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return QG_ERR_NO_DEVICE;
    int v = g_arch_ok[dev].load(std::memory_order_acquire);
    if (v == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return QG_ERR_NO_DEVICE;
        v = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_cus[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1,
                         std::memory_order_relaxed);
        g_arch_ok[dev].store(v, std::memory_order_release);
    }
    *cus = g_cus[dev].load(std::memory_order_relaxed);
    return v == 1 ? QG_OK : QG_ERR_NO_DEVICE;
}

qg_status launched(hipError_t e) { return e == hipSuccess ? QG_OK : QG_ERR_LAUNCH; }

// Shared GEMM checks.  a_nib/b_nib: operand is packed int4 (ld in nibbles).
// c_bytes: size of one C element.
qg_status check_gemm(const void *A, int64_t lda, bool a_nib, const void *B, int64_t ldb,
                     bool b_nib, const void *C, int64_t ldc, int c_bytes, int64_t M, int64_t N,
                     int64_t K, int64_t max_k)
{
    if (M < 1 || N < 1 || K < 1)
        return QG_ERR_INVALID;
    // rows, columns and K are int32 inside the kernels, with headroom for a
    // tile past the end; the grid must stay under 2^24 workgroups
    if (M > kMaxDim || N > kMaxDim || K > max_k)
        return QG_ERR_INVALID;
    if (((M + 63) / 64) * ((N + 63) / 64) >= kMaxGrid)
        return QG_ERR_INVALID;
    // a packed row must be whole 16-byte chunks: K % 32 (int4) or K % 16 (int8)
    const int64_t kmul = (a_nib || b_nib) ? 32 : 16;
    if (K % kmul != 0)
        return QG_ERR_INVALID;
    if (lda < K || ldb < K || ldc < N)
        return QG_ERR_INVALID;
    if ((a_nib ? lda % 32 : lda % 16) != 0 || (b_nib ? ldb % 32 : ldb % 16) != 0)
        return QG_ERR_INVALID;
    if (!aligned16(A) || !aligned16(B) || !aligned16(C))
        return QG_ERR_INVALID;
    // every byte offset the kernels form fits in int64
    if (lda > INT64_MAX / M || ldb > INT64_MAX / N || ldc > INT64_MAX / M / c_bytes)
        return QG_ERR_INVALID;
    return QG_OK;
}

qg_status check_params(const int32_t *bias, const int32_t *mult, const int32_t *shift)
{
    if (!aligned16(mult) || !aligned16(shift) || (bias && !aligned16(bias)))
        return QG_ERR_INVALID;
    return QG_OK;
}

// Conv checks shared by the symmetric and asymmetric entry points; returns
// the output size.
qg_status check_conv(const int8_t *X, const int8_t *W, const int8_t *Y, int32_t batch, int32_t H,
                     int32_t Wd, int32_t C_in, int32_t C_out, int32_t KH, int32_t KW,
                     int32_t stride_h, int32_t stride_w, int32_t pad_h, int32_t pad_w,
                     int64_t *Ho_out, int64_t *Wo_out)
{
    if (batch < 1 || H < 1 || Wd < 1 || C_in < 1 || C_out < 1 || KH < 1 || KW < 1 ||
        stride_h < 1 || stride_w < 1 || pad_h < 0 || pad_w < 0)
        return QG_ERR_INVALID;
    if (C_in % 16 != 0 || C_out % 16 != 0)
        return QG_ERR_INVALID;
    const int64_t span_h = (int64_t)H + 2 * (int64_t)pad_h - KH;
    const int64_t span_w = (int64_t)Wd + 2 * (int64_t)pad_w - KW;
    if (span_h < 0 || span_w < 0)
        return QG_ERR_INVALID;
    const int64_t Ho = span_h / stride_h + 1, Wo = span_w / stride_w + 1;
    // kernel indices are int32: pixels, K and element offsets must fit
    const int64_t pixels = (int64_t)batch * Ho * Wo;
    const int64_t K = (int64_t)KH * KW * C_in;
    if (pixels > kMaxDim || K > kMaxDim || (int64_t)batch * H > kMaxDim ||
        ((pixels + 63) / 64) * ((C_out + 63) / 64) >= kMaxGrid)
        return QG_ERR_INVALID;
    if (!aligned16(X) || !aligned16(W) || !aligned16(Y))
        return QG_ERR_INVALID;
    *Ho_out = Ho;
    *Wo_out = Wo;
    return QG_OK;
}

qg_status check_dwconv(const int8_t *X, const int8_t *W, const int8_t *Y, int32_t batch,
                       int32_t H, int32_t Wd, int32_t C, int32_t KH, int32_t KW,
                       int32_t stride_h, int32_t stride_w, int32_t pad_h, int32_t pad_w,
                       int64_t *Ho_out, int64_t *Wo_out)
{
    if (batch < 1 || H < 1 || Wd < 1 || C < 1 || KH < 1 || KW < 1 || stride_h < 1 ||
        stride_w < 1 || pad_h < 0 || pad_w < 0)
        return QG_ERR_INVALID;
    if (C % 16 != 0)
        return QG_ERR_INVALID;
    const int64_t span_h = (int64_t)H + 2 * (int64_t)pad_h - KH;
    const int64_t span_w = (int64_t)Wd + 2 * (int64_t)pad_w - KW;
    if (span_h < 0 || span_w < 0)
        return QG_ERR_INVALID;
    const int64_t Ho = span_h / stride_h + 1, Wo = span_w / stride_w + 1;
    // kernel indices are int32 where they count pixels, rows or LDS bytes;
    // element offsets are computed in 64 bits
    const int64_t pixels = (int64_t)batch * Ho * Wo;
    if (pixels > kMaxDim || (int64_t)batch * H * Wd > kMaxDim || C > 65536 ||
        (int64_t)KH * KW * C > kMaxDim || (pixels * (C / 4) + 255) / 256 >= kMaxGrid)
        return QG_ERR_INVALID;
    if (!aligned16(X) || !aligned16(W) || !aligned16(Y))
        return QG_ERR_INVALID;
    *Ho_out = Ho;
    *Wo_out = Wo;
    return QG_OK;
}

bool zero_point_ok(int32_t z) { return z >= -128 && z <= 127; }

bool act_ok(int32_t lo, int32_t hi) { return -128 <= lo && lo <= hi && hi <= 127; }

// a workspace of at least `need` bytes, 16-byte aligned
qg_status check_workspace(const void *ws, size_t bytes, int64_t need)
{
    if (!ws)
        return QG_ERR_NULLPTR;
    if ((int64_t)bytes < need || !aligned16(ws))
        return QG_ERR_INVALID;
    return QG_OK;
}

}  // namespace

extern "C" {

qg_status qgemm_s8s8_requant(const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb,
                             const int32_t *bias, const int32_t *mult, const int32_t *shift,
                             int8_t *C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                             void *stream)
{
    if (!A || !B || !C || !mult || !shift)
        return QG_ERR_NULLPTR;
    qg_status st = check_gemm(A, lda, false, B, ldb, false, C, ldc, 1, M, N, K, kMaxDim);
    if (st == QG_OK)
        st = check_params(bias, mult, shift);
    if (st != QG_OK)
        return st;
    int cus = 0;
    if ((st = check_device(&cus)) != QG_OK)
        return st;
    qg::GemmDesc d{A, lda, B, ldb, bias, mult, shift, C, ldc, M, N, K, cus};
    return launched(qg::launch_s8s8_requant(d, (hipStream_t)stream));
}

qg_status qgemm_s4s4_i32(const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                         int32_t *C, int64_t ldc, int64_t M, int64_t N, int64_t K, void *stream)
{
    if (!A || !B || !C)
        return QG_ERR_NULLPTR;
    qg_status st = check_gemm(A, lda, true, B, ldb, true, C, ldc, 4, M, N, K, QG_S4S4_MAX_K);
    if (st != QG_OK)
        return st;
    int cus = 0;
    if ((st = check_device(&cus)) != QG_OK)
        return st;
    qg::GemmDesc d{A, lda / 2, B, ldb / 2, nullptr, nullptr, nullptr, C, ldc, M, N, K, cus};
    return launched(qg::launch_s4s4_i32(d, (hipStream_t)stream));
}

qg_status qgemm_s4s4_f16(const uint8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                         const float *scale_a, const float *scale_b, uint16_t *C, int64_t ldc,
                         int64_t M, int64_t N, int64_t K, void *stream)
{
    if (!A || !B || !C)
        return QG_ERR_NULLPTR;
    qg_status st = check_gemm(A, lda, true, B, ldb, true, C, ldc, 2, M, N, K, QG_S4S4_MAX_K);
    if (st != QG_OK)
        return st;
    if ((scale_a && !aligned16(scale_a)) || (scale_b && !aligned16(scale_b)))
        return QG_ERR_INVALID;
    int cus = 0;
    if ((st = check_device(&cus)) != QG_OK)
        return st;
    qg::GemmDesc d{A, lda / 2, B, ldb / 2, nullptr, nullptr, nullptr, C, ldc, M, N, K, cus,
                   nullptr, 0, false, 0, 0, scale_a, scale_b};
    return launched(qg::launch_s4s4_f16(d, (hipStream_t)stream));
}

qg_status qgemm_w4a8_requant(const int8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                             const int32_t *bias, const int32_t *mult, const int32_t *shift,
                             int8_t *C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                             void *stream)
{
    if (!A || !B || !C || !mult || !shift)
        return QG_ERR_NULLPTR;
    qg_status st = check_gemm(A, lda, false, B, ldb, true, C, ldc, 1, M, N, K, QG_W4A8_MAX_K);
    if (st == QG_OK)
        st = check_params(bias, mult, shift);
    if (st != QG_OK)
        return st;
    int cus = 0;
    if ((st = check_device(&cus)) != QG_OK)
        return st;
    qg::GemmDesc d{A, lda, B, ldb / 2, bias, mult, shift, C, ldc, M, N, K, cus};
    if (M <= qg::kSkinnyMaxM)
        return launched(qg::launch_w4a8_skinny(d, (hipStream_t)stream));
    return launched(qg::launch_w4a8_tiled(d, (hipStream_t)stream));
}

qg_status qgemm_w4a8_requant_msb(const int8_t *A, int64_t lda, const uint8_t *B, int64_t ldb,
                                 const int32_t *bias, const int32_t *mult,
                                 const int32_t *shift, int8_t *C, int64_t ldc, int64_t M,
                                 int64_t N, int64_t K, void *stream)
{
    if (!A || !B || !C || !mult || !shift)
        return QG_ERR_NULLPTR;
    qg_status st = check_gemm(A, lda, false, B, ldb, true, C, ldc, 1, M, N, K, QG_W4A8_MAX_K);
    if (st == QG_OK)
        st = check_params(bias, mult, shift);
    if (st != QG_OK)
        return st;
    int cus = 0;
    if ((st = check_device(&cus)) != QG_OK)
        return st;
    qg::GemmDesc d{A, lda, B, ldb / 2, bias, mult, shift, C, ldc, M, N, K, cus, nullptr, 0, true};
    if (M <= qg::kSkinnyMaxM)
        return launched(qg::launch_w4a8_skinny(d, (hipStream_t)stream));
    return launched(qg::launch_w4a8_tiled(d, (hipStream_t)stream));
}

qg_status qconv2d_nhwc_s8_requant(const int8_t *X, const int8_t *W, const int32_t *bias,
                                  const int32_t *mult, const int32_t *shift, int8_t *Y,
                                  int32_t batch, int32_t H, int32_t Wd, int32_t C_in,
                                  int32_t C_out, int32_t KH, int32_t KW, int32_t stride_h,
                                  int32_t stride_w, int32_t pad_h, int32_t pad_w, void *stream)
{
    if (!X || !W || !Y || !mult || !shift)
        return QG_ERR_NULLPTR;
    int64_t Ho = 0, Wo = 0;
    qg_status st = check_conv(X, W, Y, batch, H, Wd, C_in, C_out, KH, KW, stride_h, stride_w,
                              pad_h, pad_w, &Ho, &Wo);
    if (st == QG_OK)
        st = check_params(bias, mult, shift);
    if (st != QG_OK)
        return st;
    int cus = 0;
    if ((st = check_device(&cus)) != QG_OK)
        return st;
    qg::ConvDesc d{X, W, bias, mult, shift, Y, batch, H, Wd, C_in, C_out, KH, KW,
                   stride_h, stride_w, pad_h, pad_w, (int)Ho, (int)Wo};
    if (qg::conv_halo_fits(d))
        return launched(qg::launch_conv_halo(d, (hipStream_t)stream));
    return launched(qg::launch_conv_nhwc(d, (hipStream_t)stream));
}

qg_status qdwconv2d_nhwc_s8_requant(const int8_t *X, const int8_t *W, const int32_t *bias,
                                    const int32_t *mult, const int32_t *shift, int8_t *Y,
                                    int32_t batch, int32_t H, int32_t Wd, int32_t C,
                                    int32_t KH, int32_t KW, int32_t stride_h, int32_t stride_w,
                                    int32_t pad_h, int32_t pad_w, void *stream)
{
    if (!X || !W || !Y || !mult || !shift)
        return QG_ERR_NULLPTR;
    int64_t Ho = 0, Wo = 0;
    qg_status st = check_dwconv(X, W, Y, batch, H, Wd, C, KH, KW, stride_h, stride_w, pad_h,
                                pad_w, &Ho, &Wo);
    if (st == QG_OK)
        st = check_params(bias, mult, shift);
    if (st != QG_OK)
        return st;
    int cus = 0;
    if ((st = check_device(&cus)) != QG_OK)
        return st;
    qg::ConvDesc d{X, W, bias, mult, shift, Y, batch, H, Wd, C, C, KH, KW,
                   stride_h, stride_w, pad_h, pad_w, (int)Ho, (int)Wo};
    return launched(qg::launch_dwconv_nhwc(d, (hipStream_t)stream));
}

qg_status qquant_per_token(const void *X, int32_t dtype, int64_t ldx, void *Q, int64_t ldq,
                           float *scale, int64_t M, int64_t K, float clip, int32_t bits,
                           void *stream)
{
    if (!X || !Q || !scale)
        return QG_ERR_NULLPTR;
    if (dtype != QG_DT_F32 && dtype != QG_DT_F16 && dtype != QG_DT_BF16)
        return QG_ERR_INVALID;
    if (bits != 8 && bits != 4)
        return QG_ERR_INVALID;
    if (!(clip > 0.0f && clip <= 1.0f))  // also rejects NaN
        return QG_ERR_INVALID;
    if (M < 1 || K < 16 || K % 16 != 0 || M > kMaxDim || K > kMaxDim)
        return QG_ERR_INVALID;
    // whole 16-byte vectors per input row; 16-byte input rows; output rows
    // 16 (int8) or 8 (int4) bytes
    if (ldx < K || ldq < K || ldx % (dtype == QG_DT_F32 ? 4 : 8) != 0 || ldq % 16 != 0)
        return QG_ERR_INVALID;
    if ((M + 3) / 4 >= kMaxGrid)
        return QG_ERR_INVALID;
    if (!aligned16(X) || !aligned16(Q) || ((uintptr_t)scale & 3u) != 0)
        return QG_ERR_INVALID;
    int cus = 0;
    qg_status st = check_device(&cus);
    if (st != QG_OK)
        return st;
    qg::QuantDesc d{X, dtype, ldx, Q, ldq, scale, M, K, clip, bits};
    return launched(qg::launch_quant_per_token(d, (hipStream_t)stream));
}

// ---- asymmetric forms ----

size_t qgemm_s8s8_requant_zp_workspace_size(int64_t M, int64_t N)
{
    if (M < 1 || N < 1 || M > kMaxDim || N > kMaxDim)
        return 0;
    return (size_t)qg::zp_gemm_workspace_bytes(M, N);
}

qg_status qgemm_s8s8_requant_zp(const int8_t *A, int64_t lda, const int8_t *B, int64_t ldb,
                                const int32_t *bias, const int32_t *mult, const int32_t *shift,
                                int32_t a_zero, int32_t b_zero, int32_t out_zero,
                                int32_t act_min, int32_t act_max, int8_t *C, int64_t ldc,
                                int64_t M, int64_t N, int64_t K, void *workspace,
                                size_t workspace_bytes, void *stream)
{
    if (!A || !B || !C || !mult || !shift)
        return QG_ERR_NULLPTR;
    qg_status st = check_gemm(A, lda, false, B, ldb, false, C, ldc, 1, M, N, K, kMaxDim);
    if (st == QG_OK)
        st = check_params(bias, mult, shift);
    if (st != QG_OK)
        return st;
    if (!zero_point_ok(a_zero) || !zero_point_ok(b_zero) || !zero_point_ok(out_zero) ||
        !act_ok(act_min, act_max))
        return QG_ERR_INVALID;
    if ((st = check_workspace(workspace, workspace_bytes, qg::zp_gemm_workspace_bytes(M, N))) !=
        QG_OK)
        return st;
    int cus = 0;
    if ((st = check_device(&cus)) != QG_OK)
        return st;
    qg::GemmDesc d{A, lda, B, ldb, bias, mult, shift, C, ldc, M, N, K, cus, nullptr, out_zero,
                   false, act_min, act_max};
    return launched(qg::run_s8s8_requant_zp(d, a_zero, b_zero, workspace, (hipStream_t)stream));
}

qg_status qgemm_s8s8_requant_zp_noalloc(const int8_t *A, int64_t lda, const int8_t *B,
                                        int64_t ldb, const int32_t *bias, const int32_t *mult,
                                        const int32_t *shift, int32_t a_zero, int32_t b_zero,
                                        int32_t out_zero, int32_t act_min, int32_t act_max,
                                        int8_t *C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                        void *stream)
{
    if (!A || !B || !C || !mult || !shift)
        return QG_ERR_NULLPTR;
    qg_status st = check_gemm(A, lda, false, B, ldb, false, C, ldc, 1, M, N, K, kMaxDim);
    if (st == QG_OK)
        st = check_params(bias, mult, shift);
    if (st != QG_OK)
        return st;
    if (!zero_point_ok(a_zero) || !zero_point_ok(b_zero) || !zero_point_ok(out_zero) ||
        !act_ok(act_min, act_max))
        return QG_ERR_INVALID;
    if (qg::zp_gemm_workspace_bytes(M, N) > qg::kNoAllocScratchBytes)
        return QG_ERR_INVALID;
    int cus = 0;
    if ((st = check_device(&cus)) != QG_OK)
        return st;
    void *ws = nullptr;
    if (qg::noalloc_scratch(&ws) != hipSuccess)
        return QG_ERR_LAUNCH;
    qg::GemmDesc d{A, lda, B, ldb, bias, mult, shift, C, ldc, M, N, K, cus, nullptr, out_zero,
                   false, act_min, act_max};
    return launched(qg::run_s8s8_requant_zp(d, a_zero, b_zero, ws, (hipStream_t)stream));
}

size_t qconv2d_nhwc_s8_requant_zp_workspace_size(int32_t batch, int32_t H, int32_t Wd,
                                                 int32_t C_out, int32_t KH, int32_t KW,
                                                 int32_t stride_h, int32_t stride_w,
                                                 int32_t pad_h, int32_t pad_w)
{
    if (batch < 1 || H < 1 || Wd < 1 || C_out < 1 || KH < 1 || KW < 1 || stride_h < 1 ||
        stride_w < 1 || pad_h < 0 || pad_w < 0)
        return 0;
    const int64_t span_h = (int64_t)H + 2 * (int64_t)pad_h - KH;
    const int64_t span_w = (int64_t)Wd + 2 * (int64_t)pad_w - KW;
    if (span_h < 0 || span_w < 0)
        return 0;
    const int64_t pixels = (int64_t)batch * (span_h / stride_h + 1) * (span_w / stride_w + 1);
    if (pixels > kMaxDim)
        return 0;
    return (size_t)qg::zp_conv_workspace_bytes(C_out, pixels);
}

qg_status qconv2d_nhwc_s8_requant_zp(const int8_t *X, const int8_t *W, const int32_t *bias,
                                     const int32_t *mult, const int32_t *shift, int32_t a_zero,
                                     int32_t b_zero, int32_t out_zero, int32_t act_min,
                                     int32_t act_max, int8_t *Y, int32_t batch,
                                     int32_t H, int32_t Wd, int32_t C_in, int32_t C_out,
                                     int32_t KH, int32_t KW, int32_t stride_h, int32_t stride_w,
                                     int32_t pad_h, int32_t pad_w, void *workspace,
                                     size_t workspace_bytes, void *stream)
{
    if (!X || !W || !Y || !mult || !shift)
        return QG_ERR_NULLPTR;
    int64_t Ho = 0, Wo = 0;
    qg_status st = check_conv(X, W, Y, batch, H, Wd, C_in, C_out, KH, KW, stride_h, stride_w,
                              pad_h, pad_w, &Ho, &Wo);
    if (st == QG_OK)
        st = check_params(bias, mult, shift);
    if (st != QG_OK)
        return st;
    if (!zero_point_ok(a_zero) || !zero_point_ok(b_zero) || !zero_point_ok(out_zero) ||
        !act_ok(act_min, act_max))
        return QG_ERR_INVALID;
    const int64_t pixels = (int64_t)batch * Ho * Wo;
    if ((st = check_workspace(workspace, workspace_bytes,
                              qg::zp_conv_workspace_bytes(C_out, pixels))) != QG_OK)
        return st;
    int cus = 0;
    if ((st = check_device(&cus)) != QG_OK)
        return st;
    qg::ConvDesc d{X, W, bias, mult, shift, Y, batch, H, Wd, C_in, C_out, KH, KW,
                   stride_h, stride_w, pad_h, pad_w, (int)Ho, (int)Wo,
                   true, a_zero, b_zero, out_zero, nullptr, act_min, act_max};
    return launched(qg::run_conv_zp(d, workspace, (hipStream_t)stream));
}

size_t qdwconv2d_nhwc_s8_requant_zp_workspace_size(int32_t C)
{
    if (C < 1)
        return 0;
    return (size_t)qg::zp_dw_workspace_bytes(C);
}

qg_status qdwconv2d_nhwc_s8_requant_zp(const int8_t *X, const int8_t *W, const int32_t *bias,
                                       const int32_t *mult, const int32_t *shift,
                                       int32_t a_zero, int32_t b_zero, int32_t out_zero,
                                       int32_t act_min, int32_t act_max,
                                       int8_t *Y, int32_t batch, int32_t H, int32_t Wd,
                                       int32_t C, int32_t KH, int32_t KW, int32_t stride_h,
                                       int32_t stride_w, int32_t pad_h, int32_t pad_w,
                                       void *workspace, size_t workspace_bytes, void *stream)
{
    if (!X || !W || !Y || !mult || !shift)
        return QG_ERR_NULLPTR;
    int64_t Ho = 0, Wo = 0;
    qg_status st = check_dwconv(X, W, Y, batch, H, Wd, C, KH, KW, stride_h, stride_w, pad_h,
                                pad_w, &Ho, &Wo);
    if (st == QG_OK)
        st = check_params(bias, mult, shift);
    if (st != QG_OK)
        return st;
    if (!zero_point_ok(a_zero) || !zero_point_ok(b_zero) || !zero_point_ok(out_zero) ||
        !act_ok(act_min, act_max))
        return QG_ERR_INVALID;
    if ((st = check_workspace(workspace, workspace_bytes, qg::zp_dw_workspace_bytes(C))) != QG_OK)
        return st;
    int cus = 0;
    if ((st = check_device(&cus)) != QG_OK)
        return st;
    qg::ConvDesc d{X, W, bias, mult, shift, Y, batch, H, Wd, C, C, KH, KW,
                   stride_h, stride_w, pad_h, pad_w, (int)Ho, (int)Wo,
                   true, a_zero, b_zero, out_zero, nullptr, act_min, act_max};
    return launched(qg::run_dwconv_zp(d, workspace, (hipStream_t)stream));
}

const char *qg_status_string(qg_status s)
{
    // A C caller may pass any int here.  In C++ an enumeration object that
    // holds a value outside the enumerators' range must not be read as the
    // enumeration (undefined behaviour), so switch on its bytes as an int.
    int v;
    static_assert(sizeof v == sizeof s, "qg_status is int-sized");
    memcpy(&v, &s, sizeof v);
    switch (v) {
    case QG_OK:
        return "QG_OK";
    case QG_ERR_NULLPTR:
        return "QG_ERR_NULLPTR: a required pointer is NULL";
    case QG_ERR_INVALID:
        return "QG_ERR_INVALID: a size, stride or alignment rule is broken";
    case QG_ERR_NO_DEVICE:
        return "QG_ERR_NO_DEVICE: no current HIP device, or it is not gfx950";
    case QG_ERR_LAUNCH:
        return "QG_ERR_LAUNCH: kernel launch failed";
    }
    return "unknown qg_status";
}

int qg_version(void) { return 100; }

}  // extern "C"
