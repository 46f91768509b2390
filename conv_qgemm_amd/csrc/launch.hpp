// launch.hpp -- host-side descriptors and kernel launchers inside libqgemm.
// Internal to the library; the public ABI is include/qgemm.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace qg {

// One GEMM: C[m][n] = epilogue(sum_k A[m][k] * B[n][k]).  Strides in bytes
// for A/B (packed int4 rows are K/2 bytes), in elements for C.
struct GemmDesc {
    const void *A;
    int64_t lda_b;
    const void *B;
    int64_t ldb_b;
    const int32_t *bias;  // may be null
    const int32_t *mult;
    const int32_t *shift;
    void *C;
    int64_t ldc;
    int64_t M, N, K;  // K in values
    int cus;          // compute units of the current device
    // asymmetric form (launch_s8s8_requant_zp): `bias` is the per-column
    // term, rterm the per-row term (or null), out_zero the output zero point
    const int32_t *rterm;
    int out_zero;
    // W4A8: the int4 weights are packed high nibble first
    bool msb_first;
    // asymmetric form: output clamp bounds (fused activation)
    int act_min, act_max;
    // binary16 output (launch_s4s4_f16): per-row / per-column scales or null
    const float *scale_a;
    const float *scale_b;
};

// One NHWC conv as an implicit GEMM: M = batch*Ho*Wo pixels, N = C_out,
// K = KH*KW*C_in, B = OHWI weights viewed as [C_out][K].
struct ConvDesc {
    const int8_t *X;
    const int8_t *W;
    const int32_t *bias;
    const int32_t *mult;
    const int32_t *shift;
    int8_t *Y;
    int batch, H, Wd, C_in, C_out, KH, KW, sh, sw, ph, pw, Ho, Wo;
    // asymmetric form: padding holds a_zero, `bias` is the per-channel term,
    // rterm the per-pixel term (or null), out_zero the output zero point;
    // b_zero is used only by the direct depthwise kernel
    bool asym;
    int a_zero, b_zero, out_zero;
    const int32_t *rterm;
    int act_min, act_max;  // asymmetric form: output clamp bounds
};

hipError_t launch_s8s8_requant(const GemmDesc &d, hipStream_t s);
hipError_t launch_s4s4_i32(const GemmDesc &d, hipStream_t s);
hipError_t launch_w4a8_tiled(const GemmDesc &d, hipStream_t s);
hipError_t launch_w4a8_skinny(const GemmDesc &d, hipStream_t s);
hipError_t launch_conv_nhwc(const ConvDesc &d, hipStream_t s);

// 256x256 ring kernel for large GEMMs (k_gemm_dma.hip)
bool dma_gemm_fits(const GemmDesc &d, bool int4);
hipError_t launch_s8s8_requant_dma(const GemmDesc &d, hipStream_t s);
hipError_t launch_s4s4_i32_dma(const GemmDesc &d, hipStream_t s);
hipError_t launch_s8s8_requant_zp_dma(const GemmDesc &d, hipStream_t s);
hipError_t launch_s4s4_f16_dma(const GemmDesc &d, hipStream_t s);
bool dma_w4a8_fits(const GemmDesc &d);
hipError_t launch_w4a8_requant_dma(const GemmDesc &d, hipStream_t s);

// INT4 x INT4 with a binary16 output: C = fp16(fp32(acc) * scale_a[m] *
// scale_b[n]) (C is [M][ldc] binary16 bit patterns)
hipError_t launch_s4s4_f16(const GemmDesc &d, hipStream_t s);

// asymmetric int8 GEMM: the terms come from launch_zp_gemm_terms
hipError_t launch_s8s8_requant_zp(const GemmDesc &d, hipStream_t s);

// Compensation terms of the asymmetric forms (k_zp.hip), modulo 2^32:
//   cterm[n] = bias[n] - za * sum_k B[n][k] + K * za * zb   (n < N)
//   rterm[m] = zb * sum_k A[m][k]                           (m < M; only
//              when rterm is not null)
// B and A are int8 [rows][ld] with K % 16 == 0 and 16-byte rows.
hipError_t launch_zp_gemm_terms(const int8_t *A, int64_t lda_b, const int8_t *B, int64_t ldb_b,
                                const int32_t *bias, int64_t M, int64_t N, int64_t K, int za,
                                int zb, int32_t *cterm, int32_t *rterm, hipStream_t s);
// Per-pixel term of the asymmetric conv: rterm[p] = zb * (sum over the taps
// and input channels of output pixel p, padding counted as za).
hipError_t launch_zp_conv_rowterm(const ConvDesc &d, int32_t *rterm, hipStream_t s);
// Per-channel term of the asymmetric depthwise conv with zb = 0:
// cterm[c] = bias[c] - za * sum over taps of W[t][c].
hipError_t launch_zp_dw_terms(const ConvDesc &d, int32_t *cterm, hipStream_t s);

// The asymmetric entry points' sequences (k_zp.hip): the terms into the
// workspace, then the GEMM / conv kernel.  Workspace bytes: cterm, then
// rterm, each rounded up to 256 bytes.
int64_t zp_gemm_workspace_bytes(int64_t M, int64_t N);
int64_t zp_conv_workspace_bytes(int64_t C_out, int64_t pixels);
int64_t zp_dw_workspace_bytes(int64_t C);
hipError_t run_s8s8_requant_zp(GemmDesc d, int za, int zb, void *ws, hipStream_t s);
// The allocation-free asymmetric GEMM keeps its compensation sums in a
// file-scope device array of kNoAllocScratchBytes (k_zp.hip); noalloc_scratch
// gives that array's address on the current device.
constexpr int64_t kNoAllocScratchBytes = (int64_t)1 << 20;
hipError_t noalloc_scratch(void **ptr);
hipError_t run_conv_zp(ConvDesc d, void *ws, hipStream_t s);
hipError_t run_dwconv_zp(ConvDesc d, void *ws, hipStream_t s);

// NHWC conv with stride 1 and 64 input channels, input rows staged in LDS
// (k_conv_halo.hip); other convs use the implicit-im2col tile kernel
bool conv_halo_fits(const ConvDesc &d);
hipError_t launch_conv_halo(const ConvDesc &d, hipStream_t s);

// depthwise NHWC conv (k_dwconv.hip); C_in == C_out == the channel count.
// dw_takes_mfma: the 3x3 matrix-core path runs (its asymmetric form needs
// the per-channel term in `bias`); otherwise the direct kernel runs.
bool dw_takes_mfma(const ConvDesc &d);
hipError_t launch_dwconv_nhwc(const ConvDesc &d, hipStream_t s);

// Per-token activation quantizer (k_quant.hip).  dtype 0 binary32, 1
// binary16, 2 bfloat16; ldx in elements; ldq in output values (nibbles for
// bits 4).
struct QuantDesc {
    const void *X;
    int dtype;
    int64_t ldx;
    void *Q;
    int64_t ldq;
    float *scale;
    int64_t M, K;
    float clip;
    int bits;
};

hipError_t launch_quant_per_token(const QuantDesc &d, hipStream_t s);

// Largest M the weight-streaming W4A8 kernel takes; larger M is tiled.
constexpr int64_t kSkinnyMaxM = 64;

}  // namespace qg
