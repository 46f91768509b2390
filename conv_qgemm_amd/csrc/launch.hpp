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

// NHWC conv with stride 1 and 64 input channels, input rows staged in LDS
// (k_conv_halo.hip); other convs use the implicit-im2col tile kernel
bool conv_halo_fits(const ConvDesc &d);
hipError_t launch_conv_halo(const ConvDesc &d, hipStream_t s);

// depthwise NHWC conv (k_dwconv.hip); C_in == C_out == the channel count
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
