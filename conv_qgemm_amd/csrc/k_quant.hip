// k_quant.hip -- per-token symmetric quantization of float activations to
// int8 or packed int4, with one float scale per token.
//
// Method: per token, scale = max|x| / (qmax / clip_ratio) (Ascend FlatQuant
// operator article, www.zwxr.cn/news/277566, per-token mode; qmax is 7 for
// int4 and 127 for int8), and the code of x is x / scale rounded half away
// from zero (Voyager quantization article, www.dpshk.com/news/2695434, §1.1,
// zero point 0), clamped to [-qmax, qmax].  Packed int4 puts element 2i in
// the low nibble of byte i (INT4 GEMM article, www.cf-1.com/news/6060138,
// §2.1).  All of it in IEEE binary32; float16 and bfloat16 inputs are first
// widened to binary32, which is exact.
//
// Each token row is owned by 64 * WPR threads (WPR waves; 256 threads for
// rows of 256 or more 16-byte vectors), reading the row as 16-byte vectors:
// vector i = s * 64 * WPR + thread, so each wave load instruction covers 1 KB
// of contiguous row and the codes of vector i land at i * (bytes out per
// vector), contiguous per store instruction too.  Rows of up to 16 vectors
// per thread stay in registers between the max|x| pass and the code pass;
// longer rows are read twice.  The waves of a row combine their maxima
// through LDS.
//
// Exactness without a division per element: the code must be that of the
// correctly rounded quotient q = x / scale.  For scale in [2^-100, 2^100]
// the kernel forms t = x * (1 / scale) with a correctly rounded reciprocal,
// so |t - q| <= 3 * 2^-24 * |x / scale| (three roundings), and takes the code
// as floor(|t| + 1/2) in binary32, clamped, with the sign of t.  While |t| <=
// 129, |t - q| < 2.31e-5 and rounding |t| + 1/2 moves it by at most 2^-17,
// together under 3.1e-5, half of 2^-14; so unless |t| + 1/2 lies within 2^-14 of an
// integer (t near a half-integer), floor(|t| + 1/2) equals round-half-away-
// from-zero of |q|.  For |t| > 129, |q| > 128.99 and both clamp to qmax.  In
// the near-tie case (about one element in 8000), and for every element when
// the scale is outside that range, the code comes from the exact division.
// Non-finite inputs are outside the method's domain.
#include "dev_common.hpp"
#include "launch.hpp"

namespace qg {

namespace {

constexpr int kWaves = 4;  // token rows per workgroup

struct QuantArgs {
    const uint8_t *X;
    int64_t ldx_b;  // bytes per input row
    int64_t M;
    int nv;         // 16-byte input vectors per row
    float clip;
    uint8_t *Q;
    int64_t ldq_b;  // bytes per output row
    float *scale;
};

// element e of a 16-byte vector: 4 binary32, or 8 binary16 / bfloat16
template <int DT>
__device__ __forceinline__ float elem(v4i r, int e)
{
    if constexpr (DT == 0) {
        return __int_as_float(r[e]);
    } else {
        const unsigned w = (unsigned)r[e >> 1];
        const unsigned h = (e & 1) ? (w >> 16) : (w & 0xFFFFu);
        if constexpr (DT == 2)
            return __uint_as_float(h << 16);  // bfloat16 is the top half of a binary32
        else
            return (float)__builtin_bit_cast(_Float16, (unsigned short)h);  // exact
    }
}

template <int DT>
__device__ __forceinline__ float vec_amax(v4i r, float amax)
{
    constexpr int NE = DT == 0 ? 4 : 8;
#pragma unroll
    for (int e = 0; e < NE; ++e)
        amax = fmaxf(amax, fabsf(elem<DT>(r, e)));
    return amax;
}

// x / sc in binary32, rounded half away from zero, clamped to [-qmax, qmax],
// as a float; sc > 0
__device__ __forceinline__ float exact_code(float x, float sc, float qmax)
{
    const float q = x / sc;
    const float a = fabsf(q);
    const float tr = truncf(a);
    const float r = fminf(tr + (a - tr >= 0.5f ? 1.0f : 0.0f), qmax);
    return copysignf(r, q);
}

// codes of one input vector, stored at dst (bytes per vector: 4 or 8 for
// int8, 2 or 4 for int4); sc == 0 gives codes 0
template <int DT, int BITS>
__device__ __forceinline__ void emit(uint8_t *dst, v4i r, float sc, float rsc, bool fast)
{
    constexpr int NE = DT == 0 ? 4 : 8;
    constexpr float QMAX = BITS == 4 ? 7.0f : 127.0f;
    float x[NE], f[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e)
        x[e] = elem<DT>(r, e);
    bool slow = !fast;
    if (fast) {
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const float t = x[e] * rsc;
            const float s = fabsf(t) + 0.5f;
            const float fl = floorf(s);
            slow |= fabsf((s - fl) - 0.5f) > 0.5f - 0x1p-14f;
            f[e] = copysignf(fminf(fl, QMAX), t);
        }
    }
    if (slow) {
#pragma unroll
        for (int e = 0; e < NE; ++e)
            f[e] = sc > 0.0f ? exact_code(x[e], sc, QMAX) : 0.0f;
    }
    int q[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e)
        q[e] = (int)f[e];
    if constexpr (BITS == 8) {
        if constexpr (NE == 4) {
            *(unsigned *)dst = pack4_i8(q[0], q[1], q[2], q[3]);
        } else {
            v2u w;
            w[0] = pack4_i8(q[0], q[1], q[2], q[3]);
            w[1] = pack4_i8(q[4], q[5], q[6], q[7]);
            *(v2u *)dst = w;
        }
    } else {
        unsigned w = 0;
#pragma unroll
        for (int e = 0; e < NE; ++e)
            w |= (unsigned)(q[e] & 0xF) << (4 * e);
        if constexpr (NE == 4)
            *(unsigned short *)dst = (unsigned short)w;
        else
            *(unsigned *)dst = w;
    }
}

// WPR waves per row, kWaves / WPR rows per workgroup; KEEP vectors per
// thread held in registers (0: the row is read twice)
template <int DT, int BITS, int WPR, int KEEP>
__global__ __launch_bounds__(kWaves * 64) void k_quant(QuantArgs p)
{
    constexpr int OB = (DT == 0 ? 4 : 8) * BITS / 8;  // output bytes per input vector
    constexpr float QMAX = BITS == 4 ? 7.0f : 127.0f;
    constexpr int TPR = WPR * 64;                      // threads per row
    __shared__ float red[kWaves];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = (wave % WPR) * 64 + lane;
    const int64_t m = (int64_t)blockIdx.x * (kWaves / WPR) + wave / WPR;
    const bool valid = m < p.M;
    // a wave past the last row reads row 0 and stores nothing
    const v4i *row = (const v4i *)(p.X + (valid ? m : 0) * p.ldx_b);
    const int nv = p.nv;

    float amax = 0.0f;
    v4i keep[KEEP > 0 ? KEEP : 1];
    if constexpr (KEEP > 0) {
        // every thread loads KEEP vectors; one past the row end re-reads the
        // last vector, which leaves the maximum unchanged
#pragma unroll
        for (int s = 0; s < KEEP; ++s)
            keep[s] = row[min(s * TPR + t, nv - 1)];
#pragma unroll
        for (int s = 0; s < KEEP; ++s)
            amax = vec_amax<DT>(keep[s], amax);
    } else {
        for (int i = t; i < nv; i += TPR)
            amax = vec_amax<DT>(row[i], amax);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        amax = fmaxf(amax, __shfl_xor(amax, o));
    if constexpr (WPR > 1) {
        if (lane == 0)
            red[wave] = amax;
        __syncthreads();
        const int w0 = wave / WPR * WPR;
#pragma unroll
        for (int j = 0; j < WPR; ++j)
            amax = fmaxf(amax, red[w0 + j]);
    }
    if (!valid)
        return;
    const float sc = amax / (QMAX / p.clip);
    if (t == 0)
        p.scale[m] = sc;
    const bool fast = sc >= 0x1p-100f && sc <= 0x1p100f;
    const float rsc = fast ? 1.0f / sc : 0.0f;

    uint8_t *qrow = p.Q + m * p.ldq_b;
    if constexpr (KEEP > 0) {
#pragma unroll
        for (int s = 0; s < KEEP; ++s) {
            const int i = s * TPR + t;
            if (i < nv)
                emit<DT, BITS>(qrow + (int64_t)i * OB, keep[s], sc, rsc, fast);
        }
    } else {
        for (int i = t; i < nv; i += TPR)
            emit<DT, BITS>(qrow + (int64_t)i * OB, row[i], sc, rsc, fast);
    }
}

template <int DT, int BITS, int WPR, int KEEP>
hipError_t run(const QuantArgs &a, hipStream_t s)
{
    constexpr int RPB = kWaves / WPR;  // rows per workgroup
    const dim3 grid((unsigned)((a.M + RPB - 1) / RPB)), block(kWaves * 64);
    hipLaunchKernelGGL((k_quant<DT, BITS, WPR, KEEP>), grid, block, 0, s, a);
    return hipGetLastError();
}

// short rows get one or two waves per row; rows of 256 vectors and more get
// the whole workgroup
template <int DT, int BITS>
hipError_t run_quant(const QuantArgs &a, hipStream_t s)
{
    const int nv = a.nv;
    if (nv <= 64)
        return run<DT, BITS, 1, 1>(a, s);
    if (nv <= 128)
        return run<DT, BITS, 2, 1>(a, s);
    if (nv <= 256)
        return run<DT, BITS, 4, 1>(a, s);
    if (nv <= 512)
        return run<DT, BITS, 4, 2>(a, s);
    if (nv <= 1024)
        return run<DT, BITS, 4, 4>(a, s);
    if (nv <= 2048)
        return run<DT, BITS, 4, 8>(a, s);
    if (nv <= 4096)
        return run<DT, BITS, 4, 16>(a, s);
    return run<DT, BITS, 4, 0>(a, s);
}

}  // namespace

hipError_t launch_quant_per_token(const QuantDesc &d, hipStream_t s)
{
    const int eb = d.dtype == 0 ? 4 : 2;
    QuantArgs a{};
    a.X = (const uint8_t *)d.X;
    a.ldx_b = d.ldx * eb;
    a.M = d.M;
    a.nv = (int)(d.K * eb / 16);
    a.clip = d.clip;
    a.Q = (uint8_t *)d.Q;
    a.ldq_b = d.bits == 8 ? d.ldq : d.ldq / 2;
    a.scale = d.scale;
    if (d.bits == 8) {
        if (d.dtype == 0)
            return run_quant<0, 8>(a, s);
        if (d.dtype == 1)
            return run_quant<1, 8>(a, s);
        return run_quant<2, 8>(a, s);
    }
    if (d.dtype == 0)
        return run_quant<0, 4>(a, s);
    if (d.dtype == 1)
        return run_quant<1, 4>(a, s);
    return run_quant<2, 4>(a, s);
}

}  // namespace qg
