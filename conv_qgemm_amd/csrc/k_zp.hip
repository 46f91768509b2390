// k_zp.hip -- the asymmetric (zero-point) forms: compensation terms and the
// host-side sequence that runs them ahead of the GEMM / conv kernels.
//
// Method: a code Q stands for (Q - zero_point) * scale (Voyager quantization
// article, www.dpshk.com/news/2695434, §1.1), so the accumulator of an
// asymmetric GEMM is sum_k (A - za)(B - zb).  Both operands carry a zero
// point, which the INT4 GEMM article (www.cf-1.com/news/6060138, §4.1)
// compensates after the product.  Expanded:
//     sum (A - za)(B - zb) = sum A*B - zb * sum_k A[m] - za * sum_k B[n]
//                            + K * za * zb,
// so the int8 matrix cores keep multiplying the raw codes, and two vectors
// of sums finish the job in the requantize epilogue:
//     cterm[n] = bias[n] - za * sum_k B[n][k] + K * za * zb   (per column)
//     rterm[m] = zb * sum_k A[m][k]                           (per row)
// x = sum A*B - rterm[m] + cterm[n] is formed modulo 2^32; it equals the
// true x whenever that fits in int32, which the API requires.
// For a conv the rows of A are im2col rows whose padding holds the input
// zero point (MCU conv front-end article, news.rkmt.cn/news/16638, §2.3);
// the conv kernels pad with za, and rterm sums those rows the same way.  The
// LDS-staged conv kernel (stride 1, 64 input channels) forms both sums
// itself from data it already holds and needs no pass here.
// The depthwise 3x3 kernel takes zb = 0 and cterm only; other depthwise
// shapes multiply (x - za)(w - zb) directly.
//
// Row sums use v_dot4_i32_i8 against 0x01010101 (four bytes per
// instruction), one wave per row, 16-byte loads with eight in flight per
// lane; they are memory-bound passes over A and B.
#include <atomic>

#include "dev_common.hpp"
#include "launch.hpp"

namespace qg {

namespace {

struct RowTermArgs {
    const int8_t *A;
    int64_t lda_b;
    const int8_t *B;
    int64_t ldb_b;
    const int32_t *bias;
    int64_t M, N;
    int K;
    int za, zb;
    int32_t *cterm;
    int32_t *rterm;  // null: no per-row terms
};

// sum of one int8 row of K bytes (K % 16 == 0, 16-byte aligned), modulo
// 2^32, reduced over the wave
__device__ __forceinline__ unsigned row_sum_s8(const int8_t *row, int nv, int lane)
{
    constexpr int kBatch = 8;  // loads in flight per lane
    unsigned s = 0;
    for (int i0 = 0; i0 < nv; i0 += 64 * kBatch) {
        v4i v[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int i = i0 + 64 * j + lane;
            v[j] = i < nv ? *(const v4i *)(row + (int64_t)i * 16) : (v4i){0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                s = (unsigned)__builtin_amdgcn_sdot4(v[j][e], 0x01010101, (int)s, false);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        s += (unsigned)__shfl_xor((int)s, o);
    return s;
}

// one wave per row: rows [0, N) are B's (-> cterm), rows [N, N + M) A's
// (-> rterm, when wanted)
__global__ __launch_bounds__(256) void k_row_terms(RowTermArgs p)
{
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t rows = p.N + (p.rterm ? p.M : 0);
    if (r >= rows)
        return;
    const int nv = p.K / 16;
    if (r < p.N) {
        const unsigned sb = row_sum_s8(p.B + r * p.ldb_b, nv, lane);
        if (lane == 0) {
            const unsigned b = p.bias ? (unsigned)p.bias[r] : 0u;
            p.cterm[r] = (int)(b - (unsigned)p.za * sb + (unsigned)p.K * (unsigned)(p.za * p.zb));
        }
    } else {
        const int64_t m = r - p.N;
        const unsigned sa = row_sum_s8(p.A + m * p.lda_b, nv, lane);
        if (lane == 0)
            p.rterm[m] = (int)((unsigned)p.zb * sa);
    }
}

struct ConvRowArgs {
    const int8_t *X;
    int H, Wd, C_in, KH, KW, sh, sw, ph, pw, Ho, Wo;
    int64_t npix;
    int za, zb;
    int32_t *rterm;
};

// one thread per output pixel: zb * (sum over its taps and input channels,
// a padded tap counting C_in * za)
__global__ __launch_bounds__(256) void k_conv_rowterm(ConvRowArgs p)
{
    const int64_t pix = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (pix >= p.npix)
        return;
    const int64_t HW = (int64_t)p.Ho * p.Wo;
    const int64_t b = pix / HW;
    const int rem = (int)(pix - b * HW);
    const int oh = rem / p.Wo, ow = rem - (rem / p.Wo) * p.Wo;
    const unsigned pad_sum = (unsigned)p.C_in * (unsigned)p.za;
    unsigned s = 0;
    for (int kh = 0; kh < p.KH; ++kh) {
        const int ih = oh * p.sh - p.ph + kh;
        for (int kw = 0; kw < p.KW; ++kw) {
            const int iw = ow * p.sw - p.pw + kw;
            if (ih < 0 || ih >= p.H || iw < 0 || iw >= p.Wd) {
                s += pad_sum;
                continue;
            }
            const int8_t *px = p.X + ((b * p.H + ih) * p.Wd + iw) * p.C_in;
            for (int c = 0; c < p.C_in; c += 16) {
                const v4i v = *(const v4i *)(px + c);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    s = (unsigned)__builtin_amdgcn_sdot4(v[e], 0x01010101, (int)s, false);
            }
        }
    }
    p.rterm[pix] = (int)((unsigned)p.zb * s);
}

// one thread per channel: bias[c] - za * sum over taps of W[t][c]
__global__ __launch_bounds__(256) void k_dw_terms(const int8_t *W, const int32_t *bias, int C,
                                                  int taps, int za, int32_t *cterm)
{
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= C)
        return;
    unsigned s = 0;
    for (int t = 0; t < taps; ++t)
        s += (unsigned)(int)W[(int64_t)t * C + c];
    const unsigned b = bias ? (unsigned)bias[c] : 0u;
    cterm[c] = (int)(b - (unsigned)za * s);
}

int64_t align256(int64_t bytes) { return (bytes + 255) & ~(int64_t)255; }

}  // namespace

hipError_t launch_zp_gemm_terms(const int8_t *A, int64_t lda_b, const int8_t *B, int64_t ldb_b,
                                const int32_t *bias, int64_t M, int64_t N, int64_t K, int za,
                                int zb, int32_t *cterm, int32_t *rterm, hipStream_t s)
{
    RowTermArgs a{A, lda_b, B, ldb_b, bias, M, N, (int)K, za, zb, cterm, rterm};
    const int64_t rows = N + (rterm ? M : 0);
    hipLaunchKernelGGL(k_row_terms, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_zp_conv_rowterm(const ConvDesc &d, int32_t *rterm, hipStream_t s)
{
    ConvRowArgs a{d.X, d.H, d.Wd, d.C_in, d.KH, d.KW, d.sh, d.sw, d.ph, d.pw, d.Ho, d.Wo,
                  (int64_t)d.batch * d.Ho * d.Wo, d.a_zero, d.b_zero, rterm};
    hipLaunchKernelGGL(k_conv_rowterm, dim3((unsigned)((a.npix + 255) / 256)), dim3(256), 0, s,
                       a);
    return hipGetLastError();
}

hipError_t launch_zp_dw_terms(const ConvDesc &d, int32_t *cterm, hipStream_t s)
{
    hipLaunchKernelGGL(k_dw_terms, dim3((unsigned)((d.C_in + 255) / 256)), dim3(256), 0, s, d.W,
                       d.bias, d.C_in, d.KH * d.KW, d.a_zero, cterm);
    return hipGetLastError();
}

// ---- workspace layouts: cterm first, then rterm, each 256-byte aligned ----

int64_t zp_gemm_workspace_bytes(int64_t M, int64_t N)
{
    return align256(4 * N) + align256(4 * M);
}

int64_t zp_conv_workspace_bytes(int64_t C_out, int64_t pixels)
{
    return align256(4 * C_out) + align256(4 * pixels);
}

int64_t zp_dw_workspace_bytes(int64_t C)
{
    return align256(4 * C);
}

hipError_t run_s8s8_requant_zp(GemmDesc d, int za, int zb, void *ws, hipStream_t s)
{
    int32_t *cterm = (int32_t *)ws;
    int32_t *rterm = (int32_t *)((uint8_t *)ws + align256(4 * d.N));
    d.rterm = nullptr;
    if (za != 0 || zb != 0) {
        hipError_t e = launch_zp_gemm_terms((const int8_t *)d.A, d.lda_b, (const int8_t *)d.B,
                                            d.ldb_b, d.bias, d.M, d.N, d.K, za, zb, cterm,
                                            zb != 0 ? rterm : nullptr, s);
        if (e != hipSuccess)
            return e;
        d.bias = cterm;
        d.rterm = zb != 0 ? rterm : nullptr;
    }
    return launch_s8s8_requant_zp(d, s);
}

hipError_t run_conv_zp(ConvDesc d, void *ws, hipStream_t s)
{
    d.asym = true;
    d.rterm = nullptr;
    // the LDS-staged kernel forms both terms itself
    if (conv_halo_fits(d))
        return launch_conv_halo(d, s);
    int32_t *cterm = (int32_t *)ws;
    int32_t *rterm = (int32_t *)((uint8_t *)ws + align256(4 * (int64_t)d.C_out));
    if (d.a_zero != 0 || d.b_zero != 0) {
        const int64_t Kc = (int64_t)d.KH * d.KW * d.C_in;
        hipError_t e = launch_zp_gemm_terms(nullptr, 0, d.W, Kc, d.bias, 0, d.C_out, Kc, d.a_zero,
                                            d.b_zero, cterm, nullptr, s);
        if (e != hipSuccess)
            return e;
        d.bias = cterm;
    }
    if (d.b_zero != 0) {
        hipError_t e = launch_zp_conv_rowterm(d, rterm, s);
        if (e != hipSuccess)
            return e;
        d.rterm = rterm;
    }
    return launch_conv_nhwc(d, s);
}

hipError_t run_dwconv_zp(ConvDesc d, void *ws, hipStream_t s)
{
    d.asym = true;
    if (dw_takes_mfma(d) && d.a_zero != 0) {
        int32_t *cterm = (int32_t *)ws;
        hipError_t e = launch_zp_dw_terms(d, cterm, s);
        if (e != hipSuccess)
            return e;
        d.bias = cterm;
    }
    return launch_dwconv_nhwc(d, s);
}

// ---- the allocation-free asymmetric GEMM: its compensation sums go to a
//      file-scope device array instead of a caller workspace.  Every GPU the
//      library runs on holds its own copy for the life of the process, and
//      every call on that GPU shares it: calls that overlap on one GPU (two
//      streams, or two host threads) race on it.  Each call writes every
//      entry it reads (cterm[n] for n < N, rterm[m] for m < M) before the
//      GEMM kernel reads it, so nothing needs clearing between calls. ----

namespace {

constexpr int kScratchDevices = 64;

__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

// device address of `scratch` on each device, taken once per device with
// that device current; in host code the array's name is only a stand-in
std::atomic<void *> g_scratch[kScratchDevices];

}  // namespace

hipError_t noalloc_scratch(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kScratchDevices)
        return hipErrorInvalidDevice;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace qg
