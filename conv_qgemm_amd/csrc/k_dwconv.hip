// k_dwconv.hip -- depthwise NHWC int8 conv with the Q31 requantize fused.
//
// Method (MCU conv front-end article, news.rkmt.cn/news/16638): in a
// depthwise conv every channel is convolved on its own, input channel c
// feeding only output channel c, with weights laid out [kh][kw][c] and the
// border filled with the zero point (§3.3); the requantize is §2.3's.
//
// The 3x3 path (stride 1 or 2, channels a multiple of 16) runs on the int8
// MFMA even though a depthwise output is only 9 products: the K axis of one
// v_mfma_i32_16x16x64_i8 is laid out as 4 taps x 16 channels, and the other
// operand holds the weights on a diagonal (weight w[t][c] at K position
// (t, c) of column c, zero elsewhere).  Three MFMAs then give 16 pixels x 16
// channels of a 3x3 conv (taps 9..11 have zero weights).  Per workgroup
// (8 waves, one workgroup per CU): 392 consecutive output pixels of one
// image (7 rows of a 56-wide output, so 32 images make one workgroup per CU
// of an MI355X) x a 64-channel slice; the 25 16-pixel MFMA tiles go to the
// waves in turn (wave w takes tiles w, w + 8, w + 16, and wave 0 also
// tile 24).
//   * the input rows those pixels touch are staged once in LDS, every pixel
//     in 80 bytes (the slice's 64 channels + 16 unused) with columns and
//     rows of the padding value (the input zero point, 0 when symmetric), so
//     a tap is a fixed LDS offset and 16 consecutive pixels fall in 16
//     different bank groups.  With stride 1 the LDS row holds a pixel count
//     congruent to Wo mod 16, so that this stays true across a row end;
//   * a 16-byte LDS read serves 16 lanes per cycle: lane rows 0 and 1 (and
//     2 and 3) share cycles, each with 8 of the 16 pixels.  Their two taps
//     then fall on 16 distinct bank groups when their LDS offsets differ by
//     a multiple of 16 pixels.  With stride 1 and Wo a multiple of 8 the
//     taps are placed so: kernel rows 0 and 2 pair up (two row pitches
//     apart), and each tap of kernel row 1 shares its cycles with a
//     zero-weight copy of itself;
//   * the diagonal weight operands live in registers (12 per lane);
//   * the requantize takes the cheapest exact form all 64 shifts of the
//     slice allow; a 4 x 4 lane transpose (permlane swaps) gives each lane
//     16 consecutive channels of one pixel for a 16-byte store.
// Other kernel sizes and strides use a direct kernel: one thread per output
// pixel and 4 channels.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "dev_common.hpp"
#include "launch.hpp"

namespace qg {

namespace {

constexpr int kTP = 392;     // output pixels per workgroup (7 rows of a 56-wide output)
constexpr int kTiles = (kTP + 15) / 16;  // 16-pixel MFMA tiles per workgroup (25)
constexpr int kCS = 64;      // channels per workgroup slice
constexpr int kPixL = 80;    // LDS bytes per staged input pixel
constexpr int kWaves = 8;    // two waves per SIMD
constexpr int kTPW = (kTiles + kWaves - 1) / kWaves;  // MFMA tiles per wave: w, w + 8, ... < kTiles
constexpr int kMaxLds = 160 * 1024;  // one workgroup per CU
constexpr int kMaxDevices = 64;

struct DwArgs {
    const int8_t *X;
    const int8_t *W;  // [KH][KW][C]
    const int32_t *bias;
    const int32_t *mult;
    const int32_t *shift;
    int8_t *Y;
    int H, Wd, C, KH, KW, sh, sw, ph, pw, Ho, Wo;
    int tiles_per_img;
    int in_bytes;   // LDS bytes of the staged input rows
    int colsL;      // LDS pixels per staged row (>= Wd + 2 pw)
    int tap_pairs;  // taps placed in bank-conflict-free pairs (stride 1, Wo % 8 == 0)
    // asymmetric form: the padding byte x4 and the zero points; the 3x3 path
    // takes zb = 0 with `bias` holding bias - za * sum_t w[t][c]
    int pad4, a_zero, b_zero, out_zero;
    int act_min, act_max;  // output clamp bounds (the int8 range when symmetric)
};

__device__ __forceinline__ void drain_and_barrier()
{
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---- 3x3 depthwise on the MFMA ----
// S: stride (both directions); ZP: the asymmetric form (padding a_zero, the
// output zero point before the saturation)
template <int S, bool ZP>
__global__ __launch_bounds__(kWaves * 64, 1) void k_dwconv3x3(DwArgs p)
{
    constexpr int KH = 3, KW = 3, KK = 9, kSlices = 3;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    uint8_t *IN = lds;
    int *prm = (int *)(lds + p.in_bytes);  // bias, mult, shift [3][64]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // the wave's last MFMA tile exists for the first kTiles % kWaves waves
    const bool has_last = wave + kWaves * (kTPW - 1) < kTiles;
    const int col = lane & 15;
    const int g = lane >> 4;

    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int b = bid / p.tiles_per_img, tile = bid - b * p.tiles_per_img;
    const int HW = p.Ho * p.Wo;
    const int p0 = tile * kTP, npix = min(kTP, HW - p0);
    const int c0 = blockIdx.y * kCS;
    const int cs = min(kCS, p.C - c0);  // channels of this slice (a multiple of 16)
    const int ngrp = cs >> 4;
    const int oh_first = p0 / p.Wo, oh_last = (p0 + npix - 1) / p.Wo;
    const int ih0 = oh_first * S - p.ph;  // input row of LDS row 0
    const int nrow_in = (oh_last - oh_first) * S + KH;
    const int ih_lo = max(ih0, 0), ih_hi = min(ih0 + nrow_in - 1, p.H - 1);
    const int colsR = p.Wd + 2 * p.pw;  // staged columns, padding included
    const int rowL = p.colsL * kPixL;

    // K slot (slice s, lane row g) -> tap, and whether it carries the tap's
    // weights or zeros.  Plain order: tap 4s + g, zeros past the ninth.
    // Paired order (4 bits a slot): slice 0 taps 0 6 1 7, slice 1 2 8 3 3,
    // slice 2 4 4 5 5, the second 3, 4 and 5 with zero weights.
    constexpr int kPairTaps[kSlices] = {0x7160, 0x3382, 0x5544};
    constexpr int kPairReal[kSlices] = {0xF, 0x7, 0x5};
    const bool pairs = S == 1 && p.tap_pairs;
    auto slot_tap = [&](int s) {
        return pairs ? (kPairTaps[s] >> (4 * g)) & 15 : min(4 * s + g, KK - 1);
    };
    auto slot_real = [&](int s) { return pairs ? ((kPairReal[s] >> g) & 1) != 0 : 4 * s + g < KK; };

    // ---- per-channel parameters and this lane's weight bytes, loaded
    //      behind the input rows (issued first, the compiler waited for
    //      them before the input loads could go); the diagonal operands are
    //      built from the bytes after the barrier ----
    // Unconditional loads at clamped indices, the raw values kept untouched
    // until after the barrier (a load under a branch, or a value used at
    // once, makes the compiler wait for the input loads issued before it).
    int bv, mv, sv;
    int wb[kSlices][4];
    auto load_params = [&]() {
        const int cc = c0 + min(tid, cs - 1);
        bv = (p.bias ? p.bias : p.mult)[cc];
        mv = p.mult[cc];
        sv = p.shift[cc];
#pragma unroll
        for (int s = 0; s < kSlices; ++s)
#pragma unroll
            for (int n = 0; n < 4; ++n)
                wb[s][n] = (uint8_t)p.W[(int64_t)slot_tap(s) * p.C + c0 + min(16 * n, cs - 16) +
                                        col];
    };

    // ---- input rows (the slice's channels) -> LDS, the padding value
    //      outside the image ----
    const int gpp = cs >> 4;  // 16-byte granules per pixel
    const int total = ih_lo <= ih_hi ? (ih_hi - ih_lo + 1) * p.Wd * gpp : 0;
    constexpr int kPass = 8 * kWaves * 64;  // granules of one pass (8 loads per thread)
    auto src_of = [&](int j) {
        const int pix = j / gpp, q = j - pix * gpp;  // pix over rows ih_lo.. x Wd
        const int64_t src = ((int64_t)b * p.H + ih_lo) * p.Wd + pix;
        return p.X + src * p.C + c0 + 16 * q;
    };
    auto put = [&](int j, const v4i &v) {
        const int pix = j / gpp, q = j - pix * gpp;
        const int rr = pix / p.Wd, iw = pix - rr * p.Wd;
        const int r = ih_lo - ih0 + rr;
        *(v4i *)(IN + r * rowL + (iw + p.pw) * kPixL + 16 * q) = v;
    };
    auto pad_rows = [&]() {
        for (int e = tid; e < nrow_in * colsR; e += kWaves * 64) {
            const int r = e / colsR, c = e - r * colsR;
            const int ih = ih0 + r;
            if (ih < 0 || ih >= p.H || c < p.pw || c >= p.pw + p.Wd) {
                v4i *z = (v4i *)(IN + r * rowL + c * kPixL);
                z[0] = z[1] = z[2] = z[3] = (v4i){p.pad4, p.pad4, p.pad4, p.pad4};
            } else if (cs < kCS) {
                // channels past the slice meet zero weights; keep them finite
                for (int q = gpp; q < 4; ++q)
                    *(v4i *)(IN + r * rowL + c * kPixL + 16 * q) = (v4i){0, 0, 0, 0};
            }
        }
    };
    if (total > 0 && total <= kPass) {
        // one pass, straight-line, every load and LDS write unconditional (a
        // granule past the end is the last one again, rewritten in place)
        v4i v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            v[k] = *(const v4i *)src_of(min(k * kWaves * 64 + tid, total - 1));
        load_params();
        pad_rows();
#pragma unroll
        for (int k = 0; k < 8; ++k)
            put(min(k * kWaves * 64 + tid, total - 1), v[k]);
    } else {
        load_params();
        for (int base = 0; base == 0 || base < total; base += kPass) {
            v4i v[8];
            if (total > 0) {
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    v[k] = *(const v4i *)src_of(min(base + k * kWaves * 64 + tid, total - 1));
            }
            if (base == 0)
                pad_rows();
            if (total > 0) {
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int j = base + k * kWaves * 64 + tid;
                    if (j < total)
                        put(j, v[k]);
                }
            }
        }
    }
    drain_and_barrier();
    if (tid < kCS) {
        const bool in = tid < cs;  // channels past the slice: 0, 0, 31
        prm[tid] = in && p.bias ? bv : 0;
        prm[kCS + tid] = in ? mv : 0;
        prm[2 * kCS + tid] = in ? sv : 31;
    }
    __syncthreads();

    // ---- diagonal weight operands: slice s, group n; the lane (column
    //      col = output channel 16n + col, K group g = tap t of slot (s, g))
    //      holds w[t][c0 + 16n + col] at byte col of 16, or 0 ----
    v4i wd[kSlices][4];
#pragma unroll
    for (int s = 0; s < kSlices; ++s)
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            v4i v = {0, 0, 0, 0};
            const int w = slot_real(s) && 16 * n < cs ? wb[s][n] : 0;
#pragma unroll
            for (int d = 0; d < 4; ++d)
                v[d] = (col >> 2) == d ? (w << (8 * (col & 3))) : 0;
            wd[s][n] = v;
        }

    // ---- this lane's pixel in each of the wave's M tiles (LDS offset of
    //      its (0, 0) tap) and its tap in each slice ----
    int abase[kTPW];
#pragma unroll
    for (int i = 0; i < kTPW; ++i) {
        const int q = min(16 * (wave + kWaves * i) + col, npix - 1);
        const int pp = p0 + q;
        const int oh = pp / p.Wo;
        const int ow = pp - oh * p.Wo;
        abase[i] = (oh - oh_first) * S * rowL + ow * S * kPixL;
    }
    int toff[kSlices];
#pragma unroll
    for (int s = 0; s < kSlices; ++s) {
        const int t = slot_tap(s);
        toff[s] = (t / KW) * rowL + (t % KW) * kPixL;
    }

    v4i acc[kTPW][4];
#pragma unroll
    for (int i = 0; i < kTPW; ++i)
#pragma unroll
        for (int n = 0; n < 4; ++n)
            acc[i][n] = (v4i){0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < kSlices; ++s) {
        v4i a[kTPW][4];
#pragma unroll
        for (int i = 0; i < kTPW; ++i)
#pragma unroll
            for (int n = 0; n < 4; ++n)
                if (i < kTPW - 1 || has_last)
                    a[i][n] = *(const v4i *)(IN + abase[i] + toff[s] + 16 * n);
#pragma unroll
        for (int i = 0; i < kTPW; ++i) {
            if (i == kTPW - 1 && !has_last)
                continue;
#pragma unroll
            for (int n = 0; n < 4; ++n)
                acc[i][n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wd[s][n], a[i][n], acc[i][n],
                                                                 0, 0, 0);
        }
    }

    // ---- requantize; lane holds pixel 16*(wave + 8*i) + col and channels
    //      16*n + 4*g + e of the slice.  A 4 x 4 transpose across the four
    //      16-lane rows (v_permlane32_swap, then v_permlane16_swap) gives
    //      lane row g channels 16g .. 16g+15, written with one 16-byte store
    //      when the slice has them ----
    const int sh_l = prm[2 * kCS + lane];
    int8_t *ybase = p.Y + ((int64_t)b * HW + p0) * p.C + c0 + 16 * g;
    auto requant_tile = [&](auto tier_tag) {
        constexpr int TIER = decltype(tier_tag)::value;
#pragma unroll
        for (int i = 0; i < kTPW; ++i) {
            if (i == kTPW - 1 && !has_last)
                continue;
            unsigned x[4];
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const int cc = 16 * n + 4 * g;
                const v4i b4 = *(const v4i *)&prm[cc];
                const v4i m4 = *(const v4i *)&prm[kCS + cc];
                const v4i s4 = *(const v4i *)&prm[2 * kCS + cc];
                int y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int xa = acc[i][n][e];
                    const int zo = ZP ? p.out_zero : 0;
                    const int lo = ZP ? p.act_min : -128, hi = ZP ? p.act_max : 127;
                    if constexpr (TIER == 2)
                        y[e] = requant_one_s33(xa, b4[e], m4[e], s4[e], zo, lo, hi);
                    else if constexpr (TIER == 1)
                        y[e] = requant_one_s31(xa, b4[e], m4[e], s4[e], 1ll << ((s4[e] - 1) & 63),
                                               zo, lo, hi);
                    else
                        y[e] = requant_one(xa, b4[e], m4[e], s4[e], 1ll << ((s4[e] - 1) & 63), zo,
                                           lo, hi);
                }
                x[n] = pack4_i8(y[0], y[1], y[2], y[3]);
            }
            const auto r02 = __builtin_amdgcn_permlane32_swap(x[0], x[2], false, false);
            const auto r13 = __builtin_amdgcn_permlane32_swap(x[1], x[3], false, false);
            const auto r01 = __builtin_amdgcn_permlane16_swap(r02[0], r13[0], false, false);
            const auto r23 = __builtin_amdgcn_permlane16_swap(r02[1], r13[1], false, false);
            const v4i out = {(int)r01[0], (int)r01[1], (int)r23[0], (int)r23[1]};
            const int q = 16 * (wave + kWaves * i) + col;
            if (q < npix && g < ngrp)
                *(v4i *)(ybase + (int64_t)q * p.C) = out;
        }
    };
    // parameters of channels past the slice read as shift 31 (a valid value)
    if (__builtin_amdgcn_ballot_w64(sh_l < 33) == 0)
        requant_tile(std::integral_constant<int, 2>{});
    else if (__builtin_amdgcn_ballot_w64(sh_l < 31) == 0)
        requant_tile(std::integral_constant<int, 1>{});
    else
        requant_tile(std::integral_constant<int, 0>{});
}

// ---- any kernel size and stride: one thread per output pixel x 4 channels;
//      the asymmetric form multiplies (x - za) * (w - zb) directly, so a
//      padded tap (x = za) adds nothing and `bias` is the plain bias ----
__global__ __launch_bounds__(256) void k_dwconv_direct(DwArgs p, int64_t nitems)
{
    const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (item >= nitems)
        return;
    const int cq = p.C >> 2;
    const int64_t pix = item / cq;
    const int c = (int)(item - pix * cq) * 4;
    const int HW = p.Ho * p.Wo;
    const int b = (int)(pix / HW);
    const int rem = (int)(pix - (int64_t)b * HW);
    const int oh = rem / p.Wo, ow = rem - (rem / p.Wo) * p.Wo;
    int acc[4] = {0, 0, 0, 0};
    for (int kh = 0; kh < p.KH; ++kh) {
        const int ih = oh * p.sh - p.ph + kh;
        if (ih < 0 || ih >= p.H)
            continue;
        for (int kw = 0; kw < p.KW; ++kw) {
            const int iw = ow * p.sw - p.pw + kw;
            if (iw < 0 || iw >= p.Wd)
                continue;
            const unsigned xv = *(const unsigned *)(p.X + (((int64_t)b * p.H + ih) * p.Wd + iw) * p.C + c);
            const unsigned wv = *(const unsigned *)(p.W + (int64_t)(kh * p.KW + kw) * p.C + c);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc[e] = wrap_add(acc[e], ((int)(int8_t)(xv >> (8 * e)) - p.a_zero) *
                                              ((int)(int8_t)(wv >> (8 * e)) - p.b_zero));
        }
    }
    int y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int s = p.shift[c + e];
        y[e] = requant_one(acc[e], p.bias ? p.bias[c + e] : 0, p.mult[c + e], s,
                           1ll << ((s - 1) & 63), p.out_zero, p.act_min, p.act_max);
    }
    *(unsigned *)(p.Y + pix * p.C + c) = pack4_i8(y[0], y[1], y[2], y[3]);
}

// LDS bytes of the staged input rows for a 3x3 conv with stride S and
// `cols` pixels per LDS row: the output rows a tile of kTP consecutive
// pixels touches (never more than the image has), times S, plus the halo;
// rounded to 1 KB.
int64_t dw_in_bytes(const ConvDesc &d, int64_t cols)
{
    const int64_t span = std::min<int64_t>((kTP - 1) / d.Wo + 1, d.Ho - 1);
    const int64_t rows = span * d.sh + d.KH;
    int64_t in = rows * cols * kPixL;
    return (in + 1023) & ~(int64_t)1023;
}

// LDS pixels per staged row: the padded width, or with stride 1 the next
// count congruent to Wo mod 16 (when that still fits), so that 16
// consecutive output pixels take 16 bank groups across a row end too
int64_t dw_cols(const ConvDesc &d)
{
    const int64_t base = d.Wd + 2 * d.pw;
    if (d.sh == 1) {
        const int64_t cols = base + (((d.Wo - base) % 16) + 16) % 16;
        if (dw_in_bytes(d, cols) + 3 * kCS * 4 <= kMaxLds)
            return cols;
    }
    return base;
}

int64_t dw_lds_bytes(const ConvDesc &d)
{
    return dw_in_bytes(d, dw_cols(d)) + 3 * kCS * 4;
}

bool dw_mfma_fits(const ConvDesc &d)
{
    if (d.KH != 3 || d.KW != 3 || d.sh != d.sw || (d.sh != 1 && d.sh != 2))
        return false;
    return d.C_in % 16 == 0 && dw_lds_bytes(d) <= kMaxLds;
}

template <int S, bool ZP>
hipError_t run_dw3x3(const DwArgs &a, int batch, int lds_bytes, hipStream_t s)
{
    static std::atomic<bool> attr_set[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    if (!attr_set[dev].load(std::memory_order_acquire)) {
        e = hipFuncSetAttribute((const void *)k_dwconv3x3<S, ZP>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
        if (e != hipSuccess)
            return e;
        attr_set[dev].store(true, std::memory_order_release);
    }
    const dim3 grid(batch * a.tiles_per_img, (a.C + kCS - 1) / kCS), block(kWaves * 64);
    hipLaunchKernelGGL((k_dwconv3x3<S, ZP>), grid, block, lds_bytes, s, a);
    return hipGetLastError();
}

}  // namespace

bool dw_takes_mfma(const ConvDesc &d)
{
    return dw_mfma_fits(d) && (!d.asym || d.b_zero == 0);
}

// The asymmetric 3x3 path reads `bias` as bias - za * sum_t w[t][c]
// (launch_zp_dw_terms); the direct path takes the plain bias.
hipError_t launch_dwconv_nhwc(const ConvDesc &d, hipStream_t s)
{
    DwArgs a{};
    a.X = d.X;
    a.W = d.W;
    a.bias = d.bias;
    a.mult = d.mult;
    a.shift = d.shift;
    a.Y = d.Y;
    a.H = d.H;
    a.Wd = d.Wd;
    a.C = d.C_in;
    a.KH = d.KH;
    a.KW = d.KW;
    a.sh = d.sh;
    a.sw = d.sw;
    a.ph = d.ph;
    a.pw = d.pw;
    a.Ho = d.Ho;
    a.Wo = d.Wo;
    a.act_min = -128;
    a.act_max = 127;
    if (d.asym) {
        a.pad4 = (int)(0x01010101u * (uint8_t)d.a_zero);
        a.a_zero = d.a_zero;
        a.b_zero = d.b_zero;
        a.out_zero = d.out_zero;
        a.act_min = d.act_min;
        a.act_max = d.act_max;
    }
    if (dw_takes_mfma(d)) {
        a.tiles_per_img = (d.Ho * d.Wo + kTP - 1) / kTP;
        a.colsL = (int)dw_cols(d);
        a.in_bytes = (int)dw_in_bytes(d, a.colsL);
        // the paired tap order needs taps two row pitches apart on one
        // bank group: stride 1, a pitch congruent to Wo, and 2 Wo = 0 mod 16
        a.tap_pairs = d.sh == 1 && d.Wo % 8 == 0 && (a.colsL - d.Wo) % 16 == 0;
        const int lds = (int)dw_lds_bytes(d);
        if (d.asym)
            return d.sh == 1 ? run_dw3x3<1, true>(a, d.batch, lds, s)
                             : run_dw3x3<2, true>(a, d.batch, lds, s);
        return d.sh == 1 ? run_dw3x3<1, false>(a, d.batch, lds, s)
                         : run_dw3x3<2, false>(a, d.batch, lds, s);
    }
    const int64_t nitems = (int64_t)d.batch * d.Ho * d.Wo * (d.C_in / 4);
    const int64_t blocks = (nitems + 255) / 256;
    hipLaunchKernelGGL(k_dwconv_direct, dim3((unsigned)blocks), dim3(256), 0, s, a, nitems);
    return hipGetLastError();
}

}  // namespace qg
