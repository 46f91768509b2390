// k_conv_halo.hip -- NHWC int8 conv with stride 1 and 64 input channels,
// the input rows of a tile staged once in LDS, Q31 requantize fused.
//
// Method: the conv is a GEMM over an im2col matrix whose rows are output
// pixels and whose K runs over (tap, input channel) (MCU conv front-end
// article, news.rkmt.cn/news/16638, §3.2; geometry and zero padding §2.1,
// §2.3; NHWC input and OHWI weights §3.1).  Walking K tap by tap makes the
// 3x3 conv nine 1x1 convs over shifted inputs (Groq ResNet50 compilation
// article, www.pwwt.cn/news/1982903, §2.1).  Nothing is materialized: every
// tap reads the same input rows, so a workgroup stages those rows in LDS
// once and reads all taps from there.
//
// Per workgroup (8 waves, one workgroup per CU): 392 consecutive output
// pixels of one image (7 rows of a 56-wide image: 32 images x 8 bands make
// one workgroup per CU of an MI355X) times 64 output channels.
//   * the input rows those pixels touch (with the KH-1 halo rows) are read
//     once with 16-byte loads and written to LDS with every pixel in 80
//     bytes (64 channels + 16 unused), row by row with padding columns on
//     both sides and padding rows above and below the image, filled with
//     the input zero point (0 for symmetric inputs): a tap of an output pixel
//     is then one fixed LDS offset away from its (0, 0) tap, with no bounds
//     test, and the padding costs nothing;
//   * the LDS is read with 16-byte reads, which gfx950 serves 16 lanes per
//     cycle over 64 4-byte banks, the 16 lanes of a cycle being those that
//     share lane bit 5 and the parity of lane bits 2..4 (measured).  Three
//     choices make every operand read conflict free: an LDS row pitch that
//     is congruent to Wo pixels modulo 256 bytes (so the bank of a pixel
//     follows its linear index across row ends), lane row g taking channel
//     chunk (0, 2, 1, 3)[g] (both operands, so the K pairing is kept), and,
//     within each 16-pixel MFMA tile, the lane quads that share a cycle
//     taking the odd and the even pixels respectively;
//   * the workgroup's 64 weight rows (KH*KW*64 bytes each, OHWI) are copied
//     with direct-to-LDS loads (global_load_lds_dwordx4, 1 KB of contiguous
//     bytes per wave instruction), weight granule G of row oc stored at
//     G ^ ((oc >> 3) & 1), which with the chunk order above spreads each read
//     cycle over all 16 bank groups;
//   * with 64 input channels one tap is exactly one K step of
//     v_mfma_i32_16x16x64_i8: weights are the first operand (rows = output
//     channels), pixels the second; the band's 25 16-pixel tiles go to the
//     waves in turn (wave w takes tiles w, w + 8, w + 16, and wave 0 also
//     tile 24), so a SIMD multiplies 6 or 7 tiles x 64 channels, and the
//     operands of tap t+1 are read from LDS while tap t is multiplied;
//   * the requantize uses the cheapest exact form that all 64 shifts of the
//     workgroup allow.  A lane holds 4 channels of one pixel per MFMA tile;
//     a 4 x 4 transpose across the four 16-lane rows (v_permlane32_swap,
//     then v_permlane16_swap) gives it 16 consecutive channels, written with
//     one 16-byte store (1 KB contiguous per wave instruction when
//     C_out == 64).
// Measured on conv3x3 32x56x56x64->64 against 256-pixel, 4-wave
// workgroups two to a CU (416 workgroups: 160 CUs ran two, the rest one):
// 8.2 vs 8.8 us, and 10.0 vs 11.3 us with zero points.  With one wave per
// SIMD instead (7 tiles each) the band is slower than either (9.1 us): the
// second wave hides the LDS latency.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "dev_common.hpp"
#include "launch.hpp"

namespace qg {

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

constexpr int kTP = 392;     // output pixels per workgroup (7 rows of a 56-wide image)
constexpr int kTiles = (kTP + 15) / 16;  // 16-pixel MFMA tiles per workgroup (25)
constexpr int kNT = 64;      // output channels per workgroup
constexpr int kCin = 64;     // input channels = bytes per input pixel
constexpr int kPixL = 80;    // LDS bytes per staged input pixel
constexpr int kWaves = 8;    // two waves per SIMD
constexpr int kTPW = (kTiles + kWaves - 1) / kWaves;  // MFMA tiles per wave: w, w + 8, ... < kTiles
constexpr int kMaxLds = 160 * 1024;  // one workgroup per CU
constexpr int kMaxDevices = 64;

struct HaloArgs {
    const int8_t *X;
    const int8_t *W;
    const int32_t *bias;
    const int32_t *mult;
    const int32_t *shift;
    int8_t *Y;
    int H, Wd, C_out, ph, pw, Ho, Wo;
    int tiles_per_img;
    int in_bytes;  // LDS bytes of the staged input rows
    int rowL;      // LDS bytes of one staged input row
    int pad4;                  // padding byte (the input zero point) x4
    int a_zero, b_zero, out_zero;  // ZP: the zero points
    int act_min, act_max;          // ZP: output clamp bounds
};

__device__ __forceinline__ void drain_and_barrier()
{
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ZP: the asymmetric form.  The kernel forms both compensation terms itself:
// the per-pixel sum of its im2col row (padding counted as za) from the
// operand fragments it multiplies, and the per-channel weight sum from the
// weight rows in LDS; x = acc - zb * rowsum + (bias - za * wsum + K za zb),
// modulo 2^32.  The output zero point joins before the saturation.
template <int KH, int KW, bool ZP>
__global__ __launch_bounds__(kWaves * 64, 1) void k_conv_halo(HaloArgs p)
{
    constexpr int KK = KH * KW;
    constexpr int kRowW = KK * kCin;  // bytes of one weight row (one output channel)
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    uint8_t *IN = lds;
    uint8_t *WT = lds + p.in_bytes;
    int *prm = (int *)(WT + kNT * kRowW);  // bias, mult, shift [3][64]

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
    const int n0 = blockIdx.y * kNT;
    const int oh_first = p0 / p.Wo, oh_last = (p0 + npix - 1) / p.Wo;
    const int ih0 = oh_first - p.ph;  // input row of LDS row 0
    const int ih_lo = max(ih0, 0), ih_hi = min(oh_last - p.ph + KH - 1, p.H - 1);
    const int rowB = p.Wd * kCin;

    // ---- per-channel parameters, loaded ahead of the bulk copies ----
    int pb = 0, pm = 0, ps = 0;
    if (tid < kNT) {
        pb = p.bias ? p.bias[n0 + tid] : 0;
        pm = p.mult[n0 + tid];
        ps = p.shift[n0 + tid];
    }

    // ---- weight rows n0..n0+63 (OHWI, contiguous) -> LDS ----
    {
        const int8_t *src = p.W + (int64_t)n0 * kRowW;
        constexpr int npieces = kNT * kRowW / 1024;
        for (int P = wave; P < npieces; P += kWaves) {
            const int pos = P * 1024 + 16 * lane;
            const int oc = pos / kRowW;
            const int G = (pos - oc * kRowW) >> 4;
            const int sG = G ^ ((oc >> 3) & 1);
            __builtin_amdgcn_global_load_lds((const glb_void_t *)(src + oc * kRowW + 16 * sG),
                                             (lds_void_t *)(WT + P * 1024), 16, 0, 0);
        }
    }

    // ---- input rows: LDS row r holds input row ih0 + r, LDS column c holds
    //      input column c - pw; the padding value outside the image ----
    const int colsL = p.Wd + 2 * p.pw;
    const int rowL = p.rowL;
    const int nrow_in = oh_last - oh_first + KH;  // LDS rows this tile reads
    // rows ih_lo..ih_hi are one contiguous NHWC span of 16-byte granules;
    // a thread loads up to 8 of them per pass (loads past the end read the
    // last granule and are not written), and the zero padding is written
    // while the first pass is in flight
    const int total = ih_lo <= ih_hi ? (ih_hi - ih_lo + 1) * p.Wd * 4 : 0;
    const int8_t *src = p.X + ((int64_t)b * p.H + ih_lo) * rowB;
    const int gpr = p.Wd * 4;  // granules per input row
    for (int base = 0; base == 0 || base < total; base += 8 * kWaves * 64) {
        v4i v[8];
        if (total > 0) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int j = min(base + k * kWaves * 64 + tid, total - 1);
                v[k] = *(const v4i *)(src + 16 * (int64_t)j);
            }
        }
        if (base == 0) {
            for (int e = tid; e < nrow_in * colsL; e += kWaves * 64) {
                const int r = e / colsL, c = e - r * colsL;
                const int ih = ih0 + r;
                if (ih < 0 || ih >= p.H || c < p.pw || c >= p.pw + p.Wd) {
                    v4i *z = (v4i *)(IN + r * rowL + c * kPixL);
                    z[0] = z[1] = z[2] = z[3] = (v4i){p.pad4, p.pad4, p.pad4, p.pad4};
                }
            }
        }
        if (total > 0) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int j = base + k * kWaves * 64 + tid;
                if (j < total) {
                    const int rr = j / gpr, rem = j - rr * gpr;
                    const int r = ih_lo - ih0 + rr;
                    *(v4i *)(IN + r * rowL + ((rem >> 2) + p.pw) * kPixL + 16 * (rem & 3)) = v[k];
                }
            }
        }
    }
    drain_and_barrier();
    if (tid < kNT) {
        prm[tid] = pb;
        prm[kNT + tid] = pm;
        prm[2 * kNT + tid] = ps;
    }
    __syncthreads();

    // ---- this lane's pixel in each of the wave's 4 M tiles, as the LDS
    //      offset of its (0, 0) tap; pixels past the tile reuse the last one ----
    // lane column col stands for pixel pcol of each 16-pixel tile, and lane
    // row g for channel chunk chk (both bank-conflict choices above)
    const int pcol = 2 * (col & 7) + ((((col >> 2) ^ (col >> 3)) & 1) ? 0 : 1);
    const int chk = ((g & 1) << 1) | (g >> 1);
    int abase[kTPW];
#pragma unroll
    for (int i = 0; i < kTPW; ++i) {
        const int q = min(16 * (wave + kWaves * i) + pcol, npix - 1);
        const int pp = p0 + q;
        const int oh = pp / p.Wo;
        const int ow = pp - oh * p.Wo;
        abase[i] = (oh - oh_first) * rowL + ow * kPixL + 16 * chk;
    }

    // ZP: per-channel weight sums of the 64 weight rows in LDS, four threads
    // per row; the bias slot of prm becomes bias - za * wsum + K * za * zb
    if (ZP && tid < 4 * kNT) {
        const int oc = tid >> 2, part = tid & 3;
        unsigned ws = 0;
        for (int G = part; G < KK * 4; G += 4) {
            const v4i v = *(const v4i *)(WT + oc * kRowW + 16 * G);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ws = (unsigned)__builtin_amdgcn_sdot4(v[e], 0x01010101, (int)ws, false);
        }
        ws += (unsigned)__shfl_xor((int)ws, 1);
        ws += (unsigned)__shfl_xor((int)ws, 2);
        if (part == 0)
            prm[oc] = (int)((unsigned)prm[oc] - (unsigned)p.a_zero * ws +
                            (unsigned)(KK * kCin) * (unsigned)(p.a_zero * p.b_zero));
    }
    // every wave's requantize reads all 64 adjusted biases
    if constexpr (ZP)
        __syncthreads();

    v4i acc[kTPW][4];
#pragma unroll
    for (int i = 0; i < kTPW; ++i)
#pragma unroll
        for (int n = 0; n < 4; ++n)
            acc[i][n] = (v4i){0, 0, 0, 0};
    unsigned rs[kTPW] = {};  // ZP: this lane's 16 channels of each pixel's im2col row

    v4i a[2][kTPW], w[2][4];
    auto read_tap = [&](int t, v4i(&at)[kTPW], v4i(&wt)[4]) {
        const int kh = t / KW, kw = t - (t / KW) * KW;
        const int toff = kh * rowL + kw * kPixL;
#pragma unroll
        for (int i = 0; i < kTPW; ++i)
            if (i < kTPW - 1 || has_last)
                at[i] = *(const v4i *)(IN + abase[i] + toff);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int oc = 16 * n + col;
            const int G = 4 * t + chk;
            wt[n] = *(const v4i *)(WT + oc * kRowW + ((G ^ ((oc >> 3) & 1)) << 4));
        }
    };
    read_tap(0, a[0], w[0]);
#pragma unroll
    for (int t = 0; t < KK; ++t) {
        if (t + 1 < KK)
            read_tap(t + 1, a[(t + 1) & 1], w[(t + 1) & 1]);
#pragma unroll
        for (int i = 0; i < kTPW; ++i) {
            if (i == kTPW - 1 && !has_last)
                continue;
#pragma unroll
            for (int n = 0; n < 4; ++n)
                acc[i][n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[t & 1][n], a[t & 1][i],
                                                                 acc[i][n], 0, 0, 0);
        }
        if constexpr (ZP) {
#pragma unroll
            for (int i = 0; i < kTPW; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    rs[i] = (unsigned)__builtin_amdgcn_sdot4(a[t & 1][i][e], 0x01010101,
                                                             (int)rs[i], false);
        }
    }
    // ZP: the four K groups of a pixel sit in lanes col, col + 16, col + 32,
    // col + 48; after the sum every one of them holds zb * (its im2col row sum)
    int rt[kTPW] = {};
    if constexpr (ZP) {
#pragma unroll
        for (int i = 0; i < kTPW; ++i) {
            unsigned v = rs[i];
            v += (unsigned)__shfl_xor((int)v, 16);
            v += (unsigned)__shfl_xor((int)v, 32);
            rt[i] = (int)((unsigned)p.b_zero * v);
        }
    }

    // ---- requantize; lane holds pixel pcol of M tile i and channels
    //      16*n + 4*g + e; the form is chosen once for the tile's 64
    //      channels ----
    const int sh_l = prm[2 * kNT + lane];
    int8_t *ybase = p.Y + ((int64_t)b * HW + p0) * p.C_out + n0 + 16 * g;
    auto requant_tile = [&](auto tier_tag) {
        constexpr int TIER = decltype(tier_tag)::value;
#pragma unroll
        for (int i = 0; i < kTPW; ++i) {
            if (i == kTPW - 1 && !has_last)
                continue;
            unsigned x[4];
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const int c0 = 16 * n + 4 * g;
                const v4i b4 = *(const v4i *)&prm[c0];
                const v4i m4 = *(const v4i *)&prm[kNT + c0];
                const v4i s4 = *(const v4i *)&prm[2 * kNT + c0];
                int y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int xa = ZP ? wrap_sub(acc[i][n][e], rt[i]) : acc[i][n][e];
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
            // 4 x 4 transpose over the lane rows: row g receives dword g of
            // rows 0..3, i.e. channels 16g .. 16g+15 in order
            const auto r02 = __builtin_amdgcn_permlane32_swap(x[0], x[2], false, false);
            const auto r13 = __builtin_amdgcn_permlane32_swap(x[1], x[3], false, false);
            const auto r01 = __builtin_amdgcn_permlane16_swap(r02[0], r13[0], false, false);
            const auto r23 = __builtin_amdgcn_permlane16_swap(r02[1], r13[1], false, false);
            const v4i out = {(int)r01[0], (int)r01[1], (int)r23[0], (int)r23[1]};
            const int q = 16 * (wave + kWaves * i) + pcol;
            if (q < npix)
                *(v4i *)(ybase + (int64_t)q * p.C_out) = out;
        }
    };
    if (__builtin_amdgcn_ballot_w64(sh_l < 33) == 0)
        requant_tile(std::integral_constant<int, 2>{});
    else if (__builtin_amdgcn_ballot_w64(sh_l < 31) == 0)
        requant_tile(std::integral_constant<int, 1>{});
    else
        requant_tile(std::integral_constant<int, 0>{});
}

template <int KH, int KW, bool ZP>
hipError_t run_halo(const HaloArgs &a, int batch, int lds_bytes, hipStream_t s)
{
    // the dynamic LDS limit above 64 KB is raised once per device
    static std::atomic<bool> attr_set[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    if (!attr_set[dev].load(std::memory_order_acquire)) {
        e = hipFuncSetAttribute((const void *)k_conv_halo<KH, KW, ZP>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
        if (e != hipSuccess)
            return e;
        attr_set[dev].store(true, std::memory_order_release);
    }
    const dim3 grid(batch * a.tiles_per_img, a.C_out / kNT), block(kWaves * 64);
    hipLaunchKernelGGL((k_conv_halo<KH, KW, ZP>), grid, block, lds_bytes, s, a);
    return hipGetLastError();
}

// LDS rows of the input region: the most output rows a tile of kTP
// consecutive pixels touches (never more than the image has), plus the
// KH-1 halo rows.
int halo_rows(const ConvDesc &d)
{
    return std::min((kTP - 1) / d.Wo + 2, d.Ho) + d.KH - 1;
}

// LDS bytes of one staged input row: Wd + 2*pw pixels of kPixL bytes, plus
// the padding that makes the pitch congruent to Wo pixels modulo 256 bytes
int halo_row_bytes(const ConvDesc &d)
{
    const int colsL = d.Wd + 2 * d.pw;
    const int pad = (((d.Wo - colsL) * kPixL) % 256 + 256) % 256;
    return colsL * kPixL + pad;
}

// LDS bytes of the input-row region, rounded up to 1 KB so that the weight
// rows start aligned.
int64_t halo_in_bytes(const ConvDesc &d)
{
    const int64_t in = (int64_t)halo_rows(d) * halo_row_bytes(d);
    return (in + 1023) & ~(int64_t)1023;
}

int64_t halo_lds_bytes(const ConvDesc &d)
{
    return halo_in_bytes(d) + (int64_t)kNT * d.KH * d.KW * kCin + 3 * kNT * 4;
}

}  // namespace

bool conv_halo_fits(const ConvDesc &d)
{
    if (d.sh != 1 || d.sw != 1 || d.C_in != kCin || d.C_out % kNT != 0)
        return false;
    if (!((d.KH == 3 && d.KW == 3) || (d.KH == 1 && d.KW == 1)))
        return false;
    return halo_lds_bytes(d) <= kMaxLds;
}

hipError_t launch_conv_halo(const ConvDesc &d, hipStream_t s)
{
    HaloArgs a{};
    a.X = d.X;
    a.W = d.W;
    a.bias = d.bias;
    a.mult = d.mult;
    a.shift = d.shift;
    a.Y = d.Y;
    a.H = d.H;
    a.Wd = d.Wd;
    a.C_out = d.C_out;
    a.ph = d.ph;
    a.pw = d.pw;
    a.Ho = d.Ho;
    a.Wo = d.Wo;
    a.tiles_per_img = (d.Ho * d.Wo + kTP - 1) / kTP;
    a.in_bytes = (int)halo_in_bytes(d);
    a.rowL = halo_row_bytes(d);
    a.pad4 = (int)(0x01010101u * (uint8_t)d.a_zero);
    a.a_zero = d.a_zero;
    a.b_zero = d.b_zero;
    a.out_zero = d.out_zero;
    a.act_min = d.act_min;
    a.act_max = d.act_max;
    const int lds = (int)halo_lds_bytes(d);
    if (d.asym) {
        if (d.KH == 3)
            return run_halo<3, 3, true>(a, d.batch, lds, s);
        return run_halo<1, 1, true>(a, d.batch, lds, s);
    }
    if (d.KH == 3)
        return run_halo<3, 3, false>(a, d.batch, lds, s);
    return run_halo<1, 1, false>(a, d.batch, lds, s);
}

}  // namespace qg
