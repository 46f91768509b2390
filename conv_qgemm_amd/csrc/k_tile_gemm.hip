// k_tile_gemm.hip -- tiled int8/int4 GEMM on the gfx950 int8 MFMA, with the
// per-channel Q31 requantize (or a raw int32 store) fused into the
// accumulator writeback.  The same kernel runs an NHWC conv as an implicit
// GEMM by swapping in an im2col operand loader.
//
// Method (pages and sections): C = A * B with int8 or packed int4 inputs and
// int32 accumulation (INT4 GEMM article, www.cf-1.com/news/6060138, §3.2);
// B column-major (same, §4.3); requantize of the MCU conv front-end article
// (news.rkmt.cn/news/16638) §2.3; conv as C = A x B over the im2col matrix
// (same, §3.2), with zero-point-0 padding (§2.3) and the K loop walking the
// taps as shifted 1x1 products (Groq TSP ResNet50 article,
// www.pwwt.cn/news/1982903, §2.1).
//
// Structure of one workgroup (256 threads = 4 waves of 64):
//   * output tile BM x BN, waves arranged WGM x WGN, each wave owning a
//     (BM/WGM) x (BN/WGN) block of 32x32 MFMA sub-tiles;
//   * K walked in tiles of KT values: the next tile's 16-byte chunks are
//     fetched global->VGPR while the current one is multiplied out of LDS,
//     then written to the other LDS buffer (two buffers, one barrier per
//     K tile);
//   * LDS rows hold 16-byte chunks XOR-swizzled by the row index, so the 32
//     rows read by one MFMA operand fetch land in different banks;
//   * operands go to v_mfma_i32_32x32x32_i8 with the B fragment as the
//     instruction's first source, so each lane ends up holding 4 adjacent
//     output columns of one output row: the epilogue packs 4 int8 results
//     into one dword store (or 4 int32 into one 16-byte store);
//   * workgroup ids are renumbered so neighbouring tiles share an XCD's L2,
//     and tiles are walked in groups of GROUP_M tile-rows.
#include "dev_common.hpp"
#include "launch.hpp"

namespace qg {

enum { OP_S8 = 8, OP_S4 = 4 };
// EPI_REQUANT_ZP is the asymmetric form: `bias` holds the per-column term
// (bias - za * sum_k B + K * za * zb), `rterm` the per-row zb * sum_k A (null
// when zb = 0), and the output zero point joins before the saturation; the
// sums wrap modulo 2^32 and give the true value whenever it fits in int32.
// EPI_F16: binary16 output, fp16(fp32(acc) * scale_a[m] * scale_b[n]).
enum { EPI_REQUANT = 0, EPI_I32 = 1, EPI_REQUANT_ZP = 2, EPI_F16 = 3 };
enum { AL_DENSE = 0, AL_CONV = 1 };

struct TileArgs {
    const uint8_t *A;
    int64_t lda_b;
    const uint8_t *B;
    int64_t ldb_b;
    const int32_t *bias;
    const int32_t *mult;
    const int32_t *shift;
    void *C;
    int64_t ldc;
    int M, N, K;
    int tiles_m, tiles_n;
    // implicit-im2col geometry (AL_CONV only)
    int H, W, C_in, KW, Ho, Wo, sh, sw, ph, pw;
    int pad4;              // AL_CONV: padding byte (the input zero point) x4
    const int32_t *rterm;  // EPI_REQUANT_ZP: per-row term, or null
    int out_zero;          // EPI_REQUANT_ZP: output zero point
    int act_min, act_max;  // EPI_REQUANT_ZP: output clamp bounds
    const float *scale_a;  // EPI_F16: per-row scales, or null
    const float *scale_b;  // EPI_F16: per-column scales, or null
};

constexpr int kThreads = 256;
constexpr int kGroupM = 4;

// byte offset of (row, kb) inside a swizzled LDS operand tile
template <int RB, int NC>
__device__ __forceinline__ int swz(int row, int kb)
{
    return row * RB + ((((kb >> 4) ^ (row & (NC - 1)))) << 4) + (kb & 15);
}

// MSB: the int4 B operand is packed high nibble first (int8 A only)
template <int KA, int KB, int EPI, int AL, int BM, int BN, int KT, int WGM, int WGN,
          bool MSB = false>
__global__ __launch_bounds__(kThreads, 1) void k_tile(TileArgs p)
{
    constexpr int RBA = KA == OP_S8 ? KT : KT / 2;  // LDS bytes per A row
    constexpr int RBB = KB == OP_S8 ? KT : KT / 2;
    constexpr int NCA = RBA / 16, NCB = RBB / 16;  // 16-byte chunks per row
    constexpr int CA = BM * NCA / kThreads, CB = BN * NCB / kThreads;
    static_assert(BM * NCA % kThreads == 0 && BN * NCB % kThreads == 0, "chunk split");
    static_assert(kThreads % NCA == 0 && kThreads % NCB == 0, "fixed chunk column");
    static_assert(WGM * WGN == kThreads / 64, "4 waves");
    constexpr int WTM = BM / WGM, WTN = BN / WGN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
    constexpr int KSTEPS = KT / 32;
    constexpr int LDS_A = BM * RBA, LDS_B = BN * RBB, STAGE = LDS_A + LDS_B;
    // widened int4 operands carry a factor 16 each (dev_common.hpp)
    constexpr int ACC_SHIFT = (KA == OP_S4 ? 4 : 0) + (KB == OP_S4 ? 4 : 0);

    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];
    // the tile's per-column requantize parameters (bias, multiplier, shift),
    // loaded with the first K tile so that the epilogue needs no second trip
    // to memory; columns past N hold column N-1's (never stored)
    constexpr bool RQ = EPI == EPI_REQUANT || EPI == EPI_REQUANT_ZP;
    static_assert(BN <= kThreads, "one column per thread");
    __shared__ __attribute__((aligned(16))) int prm[3][RQ ? BN : 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;

    // ---- tile coordinates: XCD-aware id, then grouped row-major walk ----
    const int t = xcd_remap(blockIdx.x, gridDim.x);
    const int group = kGroupM * p.tiles_n;
    const int first_m = (t / group) * kGroupM;
    const int gsz = min(p.tiles_m - first_m, kGroupM);
    const int tm = first_m + (t % group) % gsz;
    const int tn = (t % group) / gsz;
    const int m0 = tm * BM, n0 = tn * BN;

    const int KbA = KA == OP_S8 ? p.K : p.K / 2;  // valid bytes per row
    const int KbB = KB == OP_S8 ? p.K : p.K / 2;
    const int nkt = (p.K + KT - 1) / KT;

    // ---- per-thread global chunk coordinates (fixed over the K loop) ----
    const int ca = tid % NCA, cb = tid % NCB;
    int64_t a_off[CA];
    int cv_ih[AL == AL_CONV ? CA : 1], cv_iw[AL == AL_CONV ? CA : 1];
    for (int i = 0; i < CA; ++i) {
        const int r = i * (kThreads / NCA) + tid / NCA;
        const int gm = min(m0 + r, p.M - 1);  // clamped rows are never stored
        if constexpr (AL == AL_DENSE) {
            a_off[i] = (int64_t)gm * p.lda_b;
        } else {
            const int hw = p.Ho * p.Wo;
            const int b = gm / hw;
            const int rem = gm - b * hw;
            const int oh = rem / p.Wo;
            const int ow = rem - oh * p.Wo;
            cv_ih[i] = oh * p.sh - p.ph;
            cv_iw[i] = ow * p.sw - p.pw;
            a_off[i] = (int64_t)b * p.H;  // image's first input row
        }
    }
    int64_t b_off[CB];
    for (int i = 0; i < CB; ++i) {
        const int r = i * (kThreads / NCB) + tid / NCB;
        const int gn = min(n0 + r, p.N - 1);
        b_off[i] = (int64_t)gn * p.ldb_b;
    }

    v4i ra[CA], rb[CB];
    const v4i zero4 = {0, 0, 0, 0};
    const v4i pad4 = {p.pad4, p.pad4, p.pad4, p.pad4};

    auto load_tile = [&](int kt) {
        const int kbA = kt * RBA + ca * 16;
        if constexpr (AL == AL_DENSE) {
            for (int i = 0; i < CA; ++i)
                ra[i] = kbA < KbA ? *(const v4i *)(p.A + a_off[i] + kbA) : zero4;
        } else {
            // chunk holds channels [ci, ci + 16) of tap (kh, kw); C_in % 16 == 0
            const int tap = kbA / p.C_in;
            const int ci = kbA - tap * p.C_in;
            const int kh = tap / p.KW;
            const int kw = tap - kh * p.KW;
            for (int i = 0; i < CA; ++i) {
                const int ih = cv_ih[i] + kh, iw = cv_iw[i] + kw;
                const bool inside = (unsigned)ih < (unsigned)p.H && (unsigned)iw < (unsigned)p.W;
                const int64_t off = ((a_off[i] + ih) * p.W + iw) * p.C_in + ci;
                // spatial padding holds the input zero point; K past the
                // filter meets zero weights, so its value does not matter
                ra[i] = kbA < KbA && inside ? *(const v4i *)(p.A + off) : pad4;
            }
        }
        const int kbB = kt * RBB + cb * 16;
        for (int i = 0; i < CB; ++i)
            rb[i] = kbB < KbB ? *(const v4i *)(p.B + b_off[i] + kbB) : zero4;
    };

    auto store_tile = [&](int buf) {
        uint8_t *sA = lds + buf * STAGE;
        uint8_t *sB = sA + LDS_A;
        for (int i = 0; i < CA; ++i) {
            const int r = i * (kThreads / NCA) + tid / NCA;
            *(v4i *)(sA + swz<RBA, NCA>(r, ca * 16)) = ra[i];
        }
        for (int i = 0; i < CB; ++i) {
            const int r = i * (kThreads / NCB) + tid / NCB;
            *(v4i *)(sB + swz<RBB, NCB>(r, cb * 16)) = rb[i];
        }
    };

    v16i acc[TN * TM];
    for (int i = 0; i < TN * TM; ++i)
        for (int e = 0; e < 16; ++e)
            acc[i][e] = 0;

    const int arow0 = wm * WTM + (lane & 31);
    const int brow0 = wn * WTN + (lane & 31);
    const int khalf = lane >> 5;

    auto compute = [&](int buf) {
        const uint8_t *sA = lds + buf * STAGE;
        const uint8_t *sB = sA + LDS_A;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            v4i af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = arow0 + i * 32;
                if constexpr (KA == OP_S8) {
                    v4i q = *(const v4i *)(sA + swz<RBA, NCA>(row, ks * 32 + khalf * 16));
                    af[i] = KB == OP_S4 ? even_odd_split<MSB>(q) : q;
                } else {
                    v2u q = *(const v2u *)(sA + swz<RBA, NCA>(row, ks * 16 + khalf * 8));
                    af[i] = widen_int4_x16(q);
                }
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = brow0 + j * 32;
                if constexpr (KB == OP_S8) {
                    v4i q = *(const v4i *)(sB + swz<RBB, NCB>(row, ks * 32 + khalf * 16));
                    bf[j] = KA == OP_S4 ? even_odd_split(q) : q;
                } else {
                    v2u q = *(const v2u *)(sB + swz<RBB, NCB>(row, ks * 16 + khalf * 8));
                    bf[j] = widen_int4_x16(q);
                }
            }
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    acc[j * TM + i] =
                        __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[j], af[i], acc[j * TM + i], 0, 0, 0);
        }
    };

    // ---- main K loop: prefetch tile kt+1 to registers while multiplying kt ----
    int pb = 0, pm = 0, ps = 0;
    if (RQ && tid < BN) {
        const int nn = min(n0 + tid, p.N - 1);
        pb = p.bias ? p.bias[nn] : 0;
        pm = p.mult[nn];
        ps = p.shift[nn];
    }
    load_tile(0);
    store_tile(0);
    if (RQ && tid < BN) {
        prm[0][tid] = pb;
        prm[1][tid] = pm;
        prm[2][tid] = ps;
    }
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < nkt;
        if (more)
            load_tile(kt + 1);
        compute(buf);
        if (more)
            store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds rows m = m0 + wm*WTM + i*32 + lane%32 and
    //      columns n = n0 + wn*WTN + j*32 + q*8 + (lane/32)*4 + e, e = 0..3,
    //      in accumulator registers 4q + e of sub-tile (j, i) ----
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int n = n0 + wn * WTN + j * 32 + q * 8 + khalf * 4;
            const bool full = n + 3 < p.N;
            // 4 results per store when the row stride keeps them aligned
            const bool vec = full && (p.ldc & 3) == 0;
            if constexpr (EPI == EPI_REQUANT || EPI == EPI_REQUANT_ZP) {
                constexpr bool ZP = EPI == EPI_REQUANT_ZP;
                int bia[4], mul[4], shf[4];
                long long rnd[4];
                {
                    const int nl = n - n0;  // 4 consecutive local columns, 16-byte aligned
                    const v4i b4 = *(const v4i *)&prm[0][nl];
                    const v4i m4 = *(const v4i *)&prm[1][nl];
                    const v4i s4 = *(const v4i *)&prm[2][nl];
                    for (int e = 0; e < 4; ++e) {
                        bia[e] = b4[e];
                        mul[e] = m4[e];
                        shf[e] = s4[e];
                    }
                }
                for (int e = 0; e < 4; ++e)
                    rnd[e] = 1ll << ((shf[e] - 1) & 63);
                int8_t *C = (int8_t *)p.C;
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const int m = m0 + wm * WTM + i * 32 + (lane & 31);
                    const v16i &a = acc[j * TM + i];
                    const int rt = ZP && p.rterm ? p.rterm[min(m, p.M - 1)] : 0;
                    const int zo = ZP ? p.out_zero : 0;
                    const int lo = ZP ? p.act_min : -128, hi = ZP ? p.act_max : 127;
                    int y[4];
                    for (int e = 0; e < 4; ++e)
                        y[e] = requant_one(wrap_sub(a[4 * q + e] >> ACC_SHIFT, rt), bia[e], mul[e],
                                           shf[e], rnd[e], zo, lo, hi);
                    if (m < p.M) {
                        int8_t *dst = C + (int64_t)m * p.ldc + n;
                        if (vec) {
                            *(unsigned *)dst = pack4_i8(y[0], y[1], y[2], y[3]);
                        } else {
                            for (int e = 0; e < 4; ++e)
                                if (n + e < p.N)
                                    dst[e] = (int8_t)y[e];
                        }
                    }
                }
            } else if constexpr (EPI == EPI_F16) {
                float sb[4];
                for (int e = 0; e < 4; ++e)
                    sb[e] = p.scale_b ? p.scale_b[min(n + e, p.N - 1)] : 1.0f;
                uint16_t *C = (uint16_t *)p.C;
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const int m = m0 + wm * WTM + i * 32 + (lane & 31);
                    const float sa = p.scale_a ? p.scale_a[min(m, p.M - 1)] : 1.0f;
                    const v16i &a = acc[j * TM + i];
                    unsigned short h[4];
                    for (int e = 0; e < 4; ++e) {
                        const float t = (float)(a[4 * q + e] >> ACC_SHIFT) * sa;
                        h[e] = f32_to_f16_bits(t * sb[e]);
                    }
                    if (m < p.M) {
                        uint16_t *dst = C + (int64_t)m * p.ldc + n;
                        if (vec) {
                            v2u w = {(unsigned)h[0] | ((unsigned)h[1] << 16),
                                     (unsigned)h[2] | ((unsigned)h[3] << 16)};
                            *(v2u *)dst = w;
                        } else {
                            for (int e = 0; e < 4; ++e)
                                if (n + e < p.N)
                                    dst[e] = h[e];
                        }
                    }
                }
            } else {
                int32_t *C = (int32_t *)p.C;
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const int m = m0 + wm * WTM + i * 32 + (lane & 31);
                    const v16i &a = acc[j * TM + i];
                    v4i y;
                    for (int e = 0; e < 4; ++e)
                        y[e] = a[4 * q + e] >> ACC_SHIFT;
                    if (m < p.M) {
                        int32_t *dst = C + (int64_t)m * p.ldc + n;
                        if (vec) {
                            *(v4i *)dst = y;
                        } else {
                            for (int e = 0; e < 4; ++e)
                                if (n + e < p.N)
                                    dst[e] = y[e];
                        }
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// host side

template <int KA, int KB, int EPI, int AL, int BM, int BN, int KT, int WGM, int WGN,
          bool MSB = false>
static hipError_t run_tile(TileArgs a, hipStream_t s)
{
    a.tiles_m = (int)((a.M + BM - 1) / BM);
    a.tiles_n = (int)((a.N + BN - 1) / BN);
    const int tiles = a.tiles_m * a.tiles_n;
    hipLaunchKernelGGL((k_tile<KA, KB, EPI, AL, BM, BN, KT, WGM, WGN, MSB>), dim3(tiles),
                       dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

static TileArgs gemm_args(const GemmDesc &d)
{
    TileArgs a{};
    a.A = (const uint8_t *)d.A;
    a.lda_b = d.lda_b;
    a.B = (const uint8_t *)d.B;
    a.ldb_b = d.ldb_b;
    a.bias = d.bias;
    a.mult = d.mult;
    a.shift = d.shift;
    a.C = d.C;
    a.ldc = d.ldc;
    a.M = (int)d.M;
    a.N = (int)d.N;
    a.K = (int)d.K;
    a.rterm = d.rterm;
    a.out_zero = d.out_zero;
    a.act_min = d.act_min;
    a.act_max = d.act_max;
    a.scale_a = d.scale_a;
    a.scale_b = d.scale_b;
    return a;
}

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tile size: the largest tile that still gives the chip enough workgroups.
enum TileSize { TS_256, TS_128, TS_64 };
static TileSize pick_tile(int64_t M, int64_t N)
{
    if (cdiv(M, 256) * cdiv(N, 256) >= 256)
        return TS_256;
    if (cdiv(M, 128) * cdiv(N, 128) >= 128)
        return TS_128;
    return TS_64;
}

template <int KA, int KB, int EPI, int KT, bool MSB = false>
static hipError_t run_gemm(const GemmDesc &d, hipStream_t s)
{
    const TileArgs a = gemm_args(d);
    switch (pick_tile(d.M, d.N)) {
    case TS_256:
        return run_tile<KA, KB, EPI, AL_DENSE, 256, 256, KT, 2, 2, MSB>(a, s);
    case TS_128:
        return run_tile<KA, KB, EPI, AL_DENSE, 128, 128, KT, 2, 2, MSB>(a, s);
    default:
        return run_tile<KA, KB, EPI, AL_DENSE, 64, 64, KT, 2, 2, MSB>(a, s);
    }
}

hipError_t launch_s8s8_requant(const GemmDesc &d, hipStream_t s)
{
    if (dma_gemm_fits(d, false))
        return launch_s8s8_requant_dma(d, s);
    return run_gemm<OP_S8, OP_S8, EPI_REQUANT, 128>(d, s);
}

hipError_t launch_s4s4_i32(const GemmDesc &d, hipStream_t s)
{
    if (dma_gemm_fits(d, true))
        return launch_s4s4_i32_dma(d, s);
    return run_gemm<OP_S4, OP_S4, EPI_I32, 256>(d, s);
}

hipError_t launch_s4s4_f16(const GemmDesc &d, hipStream_t s)
{
    if (dma_gemm_fits(d, true))
        return launch_s4s4_f16_dma(d, s);
    return run_gemm<OP_S4, OP_S4, EPI_F16, 256>(d, s);
}

hipError_t launch_w4a8_tiled(const GemmDesc &d, hipStream_t s)
{
    if (dma_w4a8_fits(d))
        return launch_w4a8_requant_dma(d, s);
    if (d.msb_first)
        return run_gemm<OP_S8, OP_S4, EPI_REQUANT, 128, true>(d, s);
    return run_gemm<OP_S8, OP_S4, EPI_REQUANT, 128>(d, s);
}

hipError_t launch_s8s8_requant_zp(const GemmDesc &d, hipStream_t s)
{
    if (dma_gemm_fits(d, false))
        return launch_s8s8_requant_zp_dma(d, s);
    return run_gemm<OP_S8, OP_S8, EPI_REQUANT_ZP, 128>(d, s);
}

hipError_t launch_conv_nhwc(const ConvDesc &d, hipStream_t s)
{
    TileArgs a{};
    a.A = (const uint8_t *)d.X;
    a.lda_b = 0;
    a.B = (const uint8_t *)d.W;
    a.ldb_b = (int64_t)d.KH * d.KW * d.C_in;
    a.bias = d.bias;
    a.mult = d.mult;
    a.shift = d.shift;
    a.C = d.Y;
    a.ldc = d.C_out;
    a.M = d.batch * d.Ho * d.Wo;
    a.N = d.C_out;
    a.K = d.KH * d.KW * d.C_in;
    a.H = d.H;
    a.W = d.Wd;
    a.C_in = d.C_in;
    a.KW = d.KW;
    a.Ho = d.Ho;
    a.Wo = d.Wo;
    a.sh = d.sh;
    a.sw = d.sw;
    a.ph = d.ph;
    a.pw = d.pw;
    a.pad4 = (int)(0x01010101u * (uint8_t)d.a_zero);
    a.rterm = d.rterm;
    a.out_zero = d.out_zero;
    a.act_min = d.act_min;
    a.act_max = d.act_max;
    if (d.asym) {
        if (d.C_out <= 64)
            return run_tile<OP_S8, OP_S8, EPI_REQUANT_ZP, AL_CONV, 256, 64, 64, 4, 1>(a, s);
        return run_tile<OP_S8, OP_S8, EPI_REQUANT_ZP, AL_CONV, 128, 128, 64, 2, 2>(a, s);
    }
    if (d.C_out <= 64)
        return run_tile<OP_S8, OP_S8, EPI_REQUANT, AL_CONV, 256, 64, 64, 4, 1>(a, s);
    return run_tile<OP_S8, OP_S8, EPI_REQUANT, AL_CONV, 128, 128, 64, 2, 2>(a, s);
}

}  // namespace qg
