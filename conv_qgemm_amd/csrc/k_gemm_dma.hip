// k_gemm_dma.hip -- the large-GEMM kernel: 256x256 output tiles on the
// gfx950 int8 MFMA, operands streamed global->LDS by the direct-to-LDS
// loads (global_load_lds_dwordx4) through a 4-stage ring, with the
// per-channel Q31 requantize (or a raw int32 store) fused into the
// accumulator writeback.
//
// Method (pages and sections): C = A * B with int8 or packed int4 inputs and
// int32 accumulation (INT4 GEMM article, www.cf-1.com/news/6060138, §3.2,
// packing §2.1, B column-major §4.3); requantize of the MCU conv front-end
// article (news.rkmt.cn/news/16638) §2.3.  That article's §4.3 overlaps the
// next block's transfer with the current block's compute through ping-pong
// buffers; here the same idea runs as a 4-deep ring in LDS.
//
// Per workgroup (4 waves, 2x2, each owning 128x128 = 4x4 sub-tiles of
// v_mfma_i32_32x32x32_i8, 256 accumulators in AGPRs):
//   * a stage holds 64 bytes of K for the 256 A rows and 256 B rows (32 KB);
//     each wave fills a quarter of it with 8 direct-to-LDS loads.  A load
//     writes 64 lanes x 16 bytes contiguously, so the swizzle is chosen on
//     the source side: LDS slot (row, p) receives logical chunk
//     p ^ ((row >> 2) & 3) of that row, which spreads the 16 rows read in
//     one LDS cycle of an MFMA operand fetch over all banks;
//   * three stages are in flight while one is multiplied.  Each stage is
//     read as two groups of 16-byte fragments; the second group's reads
//     overlap the first group's MFMAs, and the next stage's first group is
//     read behind the last MFMAs of this one.  The one barrier per stage
//     sits between MFMAs, after this wave's loads of the next stage have
//     landed (counted with vmcnt);
//   * a stage's 8 loads are spread over two iterations (2 right after the
//     barrier that frees their slot, 6 between the next iteration's MFMAs),
//     so the four waves never queue 32 loads at once;
//   * int4 operands are widened in registers (dev_common.hpp): a 16-byte
//     fragment read of packed data covers two MFMA K steps;
//   * the int8 epilogue requantizes into an LDS copy of the output tile and
//     writes it back with row-contiguous 16-byte stores.
#include <type_traits>

#include "dev_common.hpp"
#include "launch.hpp"

namespace qg {

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

constexpr int kBM = 256, kBN = 256;
constexpr int kRowB = 64;                     // bytes of K per row per stage
#ifndef QG_DMA_STAGES
#define QG_DMA_STAGES 4
#endif
constexpr int kStages = QG_DMA_STAGES;        // ring depth (stages in LDS)
constexpr int kStageA = kBM * kRowB;          // 16 KB
constexpr int kStageB = kBN * kRowB;          // 16 KB
constexpr int kStage = kStageA + kStageB;     // 32 KB
constexpr int kLoadsPerStage = 8;             // per wave: 4 for A, 4 for B
constexpr int kEarlyLoads = 2;                // issued right after the barrier
constexpr int kGroupM = 4;
constexpr int kOutStride = kBN + 16;          // LDS row stride of the int8 output tile

// OP_MIX: int8 A x packed int4 B (W4A8); OP_MIXM: the same with B packed
// high nibble first
enum { OP_S8 = 8, OP_S4 = 4, OP_MIX = 3, OP_MIXM = 5 };

// Per operand kind: A bytes per row per stage, ring depth, direct-to-LDS
// loads per wave per stage.  A stage always covers 64 bytes of each B row;
// with int8 A facing int4 B that is 128 K values, so A rows take 128 bytes
// and the ring drops to three 48 KB stages.
template <int KIND>
struct Geo {
    static constexpr bool kMix = KIND == OP_MIX || KIND == OP_MIXM;
    static constexpr int kRowA = kMix ? 128 : kRowB;
    static constexpr int kStageA = kBM * kRowA;
    static constexpr int kStage = kStageA + kBN * kRowB;
    static constexpr int kStages = kMix ? 3 : QG_DMA_STAGES;
    static constexpr int kLoadsA = 64 * kRowA / 1024;  // per wave: 64 rows
    static constexpr int kLoads = kLoadsA + 4;
    static constexpr int kDsPerGroup = kMix ? 12 : 8;  // LDS fragment reads per read group
};
// EPI_REQUANT_ZP: the asymmetric form.  `bias` then holds the per-column
// term bias - za * sum_k B + K * za * zb, `rterm` the per-row zb * sum_k A
// (or null when zb = 0), and the output zero point is added before the int8
// saturation; all of it modulo 2^32, which gives the true value whenever
// sum (A - za)(B - zb) + bias fits in int32.
// EPI_F16: binary16 output (INT4 GEMM article §6): fp16(fp32(acc) *
// scale_a[m] * scale_b[n]), the scales optional, each product rounded to
// binary32, the conversion to nearest even.
enum { EPI_REQUANT = 0, EPI_I32 = 1, EPI_REQUANT_ZP = 2, EPI_F16 = 3 };

struct DmaArgs {
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
    const int32_t *rterm;  // EPI_REQUANT_ZP: per-row term, or null
    int out_zero;          // EPI_REQUANT_ZP: output zero point
    int act_min, act_max;  // EPI_REQUANT_ZP: output clamp bounds
    const float *scale_a;  // EPI_F16: per-row scales, or null
    const float *scale_b;  // EPI_F16: per-column scales, or null
};

// A 16-byte LDS read is served 16 lanes per cycle over 64 4-byte banks; the
// 16 lanes of one phase read 16 consecutive rows (64 bytes apart) at the
// same logical chunk.  XOR-ing the chunk with row bits 2..3 puts those 16
// reads on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }
// 128-byte rows (int8 A facing int4 B): row r starts at bank group
// 8 * (r & 1); XOR-ing the chunk (0..7) with row bits 1..3 spreads 16
// consecutive rows over all 16 groups.
__device__ __forceinline__ int swz8(int row) { return (row >> 1) & 7; }

// Wait until at most N of this wave's direct-to-LDS loads are in flight and
// all of its LDS reads have returned, then meet the other waves.  After it,
// the stage whose loads were counted is complete for every wave, and no
// wave still reads the stage that the next loads will overwrite.  The
// memory clobber keeps the compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void wait_loads_and_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int KIND, int EPI>
__global__ __launch_bounds__(256, 1) void k_gemm_dma(DmaArgs p)
{
    using G = Geo<KIND>;
    constexpr bool MIX = G::kMix;
    constexpr bool MSB = KIND == OP_MIXM;
    constexpr int kStages = G::kStages;
    constexpr int kStage = G::kStage;
    constexpr int kStageA = G::kStageA;
    constexpr int kRowA = G::kRowA;
    constexpr int kLoadsPerStage = G::kLoads;
    // int8: a 16-byte fragment is one 32-value K step; int4: two steps
    // (int8 A facing int4 B reads two A fragments per B fragment)
    constexpr int STEPS_PER_READ = KIND == OP_S8 ? 1 : 2;
    constexpr int ACC_SHIFT = KIND == OP_S4 ? 8 : (MIX ? 4 : 0);
    constexpr int MG = 16 * STEPS_PER_READ;  // MFMAs per read group
    constexpr int DSG = G::kDsPerGroup;
    constexpr bool RQ = EPI == EPI_REQUANT || EPI == EPI_REQUANT_ZP;
    constexpr bool ZP = EPI == EPI_REQUANT_ZP;
    constexpr bool F16 = EPI == EPI_F16;

    // one LDS object: the operand ring, then the per-column bias / multiplier
    // / shift of this tile's 256 output columns and the per-row term of its
    // 256 rows (a second __shared__ object makes the compiler wait for every
    // direct-to-LDS load before any read)
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages * kStage + 4 * kBN * 4];
    int(*prm)[kBN] = (int(*)[kBN])(lds + kStages * kStage);
    static_assert(kBM == kBN, "the row terms share the column-parameter layout");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    const int t = xcd_remap(blockIdx.x, gridDim.x);
    const int group = kGroupM * p.tiles_n;
    const int first_m = (t / group) * kGroupM;
    const int gsz = min(p.tiles_m - first_m, kGroupM);
    const int tm = first_m + (t % group) % gsz;
    const int tn = (t % group) / gsz;
    const int m0 = tm * kBM, n0 = tn * kBN;

    const int nkt = (KIND == OP_S8 ? p.K : p.K / 2) / kRowB;  // B bytes per row / 64

    // requantize parameters of column n0 + tid, fetched now and parked in LDS
    // (the barrier of the prologue publishes them) so the epilogue reads
    // them without global-memory latency
    int pb = 0, pm = 0, ps = 0, pr = 0;
    if constexpr (RQ) {
        const int n = min(n0 + tid, p.N - 1);
        pb = p.bias ? p.bias[n] : 0;
        pm = p.mult[n];
        ps = p.shift[n];
    }
    if constexpr (ZP) {
        if (p.rterm)
            pr = p.rterm[min(m0 + tid, p.M - 1)];
    }
    if constexpr (F16) {
        // column and row scales of the tile, as bit patterns (1.0 if absent)
        pb = __float_as_int(p.scale_b ? p.scale_b[min(n0 + tid, p.N - 1)] : 1.0f);
        pr = __float_as_int(p.scale_a ? p.scale_a[min(m0 + tid, p.M - 1)] : 1.0f);
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- direct-to-LDS sources: this wave fills rows [wave*64, wave*64+64)
    //      of the A and B stage tiles, 16 rows per load ----
    constexpr int LA = G::kLoadsA;
    uint32_t src[kLoadsPerStage];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        if constexpr (MIX) {
            // 8 rows of 128 bytes per load
            const int r = wave * 64 + i * 8 + (lane >> 3);
            const int c = (lane & 7) ^ swz8(r);
            src[i] = (uint32_t)((int64_t)min(m0 + r, p.M - 1) * p.lda_b) + c * 16;
        } else {
            const int r = wave * 64 + i * 16 + (lane >> 2);
            const int c = (lane & 3) ^ swz(r);
            src[i] = (uint32_t)((int64_t)min(m0 + r, p.M - 1) * p.lda_b) + c * 16;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = wave * 64 + i * 16 + (lane >> 2);
        const int c = (lane & 3) ^ swz(r);
        src[LA + i] = (uint32_t)((int64_t)min(n0 + r, p.N - 1) * p.ldb_b) + c * 16;
    }
    // load l (0..LA-1: A, LA..LA+3: B) of K stage `s` into ring slot
    // s % kStages; a stage past the last one re-reads the last into a slot
    // no later stage uses
    auto issue = [&](int s, int l) {
        const int kt = min(s, nkt - 1);
        const bool isb = l >= LA;
        uint8_t *dst = lds + (s % kStages) * kStage +
                       (isb ? kStageA + wave * 4096 + (l - LA) * 1024
                            : wave * (64 * kRowA) + l * 1024);
        const uint8_t *g = isb ? p.B + (int64_t)kt * kRowB : p.A + (int64_t)kt * kRowA;
        __builtin_amdgcn_global_load_lds((const glb_void_t *)(g + src[l]), (lds_void_t *)dst, 16,
                                         0, 0);
    };

    // ---- fragment addresses inside a stage: read group g covers chunk
    //      2g + (lane >> 5) of rows (lane & 31) + 32 * sub-tile.  The swizzle
    //      only sees row bits 2..3, so sub-tile i is a fixed offset i*2048 ----
    //      With 128-byte A rows the K values of B chunk c (16 bytes = 32
    //      int4 values) are A chunks 2c and 2c + 1; the swizzle sees row bits
    //      1..3, so sub-tile i is again a fixed offset (i*4096) ----
    int a_rd[2][2], b_rd[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const int ra = wm * 128 + (lane & 31);
        const int rb = wn * 128 + (lane & 31);
        const int c = 2 * g + (lane >> 5);
        if constexpr (MIX) {
            a_rd[g][0] = ra * kRowA + (((2 * c) ^ swz8(ra)) << 4);
            a_rd[g][1] = ra * kRowA + (((2 * c + 1) ^ swz8(ra)) << 4);
        } else {
            a_rd[g][0] = a_rd[g][1] = ra * kRowA + ((c ^ swz(ra)) << 4);
        }
        b_rd[g] = kStageA + rb * kRowB + ((c ^ swz(rb)) << 4);
    }

    v16i acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        for (int e = 0; e < 16; ++e)
            acc[i][e] = 0;

    // raw fragments of read groups 0 and 1 (int8 A facing int4 B: two A
    // fragments per sub-tile, [i] and [4 + i])
    constexpr int NA = MIX ? 8 : 4;
    v4i fa[2][NA], fb[2][4];

    auto read_group = [&](int kt, int g, v4i (&ra)[NA], v4i (&rb)[4]) {
        const uint8_t *st = lds + (kt % kStages) * kStage;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ra[i] = *(const v4i *)(st + a_rd[g][0] + i * 32 * kRowA);
        if constexpr (MIX) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ra[4 + i] = *(const v4i *)(st + a_rd[g][1] + i * 32 * kRowA);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            rb[i] = *(const v4i *)(st + b_rd[g] + i * 32 * kRowB);
    };

    // MFMAs of one read group over sub-tiles (j, i) in [j0, j1) x [0, 4)
    auto mma_group = [&](const v4i (&ra)[NA], const v4i (&rb)[4], int j0, int j1) {
#pragma unroll
        for (int h = 0; h < STEPS_PER_READ; ++h) {
            // int8 A facing int4 B: K step h of this group is A fragment
            // [4h + i], byte-permuted to the widened-int4 order once
            v4i as[MIX ? 4 : 1];
            if constexpr (MIX) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    as[i] = even_odd_split<MSB>(ra[4 * h + i]);
            }
#pragma unroll
            for (int j = j0; j < j1; ++j) {
                v4i bq;
                if constexpr (KIND == OP_S8) {
                    bq = rb[j];
                } else {
                    v2u w = {(unsigned)rb[j][2 * h], (unsigned)rb[j][2 * h + 1]};
                    bq = widen_int4_x16(w);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v4i aq;
                    if constexpr (KIND == OP_S8) {
                        aq = ra[i];
                    } else if constexpr (MIX) {
                        aq = as[i];
                    } else {
                        v2u w = {(unsigned)ra[i][2 * h], (unsigned)ra[i][2 * h + 1]};
                        aq = widen_int4_x16(w);
                    }
                    acc[j * 4 + i] =
                        __builtin_amdgcn_mfma_i32_32x32x32_i8(bq, aq, acc[j * 4 + i], 0, 0, 0);
                }
            }
        }
    };

    // ---- prologue: stages 0..kStages-2 and the first loads of the next
    //      issued, stage 0 readable.  Loads issued behind any stage's are
    //      always kStages-2 whole stages when it is waited for ----
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
#pragma unroll
        for (int l = 0; l < kLoadsPerStage; ++l)
            issue(s, l);
#pragma unroll
    for (int l = 0; l < kEarlyLoads; ++l)
        issue(kStages - 1, l);
    if constexpr (RQ) {
        prm[0][tid] = pb;
        prm[1][tid] = pm;
        prm[2][tid] = ps;
    }
    if constexpr (ZP)
        prm[3][tid] = pr;
    if constexpr (F16) {
        prm[0][tid] = pb;
        prm[3][tid] = pr;
    }
    wait_loads_and_barrier<(kStages - 2) * kLoadsPerStage + kEarlyLoads>();
    read_group(0, 0, fa[0], fb[0]);

    for (int kt = 0; kt < nkt; ++kt) {
        // group 1 of this stage streams in behind group 0's MFMAs, and the
        // rest of stage kt+kStages-1 (its slot was freed at the last barrier)
        read_group(kt, 1, fa[1], fb[1]);
#pragma unroll
        for (int l = kEarlyLoads; l < kLoadsPerStage; ++l)
            issue(kt + kStages - 1, l);
        mma_group(fa[0], fb[0], 0, 4);
        mma_group(fa[1], fb[1], 0, 2);
#pragma unroll
        for (int i = 0; i < DSG; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        }
#pragma unroll
        for (int i = 0; i < kLoadsPerStage - kEarlyLoads; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
        }
        __builtin_amdgcn_sched_group_barrier(
            0x008, MG + MG / 2 - DSG - 2 * (kLoadsPerStage - kEarlyLoads), 0);
        // nothing crosses the barrier: the MFMAs before it keep the matrix
        // pipe busy while the waves meet
        __builtin_amdgcn_sched_barrier(0);
        // stage kt+1 landed for this wave; after the barrier, for all.  Every
        // wave has read all of stage kt, so its slot takes stage kt+kStages.
        wait_loads_and_barrier<(kStages - 2) * kLoadsPerStage>();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int l = 0; l < kEarlyLoads; ++l)
            issue(kt + kStages, l);
        read_group(kt + 1, 0, fa[0], fb[0]);
        mma_group(fa[1], fb[1], 2, 4);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
        }
#pragma unroll
        for (int i = 0; i < DSG / 2 - 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, MG / 2 - DSG / 2, 0);
    }
    // the re-issued loads past the last stage must land before the LDS is
    // reused for the output tile, and every wave must be done reading it
    wait_loads_and_barrier<0>();

    // ---- epilogue: lane holds rows ml = wm*128 + i*32 + lane%32 and columns
    //      nl = wn*128 + j*32 + q*8 + (lane/32)*4 + e of the tile in
    //      accumulator registers 4q + e of sub-tile (j, i) ----
    const int khalf = lane >> 5;
    if constexpr (RQ) {
        // requantize into an LDS copy of the 256 x 256 int8 tile, with the
        // cheapest exact form that every shift of the tile allows (chosen
        // once, so the accumulator indices stay compile-time constants)
        uint8_t *otile = lds;
        const v4i sh4 = *(const v4i *)&prm[2][lane * 4];
        bool s33 = true, s31 = true;
        for (int e = 0; e < 4; ++e) {
            s33 = s33 && sh4[e] >= 33;
            s31 = s31 && sh4[e] >= 31;
        }
        auto requant_tile = [&](auto tier_tag) {
            constexpr int TIER = decltype(tier_tag)::value;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int nl = wn * 128 + j * 32 + q * 8 + khalf * 4;
                    const v4i b4 = *(const v4i *)&prm[0][nl];
                    const v4i m4 = *(const v4i *)&prm[1][nl];
                    const v4i s4 = *(const v4i *)&prm[2][nl];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int ml = wm * 128 + i * 32 + (lane & 31);
                        const int rt = ZP ? prm[3][ml] : 0;
                        const int zo = ZP ? p.out_zero : 0;
                        const int lo = ZP ? p.act_min : -128, hi = ZP ? p.act_max : 127;
                        int y[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            int a = acc[j * 4 + i][4 * q + e] >> ACC_SHIFT;
                            if constexpr (ZP)
                                a = wrap_sub(a, rt);
                            if constexpr (TIER == 2)
                                y[e] = requant_one_s33(a, b4[e], m4[e], s4[e], zo, lo, hi);
                            else if constexpr (TIER == 1)
                                y[e] = requant_one_s31(a, b4[e], m4[e], s4[e],
                                                       1ll << ((s4[e] - 1) & 63), zo, lo, hi);
                            else
                                y[e] = requant_one(a, b4[e], m4[e], s4[e],
                                                   1ll << ((s4[e] - 1) & 63), zo, lo, hi);
                        }
                        *(unsigned *)(otile + ml * kOutStride + nl) =
                            pack4_i8(y[0], y[1], y[2], y[3]);
                    }
                }
            }
        };
        if (__builtin_amdgcn_ballot_w64(!s33) == 0)
            requant_tile(std::integral_constant<int, 2>{});
        else if (__builtin_amdgcn_ballot_w64(!s31) == 0)
            requant_tile(std::integral_constant<int, 1>{});
        else
            requant_tile(std::integral_constant<int, 0>{});
        __syncthreads();
        // 256 rows x 16 chunks of 16 bytes; consecutive threads walk a row
        int8_t *C = (int8_t *)p.C;
        const bool vec_ok = (p.ldc & 15) == 0;
#pragma unroll 4
        for (int it = 0; it < kBM * (kBN / 16) / 256; ++it) {
            const int id = it * 256 + tid;
            const int rl = id >> 4, cl = (id & 15) * 16;
            const int m = m0 + rl, n = n0 + cl;
            const v4i v = *(const v4i *)(otile + rl * kOutStride + cl);
            if (m < p.M) {
                int8_t *dst = C + (int64_t)m * p.ldc + n;
                if (vec_ok && n + 15 < p.N) {
                    *(v4i *)dst = v;
                } else {
                    for (int b = 0; b < 16; ++b)
                        if (n + b < p.N)
                            dst[b] = (int8_t)(v[b >> 2] >> (8 * (b & 3)));
                }
            }
        }
    } else if constexpr (F16) {
        // binary16: 4 adjacent columns of one row per 8-byte store
        uint16_t *C = (uint16_t *)p.C;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nl = wn * 128 + j * 32 + q * 8 + khalf * 4;
                const int n = n0 + nl;
                const bool vec = n + 3 < p.N && (p.ldc & 3) == 0;
                const v4i sb4 = *(const v4i *)&prm[0][nl];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ml = wm * 128 + i * 32 + (lane & 31);
                    const int m = m0 + ml;
                    const float sa = __int_as_float(prm[3][ml]);
                    const v16i &a = acc[j * 4 + i];
                    unsigned short h[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float t = (float)(a[4 * q + e] >> ACC_SHIFT) * sa;
                        h[e] = f32_to_f16_bits(t * __int_as_float(sb4[e]));
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
            }
        }
    } else {
        // raw int32: 4 adjacent columns of one row per 16-byte store
        int32_t *C = (int32_t *)p.C;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * 128 + j * 32 + q * 8 + khalf * 4;
                const bool vec = n + 3 < p.N && (p.ldc & 3) == 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = m0 + wm * 128 + i * 32 + (lane & 31);
                    const v16i &a = acc[j * 4 + i];
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

template <int KIND, int EPI>
hipError_t run(const GemmDesc &d, hipStream_t s)
{
    DmaArgs a{};
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
    a.tiles_m = (int)((d.M + kBM - 1) / kBM);
    a.tiles_n = (int)((d.N + kBN - 1) / kBN);
    a.rterm = d.rterm;
    a.out_zero = d.out_zero;
    a.act_min = d.act_min;
    a.act_max = d.act_max;
    a.scale_a = d.scale_a;
    a.scale_b = d.scale_b;
    hipLaunchKernelGGL((k_gemm_dma<KIND, EPI>), dim3(a.tiles_m * a.tiles_n), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

// The ring kernel takes whole 64-byte K rows and 32-bit source offsets.
bool dma_gemm_fits(const GemmDesc &d, bool int4)
{
    const int64_t kb = int4 ? d.K / 2 : d.K;
    if (kb % kRowB != 0)
        return false;
    const int64_t lim = (int64_t)1 << 32;
    if ((d.M - 1) * d.lda_b + kb >= lim || (d.N - 1) * d.ldb_b + kb >= lim)
        return false;
    // enough 256x256 tiles to fill the chip
    return ((d.M + kBM - 1) / kBM) * ((d.N + kBN - 1) / kBN) >= 128;
}

hipError_t launch_s8s8_requant_dma(const GemmDesc &d, hipStream_t s)
{
    return run<OP_S8, EPI_REQUANT>(d, s);
}

hipError_t launch_s4s4_i32_dma(const GemmDesc &d, hipStream_t s)
{
    return run<OP_S4, EPI_I32>(d, s);
}

hipError_t launch_s8s8_requant_zp_dma(const GemmDesc &d, hipStream_t s)
{
    return run<OP_S8, EPI_REQUANT_ZP>(d, s);
}

hipError_t launch_s4s4_f16_dma(const GemmDesc &d, hipStream_t s)
{
    return run<OP_S4, EPI_F16>(d, s);
}

// int8 A x int4 B: whole 128-value K stages and 32-bit source offsets
bool dma_w4a8_fits(const GemmDesc &d)
{
    if (d.K % 128 != 0)
        return false;
    const int64_t lim = (int64_t)1 << 32;
    if ((d.M - 1) * d.lda_b + d.K >= lim || (d.N - 1) * d.ldb_b + d.K / 2 >= lim)
        return false;
    return ((d.M + kBM - 1) / kBM) * ((d.N + kBN - 1) / kBN) >= 128;
}

hipError_t launch_w4a8_requant_dma(const GemmDesc &d, hipStream_t s)
{
    if (d.msb_first)
        return run<OP_MIXM, EPI_REQUANT>(d, s);
    return run<OP_MIX, EPI_REQUANT>(d, s);
}

}  // namespace qg
