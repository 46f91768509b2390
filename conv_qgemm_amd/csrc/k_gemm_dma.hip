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
//   * the grid is one workgroup per compute unit, walking its tiles; the
//     ring runs across tile boundaries (a tile's last stages issue the next
//     tile's first), and per-tile parameters come in by direct-to-LDS loads
//     into a double buffer, so a tile starts with its operands in LDS;
//   * the epilogue works from registers: the int8 results of each 32x32
//     sub-tile row are regrouped across the two half-waves with
//     v_permlane32_swap into 16-byte stores, a 32-row band at a time so that
//     each output line fills from consecutive stores.
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
#ifndef QG_DMA_PRE_J1
#define QG_DMA_PRE_J1 2
#endif
constexpr int kPreJ1 = QG_DMA_PRE_J1;          // read group 1 sub-tile columns before the barrier
#ifndef QG_DMA_GROUP_M
#define QG_DMA_GROUP_M 4
#endif
constexpr int kGroupM = QG_DMA_GROUP_M;      // tile rows that share B panels in L2

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

// The lane id, computed afresh.  The asm is volatile so that it is not
// merged with a lane id kept from the start of the kernel: across the main
// loop such a value is spilled, and its reload would wait for every load in
// flight, the next tile's ring stages included.
__device__ __forceinline__ int fresh_lane()
{
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    return ln;
}

// One 4-byte direct-to-LDS load per lane: lane L's dword lands at dst + 4L.
__device__ __forceinline__ void dma_dword(const void *src, void *dst)
{
    __builtin_amdgcn_global_load_lds((const glb_void_t *)src, (lds_void_t *)dst, 4, 0, 0);
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
    // MFMAs of a stage before its barrier (read group 0, and the first
    // kPreJ1 sub-tile columns of group 1) and after it (the rest of group 1,
    // which covers the reads of the next stage's group 0)
    constexpr int kMfmaPerJ = 4 * STEPS_PER_READ;
    constexpr int kMfmaPre = MG + kPreJ1 * kMfmaPerJ;
    constexpr int kMfmaPost = (4 - kPreJ1) * kMfmaPerJ;
    constexpr int kPreMfmaPerLoad = (kMfmaPre - DSG) / (G::kLoads - kEarlyLoads);
    static_assert(kPreMfmaPerLoad >= 1 && kMfmaPost >= DSG / 2, "stage schedule");
    constexpr bool RQ = EPI == EPI_REQUANT || EPI == EPI_REQUANT_ZP;
    constexpr bool ZP = EPI == EPI_REQUANT_ZP;
    constexpr bool F16 = EPI == EPI_F16;

    // one LDS object: the operand ring, then two buffers of per-tile
    // parameters (a second __shared__ object makes the compiler wait for
    // every direct-to-LDS load before any read).  Buffer b holds, for its
    // tile's 256 columns / rows: [0] bias (EPI_F16: column scales), [1]
    // multiplier, [2] shift, [3] per-row term (EPI_F16: row scales).
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages * kStage + 2 * 4 * kBN * 4];
    int(*prm_buf)[4][kBN] = (int(*)[4][kBN])(lds + kStages * kStage);
    static_assert(kBM == kBN, "the row terms share the column-parameter layout");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    const int ntiles = p.tiles_m * p.tiles_n;
    const int nkt = (KIND == OP_S8 ? p.K : p.K / 2) / kRowB;  // B bytes per row / 64

    // tile v of the persistent walk -> its first row and column.  Virtual
    // tile v runs on XCD v % 8 (the grid is a multiple of 8 on MI355X), so
    // xcd_remap gives each XCD a contiguous run of tile ids, and groups of
    // kGroupM tile rows share their B panels in that XCD's L2.  A tile at
    // the bottom or right edge is moved inward to end at row M / column N
    // (M, N >= 256): it then overlaps its neighbour, whose outputs it
    // recomputes bit for bit, and no row or column is ever out of range.
    auto coords = [&](int v, int &m0, int &n0) __attribute__((always_inline)) {
        const int t = xcd_remap(v, ntiles);
        const int group = kGroupM * p.tiles_n;
        const int first_m = (t / group) * kGroupM;
        const int gsz = min(p.tiles_m - first_m, kGroupM);
        m0 = min((first_m + (t % group) % gsz) * kBM, p.M - kBM);
        n0 = min(((t % group) / gsz) * kBN, p.N - kBN);
    };

    // ---- direct-to-LDS sources: this wave fills rows [wave*64, wave*64+64)
    //      of the A and B stage tiles, 16 rows per load (8 rows of 128 bytes
    //      for the int8 A facing int4 B).  The per-lane offsets inside a
    //      tile are the same for every tile; a tile adds a scalar base ----
    constexpr int LA = G::kLoadsA;
    uint32_t src[kLoadsPerStage];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        if constexpr (MIX) {
            const int r = wave * 64 + i * 8 + (lane >> 3);
            const int c = (lane & 7) ^ swz8(r);
            src[i] = (uint32_t)r * (uint32_t)p.lda_b + c * 16;
        } else {
            const int r = wave * 64 + i * 16 + (lane >> 2);
            const int c = (lane & 3) ^ swz(r);
            src[i] = (uint32_t)r * (uint32_t)p.lda_b + c * 16;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = wave * 64 + i * 16 + (lane >> 2);
        const int c = (lane & 3) ^ swz(r);
        src[LA + i] = (uint32_t)r * (uint32_t)p.ldb_b + c * 16;
    }

    // ---- per-tile parameters: this wave's 64 columns (and rows) of the
    //      tile, one 4-byte direct-to-LDS load per array; absent arrays are
    //      constants written once ----
    auto load_prm = [&](int buf, int m0, int n0) __attribute__((always_inline)) {
        const int ln = fresh_lane();
        const int n = n0 + wave * 64 + ln;
        const int m = m0 + wave * 64 + ln;
        int(*pb)[kBN] = prm_buf[buf];
        if constexpr (RQ) {
            if (p.bias)
                dma_dword(p.bias + n, &pb[0][wave * 64]);
            dma_dword(p.mult + n, &pb[1][wave * 64]);
            dma_dword(p.shift + n, &pb[2][wave * 64]);
            if (ZP && p.rterm)
                dma_dword(p.rterm + m, &pb[3][wave * 64]);
        }
        if constexpr (F16) {
            if (p.scale_b)
                dma_dword(p.scale_b + n, &pb[0][wave * 64]);
            if (p.scale_a)
                dma_dword(p.scale_a + m, &pb[3][wave * 64]);
        }
    };
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        if (RQ && !p.bias)
            prm_buf[b][0][tid] = 0;
        if (ZP && !p.rterm)
            prm_buf[b][3][tid] = 0;
        if (F16 && !p.scale_b)
            prm_buf[b][0][tid] = __float_as_int(1.0f);
        if (F16 && !p.scale_a)
            prm_buf[b][3][tid] = __float_as_int(1.0f);
    }

    // ---- the walk: tiles v = blockIdx.x + k * gridDim.x.  The ring runs
    //      across tile boundaries: stages past this tile's last are the next
    //      tile's first, loaded while this tile's last stages multiply ----
    int v = blockIdx.x;
    int m0, n0, m0n, n0n;
    coords(v, m0, n0);
    bool has_next = v + (int)gridDim.x < ntiles;
    if (has_next)
        coords(v + (int)gridDim.x, m0n, n0n);
    else
        m0n = m0, n0n = n0;
    // byte offsets of stage 0 of this tile in A and B, and of the next
    // tile's stage 0 minus nkt stages, so that stage s (s >= nkt: the next
    // tile's stage s - nkt) is one select and one add away.  With no next
    // tile the stages past the last re-read this tile's first ones into
    // slots no later stage uses.
    int64_t a_cur, b_cur, a_nxt, b_nxt;
    auto set_bases = [&]() __attribute__((always_inline)) {
        a_cur = (int64_t)m0 * p.lda_b;
        b_cur = (int64_t)n0 * p.ldb_b;
        a_nxt = (int64_t)m0n * p.lda_b - (int64_t)nkt * kRowA;
        b_nxt = (int64_t)n0n * p.ldb_b - (int64_t)nkt * kRowB;
    };
    set_bases();

    // load l (0..LA-1: A, LA..LA+3: B) of stage s of this tile into ring
    // slot `slot`
    auto issue = [&](int s, int slot, int l) __attribute__((always_inline)) {
        const bool nxt = s >= nkt;
        const bool isb = l >= LA;
        uint8_t *dst = lds + slot * kStage +
                       (isb ? kStageA + wave * 4096 + (l - LA) * 1024
                            : wave * (64 * kRowA) + l * 1024);
        const uint8_t *g = isb ? p.B + (nxt ? b_nxt : b_cur) + (int64_t)s * kRowB
                               : p.A + (nxt ? a_nxt : a_cur) + (int64_t)s * kRowA;
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

    // raw fragments of read groups 0 and 1 (int8 A facing int4 B: two A
    // fragments per sub-tile, [i] and [4 + i])
    constexpr int NA = MIX ? 8 : 4;
    v4i fa[2][NA], fb[2][4];

    auto read_group = [&](int slot, int g, v4i(&ra)[NA], v4i(&rb)[4]) __attribute__((always_inline)) {
        const uint8_t *st = lds + slot * kStage;
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
    auto mma_group = [&](const v4i(&ra)[NA], const v4i(&rb)[4], int j0, int j1) __attribute__((always_inline)) {
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

    // ---- prologue of the first tile: its parameters, stages
    //      0..kStages-2 and the first loads of the next issued, stage 0
    //      readable.  Loads issued behind any stage's are always kStages-2
    //      whole stages when it is waited for ----
    if constexpr (RQ || F16)
        load_prm(0, m0, n0);
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
#pragma unroll
        for (int l = 0; l < kLoadsPerStage; ++l)
            issue(s, s, l);
#pragma unroll
    for (int l = 0; l < kEarlyLoads; ++l)
        issue(kStages - 1, kStages - 1, l);
    wait_loads_and_barrier<(kStages - 2) * kLoadsPerStage + kEarlyLoads>();
    read_group(0, 0, fa[0], fb[0]);
    int rs = 0;  // ring slot of the stage being multiplied

    for (int k = 0;; ++k) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            for (int e = 0; e < 16; ++e)
                acc[i][e] = 0;
        // the last kStages - 1 stages issue the next tile's first loads (the
        // ring is never deeper than a tile: nkt >= kStages)
        for (int kt = 0; kt < nkt; ++kt) {
            // slots of stages kt + kStages - 1 (the one before rs) and kt + 1
            const int ps = rs == 0 ? kStages - 1 : rs - 1;
            const int ns = rs == kStages - 1 ? 0 : rs + 1;
            // group 1 of this stage streams in behind group 0's MFMAs, and
            // the rest of stage kt+kStages-1 (its slot was freed at the last
            // barrier)
            read_group(rs, 1, fa[1], fb[1]);
#pragma unroll
            for (int l = kEarlyLoads; l < kLoadsPerStage; ++l)
                issue(kt + kStages - 1, ps, l);
            mma_group(fa[0], fb[0], 0, 4);
            if constexpr (kPreJ1 > 0)
                mma_group(fa[1], fb[1], 0, kPreJ1);
#pragma unroll
            for (int i = 0; i < DSG; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
            }
#pragma unroll
            for (int i = 0; i < kLoadsPerStage - kEarlyLoads; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, kPreMfmaPerLoad, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                // VMEM read
            }
            __builtin_amdgcn_sched_group_barrier(
                0x008, kMfmaPre - DSG - kPreMfmaPerLoad * (kLoadsPerStage - kEarlyLoads), 0);
            // nothing crosses the barrier: the MFMAs before it keep the
            // matrix pipe busy while the waves meet
            __builtin_amdgcn_sched_barrier(0);
            // stage kt+1 landed for this wave; after the barrier, for all.
            // Every wave has read all of stage kt, so its slot takes stage
            // kt+kStages.
            wait_loads_and_barrier<(kStages - 2) * kLoadsPerStage>();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int l = 0; l < kEarlyLoads; ++l)
                issue(kt + kStages, rs, l);
            // after the last stage this reads the next tile's first
            // fragments, which are read again once the epilogue is done
            read_group(ns, 0, fa[0], fb[0]);
            mma_group(fa[1], fb[1], kPreJ1, 4);
#pragma unroll
            for (int i = 0; i < kEarlyLoads; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
            }
#pragma unroll
            for (int i = 0; i < DSG / 2 - kEarlyLoads; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPost - DSG / 2, 0);
            rs = ns;
        }

        // ---- epilogue: lane holds rows ml = wm*128 + i*32 + lane%32 and
        //      columns nl = wn*128 + j*32 + q*8 + (lane/32)*4 + e of the
        //      tile in accumulator registers 4q + e of sub-tile (j, i).  Its
        //      parameters landed before the last stage's barrier; the ring
        //      already holds the next tile's first stages ----
        int(*prm)[kBN] = prm_buf[k & 1];
        const int lane = fresh_lane();
        const int khalf = lane >> 5;
        if constexpr (RQ) {
            // requantize with the cheapest exact form that every shift of
            // the tile allows (chosen once, so the accumulator indices stay
            // compile-time constants).  For each 32x32 sub-tile a lane
            // packs its 16 results of one row into 4 dwords (q = 0..3, 4
            // columns each); one v_permlane32_swap per dword pair gives the
            // lower half-wave columns 0..15 and the upper columns 16..31 of
            // that row, stored as one 16-byte write.
            const v4i sh4 = *(const v4i *)&prm[2][lane * 4];
            bool s33 = true, s31 = true;
            for (int e = 0; e < 4; ++e) {
                s33 = s33 && sh4[e] >= 33;
                s31 = s31 && sh4[e] >= 31;
            }
            int8_t *C = (int8_t *)p.C;
            const bool vec_ok = (p.ldc & 15) == 0;
            auto requant_tile = [&](auto tier_tag) __attribute__((always_inline)) {
                constexpr int TIER = decltype(tier_tag)::value;
                // one 32-row band at a time, its four sub-tiles back to back,
                // so that each 128-byte line of a row is written by
                // consecutive stores (a line left partly written in L2 for
                // long is written back in pieces)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ml = wm * 128 + i * 32 + (lane & 31);
                    const int rt = ZP ? prm[3][ml] : 0;
                    const int zo = ZP ? p.out_zero : 0;
                    const int lo = ZP ? p.act_min : -128, hi = ZP ? p.act_max : 127;
                    int8_t *row = C + (int64_t)(m0 + ml) * p.ldc + n0 + wn * 128 + khalf * 16;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        unsigned d[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int nl = wn * 128 + j * 32 + q * 8 + khalf * 4;
                            const v4i b4 = *(const v4i *)&prm[0][nl];
                            const v4i m4 = *(const v4i *)&prm[1][nl];
                            const v4i s4 = *(const v4i *)&prm[2][nl];
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
                            d[q] = pack4_i8(y[0], y[1], y[2], y[3]);
                            // int8 x int4: 4 values at a time, or
                            // accumulators spill, and each reload's wait
                            // holds the epilogue until the next tile's stages
                            // have landed (W4A8 prefill 426.6 -> 416.3 us).
                            // The int8 x int8 forms are no faster with it.
                            if constexpr (MIX)
                                __builtin_amdgcn_sched_barrier(0);
                        }
                        const auto r02 = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
                        const auto r13 = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
                        const v4i out = {(int)r02[0], (int)r02[1], (int)r13[0], (int)r13[1]};
                        int8_t *dst = row + j * 32;
                        if (vec_ok) {
                            *(v4i *)dst = out;
                        } else {
                            for (int b = 0; b < 16; ++b)
                                dst[b] = (int8_t)(out[b >> 2] >> (8 * (b & 3)));
                        }
                        // one sub-tile's parameters in registers at a time:
                        // hoisting a whole band's would spill
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            };
            if (__builtin_amdgcn_ballot_w64(!s33) == 0)
                requant_tile(std::integral_constant<int, 2>{});
            else if (__builtin_amdgcn_ballot_w64(!s31) == 0)
                requant_tile(std::integral_constant<int, 1>{});
            else
                requant_tile(std::integral_constant<int, 0>{});
        } else if constexpr (F16) {
            // binary16: 4 adjacent columns of one row per 8-byte store, a
            // 32-row band at a time so that each row's lines fill from
            // consecutive stores
            uint16_t *C = (uint16_t *)p.C;
            const bool vec = (p.ldc & 3) == 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ml = wm * 128 + i * 32 + (lane & 31);
                const float sa = __int_as_float(prm[3][ml]);
                uint16_t *row = C + (int64_t)(m0 + ml) * p.ldc + n0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const v16i &a = acc[j * 4 + i];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int nl = wn * 128 + j * 32 + q * 8 + khalf * 4;
                        const v4i sb4 = *(const v4i *)&prm[0][nl];
                        unsigned short h[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float t = (float)(a[4 * q + e] >> ACC_SHIFT) * sa;
                            h[e] = f32_to_f16_bits(t * __int_as_float(sb4[e]));
                        }
                        uint16_t *dst = row + nl;
                        if (vec) {
                            v2u w = {(unsigned)h[0] | ((unsigned)h[1] << 16),
                                     (unsigned)h[2] | ((unsigned)h[3] << 16)};
                            *(v2u *)dst = w;
                        } else {
                            for (int e = 0; e < 4; ++e)
                                dst[e] = h[e];
                        }
                    }
                }
            }
        } else {
            // raw int32: 4 adjacent columns of one row per 16-byte store, a
            // 32-row band at a time so that each row's lines fill from
            // consecutive stores
            int32_t *C = (int32_t *)p.C;
            const bool vec = (p.ldc & 3) == 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ml = wm * 128 + i * 32 + (lane & 31);
                int32_t *row = C + (int64_t)(m0 + ml) * p.ldc + n0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const v16i &a = acc[j * 4 + i];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int nl = wn * 128 + j * 32 + q * 8 + khalf * 4;
                        v4i y;
                        for (int e = 0; e < 4; ++e)
                            y[e] = a[4 * q + e] >> ACC_SHIFT;
                        int32_t *dst = row + nl;
                        if (vec) {
                            *(v4i *)dst = y;
                        } else {
                            for (int e = 0; e < 4; ++e)
                                dst[e] = y[e];
                        }
                    }
                }
            }
        }

        if (!has_next)
            break;
        // ---- advance: the next tile's stage 0 landed before the last
        //      barrier; its parameters go to the other buffer, whose last
        //      reader (the epilogue two tiles back) finished long ago ----
        v += (int)gridDim.x;
        m0 = m0n;
        n0 = n0n;
        has_next = v + (int)gridDim.x < ntiles;
        if (has_next)
            coords(v + (int)gridDim.x, m0n, n0n);
        set_bases();
        if constexpr (RQ || F16)
            load_prm((k + 1) & 1, m0, n0);
        read_group(rs, 0, fa[0], fb[0]);
    }
    // the re-reads past the last stage must land before the workgroup ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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
    // one persistent workgroup per CU (the LDS ring allows no second)
    const int ntiles = a.tiles_m * a.tiles_n;
    const int grid = ntiles < d.cus ? ntiles : d.cus;
    hipLaunchKernelGGL((k_gemm_dma<KIND, EPI>), dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

// The ring kernel takes whole 64-byte K rows, at least a ring's worth of
// them (the ring then only ever holds stages of this tile and the next), at
// least one whole tile each way (edge tiles move inward), and 32-bit offsets
// inside a tile.
bool dma_gemm_fits(const GemmDesc &d, bool int4)
{
    const int64_t kb = int4 ? d.K / 2 : d.K;
    if (kb % kRowB != 0 || kb / kRowB < (int4 ? Geo<OP_S4>::kStages : Geo<OP_S8>::kStages))
        return false;
    if (d.M < kBM || d.N < kBN)
        return false;
    const int64_t lim = (int64_t)1 << 32;
    if ((kBM - 1) * d.lda_b + kb >= lim || (kBN - 1) * d.ldb_b + kb >= lim)
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

// int8 A x int4 B: whole 128-value K stages, at least a ring's worth, at
// least one whole tile each way, and 32-bit offsets inside a tile
bool dma_w4a8_fits(const GemmDesc &d)
{
    if (d.K % 128 != 0 || d.K / 128 < Geo<OP_MIX>::kStages)
        return false;
    if (d.M < kBM || d.N < kBN)
        return false;
    const int64_t lim = (int64_t)1 << 32;
    if ((kBM - 1) * d.lda_b + d.K >= lim || (kBN - 1) * d.ldb_b + d.K / 2 >= lim)
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
