// k_gemm_dma.hip -- the large-GEMM kernel: 256x256 output tiles on the
// gfx950 int8 MFMA, operands streamed global->LDS by the direct-to-LDS
// buffer loads (buffer_load_dwordx4 ... lds) through a 4-stage ring, with the
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
// Per workgroup (int8 x int8: 4 waves, 2x2, each owning 128x128 = 8x8 tiles
// of v_mfma_i32_16x16x64_i8, 256 accumulators; the int4 kinds: 8 waves, 2x4,
// each owning 128x64): the 16x16x64 shape, not
// 32x32x32, because under the board's power limit a stream of it runs at a
// higher engine clock (measured: 4.08 against 3.38 POP/s, 2045 against
// 1700 MHz, on random operands with the same 256 accumulators);
//   * a stage holds 64 bytes of K for the 256 A rows and 256 B rows (32 KB);
//     each wave fills a quarter of it with 8 direct-to-LDS loads.  A load
//     writes 64 lanes x 16 bytes contiguously, so the swizzle is chosen on
//     the source side: LDS slot (row, p) receives logical chunk
//     p ^ swz(row) of that row, which puts the 16 lanes of each LDS read
//     cycle of a fragment fetch (16 rows, one 16-byte chunk each) on 16
//     different bank groups.  The loads go
//     through buffer resources: a lane's offset inside a tile is one VGPR,
//     fixed for the whole walk, and the tile and stage enter as the scalar
//     offset, so the loop forms no per-lane addresses (a flat 64-bit address
//     per load cost about 2.5% of the s8s8 8192^3 time);
//   * three stages are in flight while one is multiplied.  A wave's
//     fragments of a stage are 8 A and 8 B row blocks of 16 rows; read
//     group 0 is A and B blocks 0..3, group 1 blocks 4..7.  The quadrants
//     (0,0), (0,1), (1,0) of the wave's 8x8 tiles multiply before the
//     stage's one barrier, (1,1) after it: group 1 streams in behind (0,0),
//     and the next stage's group 0 lands in the registers that (0,1) and
//     (1,0) freed, behind (1,1).  The barrier sits after this wave's loads
//     of the next stage have landed (counted with vmcnt);
//   * stage by stage, a wave's loads of a stage (8 for int8 x int8 on 4
//     waves, 6 for int8 x int4 on 8) are spread over two iterations (2
//     right after the barrier that frees their slot, the rest between the
//     next iteration's MFMAs), so the waves never queue all of them at once;
//   * int8 x int8 and int4 x int4, when K gives an even number (>= 4) of
//     stages, pair them instead: stages 2j and 2j+1 share one 64 KB slot of
//     128-byte rows, each load fetches 8 whole 128-byte lines, and the ring
//     is two such slots.  With 4 waves a second barrier, in the middle of a
//     pair's second stage, frees the slot for the pair after next: half of
//     that pair's loads go out there (two and a half stages to land), the
//     other half in the next pair's first stage, so that the four waves'
//     loads, issued at the same points of the same schedule, never queue
//     all at once at the CU's address unit; the int4 x int4 kernel
//     (8 waves, 2x4, each 128x64) keeps one barrier per pair.  int8 A facing
//     int4 B, whose A rows already take 128 bytes per stage, keeps a
//     3-stage ring of single stages;
//   * int4 operands are widened in registers: a 16-byte fragment read of
//     packed data covers two MFMA K steps.  int4 x int4 widens both sides
//     into the same even/odd order (dev_common.hpp); int8 A facing int4 B
//     widens B into natural order, whose 8-wave layout (each wave 128 rows
//     x 64 columns) reads twice as many A fragments as B ones;
//   * the grid is one workgroup per compute unit, walking its tiles; the
//     ring runs across tile boundaries (a tile's last stages issue the next
//     tile's first), and per-tile parameters come in by direct-to-LDS loads
//     into a double buffer, so a tile starts with its operands in LDS;
//   * the epilogue works from registers: a lane holds 4 adjacent columns
//     of one row per 16x16 tile; for four tiles side by side a 4x4
//     transpose over the 16-lane rows (v_permlane32_swap, then
//     v_permlane16_swap) gives it 16 adjacent int8 results, one 16-byte
//     store, a 16-row band at a time so that each output line fills from
//     consecutive stores.
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
#ifndef QG_DMA_EARLY_LOADS
#define QG_DMA_EARLY_LOADS 2
#endif
constexpr int kEarlyLoads = QG_DMA_EARLY_LOADS;  // issued right after the barrier
#ifndef QG_DMA_PAIRS
#define QG_DMA_PAIRS 1                        // paired stages for int8 / int4 operands
#endif
#ifndef QG_DMA_PAIR_EARLY
#define QG_DMA_PAIR_EARLY 1                   // 4-wave pairs: a second barrier, the next pair's loads earlier
#endif
#ifndef QG_DMA_PAIR_DEFER
#define QG_DMA_PAIR_DEFER 2                   // early form: quarters of a pair's loads issued in the stage after the rest
#endif
#ifndef QG_DMA_PAIR_EARLY_WAVES
#define QG_DMA_PAIR_EARLY_WAVES 4             // early form up to this many waves per workgroup
#endif
#ifndef QG_DMA_PAIR_FIRST
#define QG_DMA_PAIR_FIRST 4                   // quarters of a pair's loads issued in its first stage
#endif
// waves per workgroup: int4 x int4 and int8 x int4 run fastest with 8,
// int8 x int8 with 4 (measured)
#ifndef QG_DMA_WAVES
#define QG_DMA_WAVES 4
#endif
#ifndef QG_DMA_WAVES_MIX
#define QG_DMA_WAVES_MIX 8
#endif
#ifndef QG_DMA_MIX_NATURAL
#define QG_DMA_MIX_NATURAL 1                  // int8 x int4: widen B into A's natural byte order
#endif
#ifndef QG_DMA_WAVES_S4
#define QG_DMA_WAVES_S4 8
#endif
// NW waves per workgroup, 2 along M x NW/2 along N; every wave owns 128
// rows and kTN columns of the tile and loads kRPW of its A and B rows
template <int NW>
struct Waves {
    static_assert(NW == 4 || NW == 8, "2x2 or 2x4 waves");
    static constexpr int kWN = NW / 2;
    static constexpr int kTN = kBN / kWN;      // 128 or 64
    static constexpr int kNBJ = kTN / 16;      // 16-column tiles per wave
    static constexpr int kRPW = kBM / NW;      // rows per wave per operand per stage
};
#ifndef QG_DMA_GROUP_M
#define QG_DMA_GROUP_M 4
#endif
constexpr int kGroupM = QG_DMA_GROUP_M;      // tile rows that share B panels in L2

// 8 packed bytes (16 int4 values) -> 16 int8 bytes in natural order, each
// value scaled by 16 (dev_common.hpp's widen_int4_x16 gives the even/odd
// order): the low and high nibbles are masked in place as there, then
// interleaved by v_perm_b32, 5 instructions per packed dword against 3, and
// the int8 operand needs no permutation.  MSB: packed high nibble first, so
// the even elements are the high nibbles.
template <bool MSB>
__device__ __forceinline__ v4i widen_int4_x16_natural(v2u p)
{
    const unsigned lx = (p.x << 4) & 0xF0F0F0F0u, hx = p.x & 0xF0F0F0F0u;
    const unsigned ly = (p.y << 4) & 0xF0F0F0F0u, hy = p.y & 0xF0F0F0F0u;
    const unsigned ex = MSB ? hx : lx, ox = MSB ? lx : hx;
    const unsigned ey = MSB ? hy : ly, oy = MSB ? ly : hy;
    v4i r;
    r[0] = (int)__builtin_amdgcn_perm(ox, ex, 0x05010400u);
    r[1] = (int)__builtin_amdgcn_perm(ox, ex, 0x07030602u);
    r[2] = (int)__builtin_amdgcn_perm(oy, ey, 0x05010400u);
    r[3] = (int)__builtin_amdgcn_perm(oy, ey, 0x07030602u);
    return r;
}

// OP_MIX: int8 A x packed int4 B (W4A8); OP_MIXM: the same with B packed
// high nibble first
enum { OP_S8 = 8, OP_S4 = 4, OP_MIX = 3, OP_MIXM = 5 };

// Per operand kind: A bytes per row per stage, ring depth, direct-to-LDS
// loads per wave per stage.  A stage always covers 64 bytes of each B row;
// with int8 A facing int4 B that is 128 K values, so A rows take 128 bytes
// and the ring drops to three 48 KB stages.
template <int KIND, int NW>
struct Geo {
    static constexpr int kRPW = Waves<NW>::kRPW;
    static constexpr int kNBJ = Waves<NW>::kNBJ;
    static constexpr bool kMix = KIND == OP_MIX || KIND == OP_MIXM;
    static constexpr int kRowA = kMix ? 128 : kRowB;
    static constexpr int kStageA = kBM * kRowA;
    static constexpr int kStage = kStageA + kBN * kRowB;
    static constexpr int kStages = kMix ? 3 : QG_DMA_STAGES;
    static constexpr int kLoadsA = kRPW * kRowA / 1024;  // per wave: kRPW rows
    static constexpr int kLoadsB = kRPW * kRowB / 1024;
    static constexpr int kLoads = kLoadsA + kLoadsB;
    // LDS fragment reads per read group: 4 A blocks (two K steps each with
    // 128-byte A rows) and half the wave's B blocks
    static constexpr int kDsPerGroup = (kMix ? 8 : 4) + kNBJ / 2;
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
    uint32_t a_bytes, b_bytes;  // bytes of A and B the buffer loads may read
    int tiles_m, tiles_n;
    const int32_t *rterm;  // EPI_REQUANT_ZP: per-row term, or null
    int out_zero;          // EPI_REQUANT_ZP: output zero point
    int act_min, act_max;  // EPI_REQUANT_ZP: output clamp bounds
    const float *scale_a;  // EPI_F16: per-row scales, or null
    const float *scale_b;  // EPI_F16: per-column scales, or null
};

// A 16-byte LDS read is served 16 lanes per cycle over 64 4-byte banks
// (16 bank groups of 16 bytes); the lanes of one cycle share lane bit 5 and
// the parity of lane bits 2..4 (measured).  A fragment read gives lane L row
// L & 15 of a 16-row block and logical chunk L >> 4, so one cycle holds
// rows 0-3 and 12-15 at one chunk and rows 4-11 at the chunk next to it.
// With 64-byte rows a row's bank groups are 4 (r & 3) + chunk; XOR-ing the
// chunk with 3 * (row bit 3) makes the 16 (row, chunk) pairs of every cycle
// land on 16 different groups.
__device__ __forceinline__ int swz(int row) { return 3 * ((row >> 3) & 1); }
// 128-byte rows (int8 A facing int4 B, chunk 2 (L >> 4) + h for K step h):
// a row's groups are 8 (r & 1) + chunk, and XOR-ing the chunk (0..7) with
// row bit 1 and 4 * row bit 3 does the same for both steps.
__device__ __forceinline__ int swz8(int row) { return ((row >> 1) & 1) | (((row >> 3) & 1) << 2); }
// Paired stages (int8 and int4 operands): stages 2j and 2j+1 share a slot
// with 128-byte rows, stage 2j+h in chunks 4h .. 4h+3, read as chunk
// 4h + (L >> 4).  XOR-ing the chunk with row bits 1..3 spreads both halves'
// 16 reads of a cycle over the 16 bank groups.
__device__ __forceinline__ int swzp(int row) { return (row >> 1) & 7; }

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

template <int KIND, int EPI, bool PAIRS, int NW>
__global__ __launch_bounds__(NW * 64, 1) void k_gemm_dma(DmaArgs p)
{
    using G = Geo<KIND, NW>;
    constexpr int kWaves = NW;
    constexpr int kWN = Waves<NW>::kWN, kTN = Waves<NW>::kTN;
    constexpr int kNBJ = Waves<NW>::kNBJ, kRPW = Waves<NW>::kRPW;
    constexpr bool MIX = G::kMix;
    static_assert(!(PAIRS && MIX), "paired stages take 64-byte rows of both operands");
    // paired stages: slot of two stages, 128-byte rows, kLP loads per wave
    // per pair (8 rows x 128 bytes each), kLP1 of them in the pair's first
    // stage
    constexpr int kRowP = 2 * kRowB;
    constexpr int kPairA = kBM * kRowP;
    constexpr int kPair = kPairA + kBN * kRowP;
    constexpr int kLP = 2 * kRPW * kRowP / 1024;
    constexpr int kLP1 = kLP * QG_DMA_PAIR_FIRST / 4;
    static_assert(!PAIRS || 2 * kPair == G::kStages * G::kStage, "same LDS ring");
    // paired stages, early form: a second barrier in the middle of a pair's
    // second stage frees its slot for the pair after next, whose loads then
    // have two and a half stages to land instead of two.  Four waves gain
    // (their barrier waits were the longer); with eight, the int4 kind, the
    // extra barrier costs more than the earlier loads save.
    constexpr bool kPairEarly = PAIRS && QG_DMA_PAIR_EARLY && NW <= QG_DMA_PAIR_EARLY_WAVES;
    // early form: the first kEarly of pair j+2's loads go out after the
    // middle barrier of pair j, the other kDefer in the first stage of pair
    // j+1, so that the four waves' loads do not all queue in one window
    constexpr int kDefer = kPairEarly ? kLP * QG_DMA_PAIR_DEFER / 4 : 0;
    constexpr int kEarly = kLP - kDefer;
    static_assert(kDefer >= 0 && kEarly >= 1, "pair load split");
    constexpr bool MSB = KIND == OP_MIXM;
    constexpr int kStages = G::kStages;
    constexpr int kStage = G::kStage;
    constexpr int kStageA = G::kStageA;
    constexpr int kRowA = G::kRowA;
    constexpr int kLoadsPerStage = G::kLoads;
    // int8: a lane's 16-byte fragment is its 16 values of one 64-value K
    // step; int4: of two steps (int8 A facing int4 B reads two A fragments
    // per B fragment)
    constexpr int STEPS_PER_READ = KIND == OP_S8 ? 1 : 2;
    constexpr int ACC_SHIFT = KIND == OP_S4 ? 8 : (MIX ? 4 : 0);
    constexpr int MQ = 4 * (kNBJ / 2) * STEPS_PER_READ;  // MFMAs per quadrant of the wave's tiles
    constexpr int DSG = G::kDsPerGroup;
    // MFMAs of a stage before its barrier (quadrants (0,0), (0,1), (1,0))
    // and after it (quadrant (1,1), which covers the reads of the next
    // stage's group 0)
    constexpr int kMfmaPre = 3 * MQ;
    constexpr int kMfmaPost = MQ;
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
    const int wm = wave / kWN, wn = wave % kWN;

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
    constexpr int NSRC = PAIRS ? kLP : kLoadsPerStage;
    uint32_t src[NSRC];
    if constexpr (PAIRS) {
        // load i: A rows (i < kLP/2) or B rows, 8 rows of 128 bytes each;
        // lane L fetches logical chunk (L & 7) ^ swzp(row) of its row
#pragma unroll
        for (int i = 0; i < kLP; ++i) {
            const bool isb = i >= kLP / 2;
            const int r = wave * kRPW + (isb ? i - kLP / 2 : i) * 8 + (lane >> 3);
            const int c = (lane & 7) ^ swzp(r);
            src[i] = (uint32_t)r * (uint32_t)(isb ? p.ldb_b : p.lda_b) + c * 16;
        }
    } else {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        if constexpr (MIX) {
            const int r = wave * kRPW + i * 8 + (lane >> 3);
            const int c = (lane & 7) ^ swz8(r);
            src[i] = (uint32_t)r * (uint32_t)p.lda_b + c * 16;
        } else {
            const int r = wave * kRPW + i * 16 + (lane >> 2);
            const int c = (lane & 3) ^ swz(r);
            src[i] = (uint32_t)r * (uint32_t)p.lda_b + c * 16;
        }
    }
#pragma unroll
    for (int i = 0; i < G::kLoadsB; ++i) {
        const int r = wave * kRPW + i * 16 + (lane >> 2);
        const int c = (lane & 3) ^ swz(r);
        src[LA + i] = (uint32_t)r * (uint32_t)p.ldb_b + c * 16;
    }
    }

    // ---- per-tile parameters: this wave's 64 columns (and rows) of the
    //      tile, one 4-byte direct-to-LDS load per array; absent arrays are
    //      constants written once ----
    auto load_prm = [&](int buf, int m0, int n0) __attribute__((always_inline)) {
        // waves 0..3 cover the tile's 256 columns (and rows), 64 each
        if (kWaves > 4 && wave >= 4)
            return;
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
        if (tid >= kBN)
            break;
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
                       (isb ? kStageA + wave * (kRPW * kRowB) + (l - LA) * 1024
                            : wave * (kRPW * kRowA) + l * 1024);
        const int64_t off = isb ? (nxt ? b_nxt : b_cur) + (int64_t)s * kRowB
                                : (nxt ? a_nxt : a_cur) + (int64_t)s * kRowA;
        buffer_load_lds16(isb ? (const void *)p.B : (const void *)p.A,
                          isb ? p.b_bytes : p.a_bytes, src[l], (uint32_t)off, dst);
    };
    // paired stages: load l (0..kLP/2-1: A, the rest B) of pair jp (stages
    // 2jp, 2jp+1; jp >= nkt/2: the next tile's pair jp - nkt/2) into pair
    // slot `slot`
    auto issue_pair = [&](int jp, int slot, int l) __attribute__((always_inline)) {
        const bool nxt = 2 * jp >= nkt;
        const bool isb = l >= kLP / 2;
        uint8_t *dst = lds + slot * kPair +
                       (isb ? kPairA + wave * (kRPW * kRowP) + (l - kLP / 2) * 1024
                            : wave * (kRPW * kRowP) + l * 1024);
        const int64_t off = (isb ? (nxt ? b_nxt : b_cur) : (nxt ? a_nxt : a_cur)) +
                            (int64_t)jp * kRowP;
        buffer_load_lds16(isb ? (const void *)p.B : (const void *)p.A,
                          isb ? p.b_bytes : p.a_bytes, src[l], (uint32_t)off, dst);
    };

    // ---- fragment addresses inside a stage: lane L reads row L & 15 of a
    //      16-row block at logical chunk L >> 4 (with 128-byte A rows, chunks
    //      2 (L >> 4) and 2 (L >> 4) + 1, one per K step of the int4 B
    //      fragment).  The swizzles see row bits 1..3 only, so A block i is
    //      a fixed offset i * 16 * kRowA and B block j one of j * 16 * kRowB ----
    int a_rd[2], b_rd;
    // paired stages: A and B fragment addresses of stage half h
    int ap_rd[2], bp_rd[2];
    {
        const int ra = wm * 128 + (lane & 15);
        const int rb = wn * kTN + (lane & 15);
        const int c = lane >> 4;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            ap_rd[h] = ra * kRowP + (((4 * h + c) ^ swzp(ra)) << 4);
            bp_rd[h] = kPairA + rb * kRowP + (((4 * h + c) ^ swzp(rb)) << 4);
        }
        if constexpr (MIX) {
            a_rd[0] = ra * kRowA + (((2 * c) ^ swz8(ra)) << 4);
            a_rd[1] = ra * kRowA + (((2 * c + 1) ^ swz8(ra)) << 4);
        } else {
            a_rd[0] = a_rd[1] = ra * kRowA + ((c ^ swz(ra)) << 4);
        }
        b_rd = kStageA + rb * kRowB + ((c ^ swz(rb)) << 4);
    }

    // tile (i, j) of the wave's 8 x kNBJ: rows wm*128 + 16i .., columns
    // wn*kTN + 16j ..
    v4i acc[8 * kNBJ];

    // raw fragments of read groups 0 and 1: A blocks 4g .. 4g+3 (int8 A
    // facing int4 B: the second K step's in [4 + ..]) and the wave's B
    // blocks NB g .. NB g + NB - 1 (NB = kNBJ / 2)
    constexpr int NA = MIX ? 8 : 4;
    constexpr int NB = kNBJ / 2;
    v4i fa[2][NA], fb[2][NB];

    // in the order the MFMAs consume them: group 0 feeds quadrant (0,0)
    // first, group 1 quadrant (0,1) (its B blocks) before (1,0) (its A)
    // (paired stages: h is the stage's half of its pair slot)
    auto read_group = [&](int slot, int g, v4i(&ra)[NA], v4i(&rb)[NB], int h = 0) __attribute__((always_inline)) {
        const uint8_t *st = lds + slot * (PAIRS ? kPair : kStage);
        constexpr int pa = PAIRS ? kRowP : kRowA, pb = PAIRS ? kRowP : kRowB;
        const int ard = PAIRS ? ap_rd[h] : a_rd[0], brd = PAIRS ? bp_rd[h] : b_rd;
        auto rd_a = [&](int ii) __attribute__((always_inline)) {
            ra[ii] = *(const v4i *)(st + ard + (4 * g + ii) * 16 * pa);
            if constexpr (MIX)
                ra[4 + ii] = *(const v4i *)(st + a_rd[1] + (4 * g + ii) * 16 * kRowA);
        };
        auto rd_b = [&](int jj) __attribute__((always_inline)) {
            rb[jj] = *(const v4i *)(st + brd + (NB * g + jj) * 16 * pb);
        };
        if (g == 0) {
            rd_b(0);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                rd_a(ii);
#pragma unroll
            for (int jj = 1; jj < NB; ++jj)
                rd_b(jj);
        } else {
#pragma unroll
            for (int jj = 0; jj < NB; ++jj)
                rd_b(jj);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                rd_a(ii);
        }
    };

    // the 4x4 tiles of quadrant (qa, qb) from one A group and one B group
    auto mma_quad = [&](const v4i(&ra)[NA], const v4i(&rb)[NB], int qa, int qb) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < STEPS_PER_READ; ++h) {
            // int8 A facing int4 B: K step h of this group is A fragment
            // [4h + i], byte-permuted to the widened-int4 order once (or
            // taken as it is, with B widened into natural order)
            v4i as[MIX ? 4 : 1];
            if constexpr (MIX) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii)
                    as[ii] = QG_DMA_MIX_NATURAL ? ra[4 * h + ii] : even_odd_split<MSB>(ra[4 * h + ii]);
            }
#pragma unroll
            for (int jj = 0; jj < NB; ++jj) {
                v4i bq;
                if constexpr (KIND == OP_S8) {
                    bq = rb[jj];
                } else {
                    v2u w = {(unsigned)rb[jj][2 * h], (unsigned)rb[jj][2 * h + 1]};
                    if constexpr (MIX && QG_DMA_MIX_NATURAL)
                        bq = widen_int4_x16_natural<MSB>(w);
                    else
                        bq = widen_int4_x16(w);
                }
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    v4i aq;
                    if constexpr (KIND == OP_S8) {
                        aq = ra[ii];
                    } else if constexpr (MIX) {
                        aq = as[ii];
                    } else {
                        v2u w = {(unsigned)ra[ii][2 * h], (unsigned)ra[ii][2 * h + 1]};
                        aq = widen_int4_x16(w);
                    }
                    const int t = (4 * qa + ii) * kNBJ + NB * qb + jj;
                    acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bq, aq, acc[t], 0, 0, 0);
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
    if constexpr (kPairEarly) {
        // pairs 0 and 1 in slots 0 and 1; pair j+2 streams in from the
        // middle of pair j's second stage
#pragma unroll
        for (int l = 0; l < kLP; ++l)
            issue_pair(0, 0, l);
#pragma unroll
        for (int l = 0; l < kEarly; ++l)
            issue_pair(1, 1, l);
        wait_loads_and_barrier<kEarly>();
    } else if constexpr (PAIRS) {
        // paired stages: pair 0 in slot 0; pair 1 follows during pair 0
#pragma unroll
        for (int l = 0; l < kLP; ++l)
            issue_pair(0, 0, l);
        wait_loads_and_barrier<0>();
    } else {
#pragma unroll
        for (int s = 0; s < kStages - 1; ++s)
#pragma unroll
            for (int l = 0; l < kLoadsPerStage; ++l)
                issue(s, s, l);
#pragma unroll
        for (int l = 0; l < kEarlyLoads; ++l)
            issue(kStages - 1, kStages - 1, l);
        wait_loads_and_barrier<(kStages - 2) * kLoadsPerStage + kEarlyLoads>();
    }
    read_group(0, 0, fa[0], fb[0]);
    int rs = 0;  // ring slot (paired stages: pair slot) of the stage being multiplied

    // paired stages: the MFMA / LDS-read / load interleave of one stage,
    // NL loads before the stage's last quadrant
    auto pre_hints = [&]<int NL>() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < DSG; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        }
        if constexpr (NL > 0) {
            constexpr int per = (kMfmaPre - DSG) / NL;
            static_assert(per >= 1, "stage schedule");
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, per, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);    // VMEM read
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPre - DSG - per * NL, 0);
        } else {
            __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPre - DSG, 0);
        }
    };
    auto post_hints = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < DSG / 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kMfmaPost - DSG / 2, 0);
    };

    for (int k = 0;; ++k) {
#pragma unroll
        for (int t = 0; t < 8 * kNBJ; ++t)
            acc[t] = (v4i){0, 0, 0, 0};
        // paired stages: pair j multiplies from slot rs while pair j+1
        // lands in the other slot; pairs past the tile's last are the next
        // tile's first
        if constexpr (kPairEarly) {
            // two barriers per pair: once every wave has read its last
            // fragments of pair j (the middle of stage 2j+1), pair j+2
            // streams into slot rs; the pair's last barrier waits for pair
            // j+1 with pair j+2 still in flight
            for (int j = 0; j < nkt / 2; ++j) {
                const int ns = rs ^ 1;
                // stage 2j; the deferred loads of pair j+1 (slot ns has had
                // no reader since the middle of pair j-1)
                read_group(rs, 1, fa[1], fb[1], 0);
#pragma unroll
                for (int l = kEarly; l < kLP; ++l)
                    issue_pair(j + 1, ns, l);
                mma_quad(fa[0], fb[0], 0, 0);
                mma_quad(fa[0], fb[1], 0, 1);
                mma_quad(fa[1], fb[0], 1, 0);
                pre_hints.template operator()<kDefer>();
                __builtin_amdgcn_sched_barrier(0);
                read_group(rs, 0, fa[0], fb[0], 1);
                mma_quad(fa[1], fb[1], 1, 1);
                post_hints();
                __builtin_amdgcn_sched_barrier(0);
                // stage 2j + 1
                read_group(rs, 1, fa[1], fb[1], 1);
                mma_quad(fa[0], fb[0], 0, 0);
#pragma unroll
                for (int i = 0; i < DSG; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
                }
                __builtin_amdgcn_sched_group_barrier(0x008, MQ - DSG, 0);
                __builtin_amdgcn_sched_barrier(0);
                // this wave's reads of slot rs are back; after the barrier,
                // every wave's
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int l = 0; l < kEarly; ++l)
                    issue_pair(j + 2, rs, l);
                mma_quad(fa[0], fb[1], 0, 1);
                mma_quad(fa[1], fb[0], 1, 0);
                {
                    constexpr int per = 2 * MQ / kEarly;
                    static_assert(per >= 1, "stage schedule");
#pragma unroll
                    for (int i = 0; i < kEarly; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);    // VMEM read
                        __builtin_amdgcn_sched_group_barrier(0x008, per, 0);  // MFMA
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, 2 * MQ - per * kEarly, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                // all but pair j+2's first kEarly loads have landed for this
                // wave (a new tile's parameters are issued before its pair
                // 2), pair j+1's among them; after the barrier, for every
                // wave
                wait_loads_and_barrier<kEarly>();
                __builtin_amdgcn_sched_barrier(0);
                read_group(ns, 0, fa[0], fb[0], 0);
                mma_quad(fa[1], fb[1], 1, 1);
                post_hints();
                rs = ns;
            }
        } else if constexpr (PAIRS) {
            // one barrier per pair, after which pair j+1 has landed for
            // every wave and no wave reads pair j any more
            for (int j = 0; j < nkt / 2; ++j) {
                const int ns = rs ^ 1;
                // stage 2j (first half of the slot)
                read_group(rs, 1, fa[1], fb[1], 0);
#pragma unroll
                for (int l = 0; l < kLP1; ++l)
                    issue_pair(j + 1, ns, l);
                mma_quad(fa[0], fb[0], 0, 0);
                mma_quad(fa[0], fb[1], 0, 1);
                mma_quad(fa[1], fb[0], 1, 0);
                pre_hints.template operator()<kLP1>();
                __builtin_amdgcn_sched_barrier(0);
                read_group(rs, 0, fa[0], fb[0], 1);
                mma_quad(fa[1], fb[1], 1, 1);
                post_hints();
                __builtin_amdgcn_sched_barrier(0);
                // stage 2j + 1 (second half)
                read_group(rs, 1, fa[1], fb[1], 1);
#pragma unroll
                for (int l = kLP1; l < kLP; ++l)
                    issue_pair(j + 1, ns, l);
                mma_quad(fa[0], fb[0], 0, 0);
                mma_quad(fa[0], fb[1], 0, 1);
                mma_quad(fa[1], fb[0], 1, 0);
                pre_hints.template operator()<kLP - kLP1>();
                __builtin_amdgcn_sched_barrier(0);
                wait_loads_and_barrier<0>();
                __builtin_amdgcn_sched_barrier(0);
                read_group(ns, 0, fa[0], fb[0], 0);
                mma_quad(fa[1], fb[1], 1, 1);
                post_hints();
                rs = ns;
            }
        }
        // the last kStages - 1 stages issue the next tile's first loads (the
        // ring is never deeper than a tile: nkt >= kStages)
        for (int kt = 0; kt < (PAIRS ? 0 : nkt); ++kt) {
            // slots of stages kt + kStages - 1 (the one before rs) and kt + 1
            const int ps = rs == 0 ? kStages - 1 : rs - 1;
            const int ns = rs == kStages - 1 ? 0 : rs + 1;
            // group 1 of this stage streams in behind quadrant (0,0), and
            // the rest of stage kt+kStages-1 (its slot was freed at the last
            // barrier)
            read_group(rs, 1, fa[1], fb[1]);
#pragma unroll
            for (int l = kEarlyLoads; l < kLoadsPerStage; ++l)
                issue(kt + kStages - 1, ps, l);
            mma_quad(fa[0], fb[0], 0, 0);
            mma_quad(fa[0], fb[1], 0, 1);
            mma_quad(fa[1], fb[0], 1, 0);
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
            mma_quad(fa[1], fb[1], 1, 1);
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

        // ---- epilogue: for tile (i, j) a lane holds row
        //      ml = wm*128 + 16i + lane%16 and columns
        //      nl = wn*128 + 16j + 4 (lane/16) + e, e = 0..3, of the tile in
        //      acc[i*8 + j][e].  Its parameters landed before the last
        //      stage's barrier; the ring already holds the next tile's first
        //      stages ----
        int(*prm)[kBN] = prm_buf[k & 1];
        const int lane = fresh_lane();
        const int lg = lane >> 4;
        if constexpr (RQ) {
            // requantize with the cheapest exact form that every shift of
            // the tile allows (chosen once, so the accumulator indices stay
            // compile-time constants).  A lane packs the 4 results of each
            // tile into a dword; over four tiles side by side a 4x4
            // transpose across the 16-lane rows gives lane row g the 16
            // adjacent results of tile 4J + g, stored as one 16-byte write.
            const v4i sh4 = *(const v4i *)&prm[2][lane * 4];
            bool s33 = true, s31 = true;
            for (int e = 0; e < 4; ++e) {
                s33 = s33 && sh4[e] >= 33;
                s31 = s31 && sh4[e] >= 31;
            }
            int8_t *C = (int8_t *)p.C;
            // 16-byte stores need every row start and the tile's first
            // column on 16 bytes: an edge tile moved inward starts at
            // n0 = N - 256, which need not be
            const bool vec_ok = ((p.ldc | n0) & 15) == 0;
            auto requant_tile = [&](auto tier_tag) __attribute__((always_inline)) {
                constexpr int TIER = decltype(tier_tag)::value;
                // one 16-row band at a time, its 128 columns back to back,
                // so that each 128-byte line of a row is written by
                // consecutive stores (a line left partly written in L2 for
                // long is written back in pieces)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int ml = wm * 128 + i * 16 + (lane & 15);
                    const int rt = ZP ? prm[3][ml] : 0;
                    const int zo = ZP ? p.out_zero : 0;
                    const int lo = ZP ? p.act_min : -128, hi = ZP ? p.act_max : 127;
                    int8_t *row = C + (int64_t)(m0 + ml) * p.ldc + n0 + wn * kTN;
#pragma unroll
                    for (int J = 0; J < kNBJ / 4; ++J) {
                        unsigned d[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int j = 4 * J + q;
                            const int nl = wn * kTN + j * 16 + lg * 4;
                            const v4i b4 = *(const v4i *)&prm[0][nl];
                            const v4i m4 = *(const v4i *)&prm[1][nl];
                            const v4i s4 = *(const v4i *)&prm[2][nl];
                            int y[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                int a = acc[i * kNBJ + j][e] >> ACC_SHIFT;
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
                            // have landed.  The int8 x int8 forms are no
                            // faster with it.
                            if constexpr (MIX)
                                __builtin_amdgcn_sched_barrier(0);
                        }
                        // 4x4 transpose over the lane rows: row g receives
                        // dword g of rows 0..3, i.e. the 16 columns of tile
                        // 4J + g in order
                        const auto r02 = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
                        const auto r13 = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
                        const auto r01 = __builtin_amdgcn_permlane16_swap(r02[0], r13[0], false, false);
                        const auto r23 = __builtin_amdgcn_permlane16_swap(r02[1], r13[1], false, false);
                        const v4i out = {(int)r01[0], (int)r01[1], (int)r23[0], (int)r23[1]};
                        int8_t *dst = row + (4 * J + lg) * 16;
                        if (vec_ok) {
                            *(v4i *)dst = out;
                        } else {
                            for (int b = 0; b < 16; ++b)
                                dst[b] = (int8_t)(out[b >> 2] >> (8 * (b & 3)));
                        }
                        // four tiles' parameters in registers at a time:
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
            // binary16: a tile's 4 adjacent columns of one row per 8-byte
            // store, a 16-row band at a time so that each row's lines fill
            // from consecutive stores
            uint16_t *C = (uint16_t *)p.C;
            const bool vec = ((p.ldc | n0) & 3) == 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int ml = wm * 128 + i * 16 + (lane & 15);
                const float sa = __int_as_float(prm[3][ml]);
                uint16_t *row = C + (int64_t)(m0 + ml) * p.ldc + n0;
#pragma unroll
                for (int j = 0; j < kNBJ; ++j) {
                    const int nl = wn * kTN + j * 16 + lg * 4;
                    const v4i sb4 = *(const v4i *)&prm[0][nl];
                    unsigned short h[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float t = (float)(acc[i * kNBJ + j][e] >> ACC_SHIFT) * sa;
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
        } else {
            // raw int32: a tile's 4 adjacent columns of one row per 16-byte
            // store, a 16-row band at a time so that each row's lines fill
            // from consecutive stores
            int32_t *C = (int32_t *)p.C;
            const bool vec = ((p.ldc | n0) & 3) == 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int ml = wm * 128 + i * 16 + (lane & 15);
                int32_t *row = C + (int64_t)(m0 + ml) * p.ldc + n0;
#pragma unroll
                for (int j = 0; j < kNBJ; ++j) {
                    const int nl = wn * kTN + j * 16 + lg * 4;
                    v4i y;
                    for (int e = 0; e < 4; ++e)
                        y[e] = acc[i * kNBJ + j][e] >> ACC_SHIFT;
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
    a.a_bytes = (uint32_t)(d.M * d.lda_b);
    a.b_bytes = (uint32_t)(d.N * d.ldb_b);
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
    // paired stages for int8 and int4 operands whenever the stages pair up
    // (the ring then holds this tile's pair and the next one: >= 2 pairs)
    constexpr int NW = KIND == OP_S4 ? QG_DMA_WAVES_S4
                       : (KIND == OP_MIX || KIND == OP_MIXM) ? QG_DMA_WAVES_MIX
                                                               : QG_DMA_WAVES;
    constexpr bool kCanPair = !Geo<KIND, NW>::kMix && QG_DMA_PAIRS;
    const int64_t nkt = (KIND == OP_S8 ? d.K : d.K / 2) / kRowB;
    if (kCanPair && nkt % 2 == 0 && nkt >= 4)
        hipLaunchKernelGGL((k_gemm_dma<KIND, EPI, kCanPair, NW>), dim3(grid), dim3(NW * 64), 0, s, a);
    else
        hipLaunchKernelGGL((k_gemm_dma<KIND, EPI, false, NW>), dim3(grid), dim3(NW * 64), 0, s, a);
    return hipGetLastError();
}

}  // namespace

// The ring kernel takes whole 64-byte K rows, at least a ring's worth of
// them (the ring then only ever holds stages of this tile and the next), at
// least one whole tile each way (edge tiles move inward), and operands of
// under 4 GiB (32-bit buffer offsets).
bool dma_gemm_fits(const GemmDesc &d, bool int4)
{
    const int64_t kb = int4 ? d.K / 2 : d.K;
    if (kb % kRowB != 0 || kb / kRowB < (int4 ? Geo<OP_S4, QG_DMA_WAVES_S4>::kStages : Geo<OP_S8, QG_DMA_WAVES>::kStages))
        return false;
    if (d.M < kBM || d.N < kBN)
        return false;
    // each operand inside one 32-bit buffer range
    const int64_t lim = (int64_t)1 << 32;
    if (d.M * d.lda_b >= lim || d.N * d.ldb_b >= lim)
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
// least one whole tile each way, and operands of under 4 GiB
bool dma_w4a8_fits(const GemmDesc &d)
{
    if (d.K % 128 != 0 || d.K / 128 < Geo<OP_MIX, QG_DMA_WAVES_MIX>::kStages)
        return false;
    if (d.M < kBM || d.N < kBN)
        return false;
    const int64_t lim = (int64_t)1 << 32;
    if (d.M * d.lda_b >= lim || d.N * d.ldb_b >= lim)
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
