// k_skinny_w4a8.hip -- weight-streaming GEMM for a few tokens of int8
// activations against packed int4 weights, with the Q31 requantize fused.
//
// With M <= 16 tokens the product does 64 int ops per packed weight byte,
// far below the MI355X ridge point, so the kernel is bound by reading the
// weights from HBM once.  (Arithmetic intensity as the bound: MCU conv
// front-end article, news.rkmt.cn/news/16638, §2.2; the requantize: same
// article §2.3; packed int4 operands: INT4 GEMM article,
// www.cf-1.com/news/6060138, §2.1.)
//
// What the memory system wants, measured on MI355X: every wave-wide load
// should cover 1 KB of contiguous bytes, and a CU should keep about one
// 64 KB burst in flight -- deeper rings of outstanding loads run slower, not
// faster (each XCD's L2 has to hold the lines in flight).  The MFMA operand
// layout wants the opposite (one lane per weight row), so the weights pass
// through LDS:
//   * one workgroup of 8 waves per CU walks a strided list of 16-row column
//     groups; a unit is one group times one K chunk of 8192 values
//     (16 rows x 4 KB), and units alternate between two 64 KB LDS slots;
//   * more than 16 tokens (up to 64) run as blocks side by side on the CUs,
//     32 tokens to a workgroup when K fits one chunk (each weight fragment
//     read and widened once feeds two MFMA chains), the blocks of one column
//     set on one XCD at the same time, so each weight byte is read from HBM
//     once (the other blocks read it from L2);
//   * the direct-to-LDS load (global_load_lds_dwordx4) writes lane L's 16
//     bytes at LDS offset 16*L of a 1 KB piece, so every load reads one
//     contiguous KB of one weight row; lane L fetches granule L ^ row of that
//     KB, which makes the reads below bank-conflict free;
//   * wave w multiplies K values [1024w, 1024w+1024) of the chunk: per
//     64-value step a lane needs 8 packed bytes of weight row lane%16, read
//     from LDS 16 bytes (two steps) at a time, widened in registers
//     (dev_common.hpp) and fed to v_mfma_i32_16x16x64_i8 with the
//     activations as the second operand;
//   * activations live in registers, loaded once when K <= 8192 and double-
//     buffered per unit otherwise; values past the end of K are zeroed, so
//     whatever sits in LDS there (clamped or stale bytes) adds nothing.
//     When K <= 8192, six of the eight waves bring theirs through LDS regions
//     that are idle until the first barrier, with loads in which
//     neighbouring lanes read contiguous bytes;
//   * one barrier per unit: after it, this unit's bytes have landed for every
//     wave and the other slot is free, so the next unit's loads go out at
//     once; the 8 partial 16x16 sums of a finished group are added by one
//     wave (rotating) behind the same barrier, requantized and kept in LDS
//     until the end.
#include "dev_common.hpp"
#include "launch.hpp"

namespace qg {

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

constexpr int kWaves = 8;
constexpr int kSteps = 16;                     // MFMA K steps (64 values) per wave per unit
constexpr int kChunk = kWaves * kSteps * 64;   // K values per unit (8192)
constexpr int kRowBytes = kChunk / 2;          // packed bytes per weight row per unit (4 KB)
constexpr int kSlot = 16 * kRowBytes;          // 64 KB
constexpr int kPieces = kRowBytes / 1024;      // 1 KB pieces per row per unit
constexpr int kLoads = 16 * kPieces / kWaves;  // direct-to-LDS loads per wave per unit (8)
constexpr int kMaxGroups = 32;                 // column groups per workgroup (LDS staging)
constexpr int kMaxGroups2 = 16;                // the same with two token blocks (32 tokens)

// LDS map, one object so that the compiler sees one buffer
constexpr int kRedOff = 2 * kSlot;                          // v4i red[2][kWaves][64]
constexpr int kPrmOff = kRedOff + 2 * kWaves * 64 * 16;     // int prm[3][kMaxGroups*16]
constexpr int kOutOff = kPrmOff + 3 * kMaxGroups * 16 * 4;  // unsigned outb[kMaxGroups][64]
constexpr int kLdsBytes = 160 * 1024;
static_assert(kOutOff + kMaxGroups * 64 * 4 <= kLdsBytes, "LDS budget");

struct SkinnyArgs {
    const int8_t *A;
    int64_t lda;  // bytes
    const uint8_t *B;
    int64_t ldb_b;  // bytes per packed weight row
    const int32_t *bias;
    const int32_t *mult;
    const int32_t *shift;
    int8_t *C;
    int64_t ldc;
    int M, N, K;
    int ngroups;  // ceil(N / 16)
};

// Wait until this wave's vector memory operations (the direct-to-LDS loads
// included) and LDS operations are done, then meet the other waves.
// The wait is the builtin, not inline asm, so that the compiler knows every
// load (direct-to-LDS ones included) has landed behind the barrier and adds
// no waits of its own for them.
__device__ __forceinline__ void drain_and_barrier()
{
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) expcnt(7) lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}

// Plain LDS barrier: this wave's LDS reads are done, then meet the other
// waves; loads in flight stay in flight.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ONE: K fits one chunk, so the activations are loaded once.
// TB: 16-token blocks per workgroup (1, or 2 when K fits one chunk).  With
// two, every weight fragment read from LDS and widened feeds two MFMA
// chains, the reduction buffer's two halves hold the two blocks (one group
// at a time, behind an extra barrier), and the results wait in the output
// block (16 groups at most) until the end, as with one block.
template <bool ONE, bool MSB, int TB>
__global__ __launch_bounds__(kWaves * 64, 1) void k_skinny_w4a8(SkinnyArgs p)
{
    static_assert(TB == 1 || (TB == 2 && ONE), "two token blocks need K within one chunk");
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
    v4i(*red)[kWaves][64] = (v4i(*)[kWaves][64])(lds + kRedOff);
    int(*prm)[kMaxGroups * 16] = (int(*)[kMaxGroups * 16])(lds + kPrmOff);
    unsigned(*outb)[64] = (unsigned(*)[64])(lds + kOutOff);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;  // weight row within the group / token index
    const int g = lane >> 4;    // 16-value group within a 64-value K step
    const int tok = blockIdx.y * 16 * TB + col;  // token of block 0; block b adds 16 b
    const int nchunks = ONE ? 1 : (p.K + kChunk - 1) / kChunk;
    const int KbB = p.K / 2;

    // groups of this workgroup: blockIdx.x + i * gridDim.x, i < ng
    const int ng = (p.ngroups - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    const int nunits = ng * nchunks;  // (group, chunk) units, group-major

    // group i of this workgroup
    auto group_of = [&](int i) { return (int)blockIdx.x + i * (int)gridDim.x; };

    // ---- activations: token rows past M read row M-1 (never stored) ----
    // value offset of (step s, lane group g) inside a wave's 1024 values: a
    // 16-byte weight read covers two steps, lane group g taking 32 values
    auto kofs = [&](int s) { return (s >> 1) * 128 + g * 32 + (s & 1) * 16; };
    auto load_acts = [&](int chunk, v4i(&af)[kSteps], int b = 0) {
        const int8_t *arow = p.A + (int64_t)min(tok + 16 * b, p.M - 1) * p.lda;
        const int kbase = chunk * kChunk + wave * (kSteps * 64);
#pragma unroll
        for (int s = 0; s < kSteps; ++s)
            af[s] = *(const v4i *)(arow + min(kbase + kofs(s), p.K - 16));
    };
    // zero the values at or past K, then match the widened int4 order
    auto fix_acts = [&](int chunk, v4i(&af)[kSteps]) {
        const int kbase = chunk * kChunk + wave * (kSteps * 64);
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            const int keep = kbase + kofs(s) < p.K ? -1 : 0;
            v4i q = af[s];
            for (int e = 0; e < 4; ++e)
                q[e] &= keep;
            af[s] = even_odd_split<MSB>(q);
        }
    };

    // ---- direct-to-LDS loads of unit u into slot `slot` ----
    // wave w loads rows 2w and 2w+1, kPieces KB each; a piece crossing or
    // lying past the end of the row reads clamped in-bounds addresses (those
    // LDS bytes meet zero activations).  Every wave issues exactly kLoads,
    // which the wait for the staged activations below counts on.
    auto issue = [&](int u, int slot) {
        const int i = u / nchunks, c = u - i * nchunks;
        const int grp = group_of(i);
#pragma unroll
        for (int l = 0; l < kLoads; ++l) {
            const int r = 2 * wave + l / kPieces, piece = l % kPieces;
            const int kb0 = c * kRowBytes + piece * 1024;  // packed byte offset in the row
            const int n = min(grp * 16 + r, p.N - 1);  // clamped rows are never stored
            const int kb = min(kb0 + ((lane ^ r) << 4), KbB - 16);
            uint8_t *dst = lds + slot * kSlot + (r * kPieces + piece) * 1024;
            __builtin_amdgcn_global_load_lds((const glb_void_t *)(p.B + (int64_t)n * p.ldb_b + kb),
                                             (lds_void_t *)dst, 16, 0, 0);
        }
    };

    // ---- LDS read addresses of this lane's 8 16-byte weight fragments ----
    // the fragment of steps 2l, 2l+1 is byte 512w + 64l + 16g of row `col`:
    // piece w/2, granule 32(w&1) + 4l + g, stored at granule ^ col
    int rd[kSteps / 2];
#pragma unroll
    for (int l = 0; l < kSteps / 2; ++l)
        rd[l] = (col * kPieces + (wave >> 1)) * 1024 + ((((wave & 1) * 32 + 4 * l + g) ^ col) << 4);

    v4i acc = {0, 0, 0, 0}, acc2 = {0, 0, 0, 0};  // acc2: the second token block
    v4i af2[TB == 2 ? kSteps : 1];
    auto consume = [&](int slot, const v4i(&af)[kSteps]) {
#pragma unroll
        for (int l = 0; l < kSteps / 2; ++l) {
            const v4i wl = *(const v4i *)(lds + slot * kSlot + rd[l]);
            const v2u lo = {(unsigned)wl[0], (unsigned)wl[1]};
            const v2u hi = {(unsigned)wl[2], (unsigned)wl[3]};
            const v4i wlo = widen_int4_x16(lo), whi = widen_int4_x16(hi);
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wlo, af[2 * l], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(whi, af[2 * l + 1], acc, 0, 0, 0);
            if constexpr (TB == 2) {
                acc2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(wlo, af2[2 * l], acc2, 0, 0, 0);
                acc2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(whi, af2[2 * l + 1], acc2, 0, 0, 0);
            }
        }
    };

    // one wave adds the 8 partial sums of group i and requantizes; the lane
    // holds token lane%16 and columns 4*(lane/16) + e of the group
    // two blocks: all 512 threads take one output value each (block b =
    // tid / 256; the partial sums of source lane L, value e at
    // red[b][v][L][e]: 16 lanes x 16 bytes contiguous per 64 threads, no
    // bank conflicts), then lanes e = 1..3 hand their byte to lane e = 0,
    // which puts the dword in the output block
    auto reduce2 = [&](int i) {
        const int b = tid >> 8, r = tid & 255, ls = r >> 2, e = r & 3;
        const int *rp = (const int *)&red[b][0][ls] + e;
        int sum = 0;
#pragma unroll
        for (int v = 0; v < kWaves; ++v)
            sum += rp[v * 64 * 4];
        const int c = i * 16 + 4 * (ls >> 4) + e;
        const int y = requant_one(sum >> 4, prm[0][c], prm[1][c], prm[2][c],
                                  1ll << ((prm[2][c] - 1) & 63));
        // lanes 4k .. 4k+3 hold e = 0..3: after two exchanges each holds all four bytes
        unsigned v = (unsigned)(y & 0xFF) << (8 * e);
        v |= (unsigned)__shfl_xor((int)v, 1);
        v |= (unsigned)__shfl_xor((int)v, 2);
        // kept in LDS until the end (token 16 b + ls % 16, column quad ls / 16):
        // stores here would sit in the count that the next unit's wait drains
        if (e == 0)
            outb[i * 2 + b][4 * (ls & 15) + (ls >> 4)] = v;
    };
    auto reduce = [&](int i) {
        if constexpr (TB == 2) {
            reduce2(i);
            return;
        }
        const int b = 0;
        if (wave != i % kWaves)
            return;
        const int rb = i & 1;
        v4i sum = red[rb][0][lane];
#pragma unroll
        for (int v = 1; v < kWaves; ++v) {
            const v4i x = red[rb][v][lane];
            for (int e = 0; e < 4; ++e)
                sum[e] += x[e];
        }
        const v4i b4 = *(const v4i *)&prm[0][i * 16 + 4 * g];
        const v4i m4 = *(const v4i *)&prm[1][i * 16 + 4 * g];
        const v4i s4 = *(const v4i *)&prm[2][i * 16 + 4 * g];
        int y[4];
        for (int e = 0; e < 4; ++e)
            y[e] = requant_one(sum[e] >> 4, b4[e], m4[e], s4[e], 1ll << ((s4[e] - 1) & 63));
        (void)b;
        outb[i][lane] = pack4_i8(y[0], y[1], y[2], y[3]);
    };

    // ---- per-column parameters of this workgroup's columns (at most
    // kMaxGroups * 16, one per thread), copied by 4-byte direct-to-LDS loads
    // at the end of the first unit (until its barrier their region holds
    // staged activations); the first reduce reads them a barrier later.  Loads into
    // registers here would make the compiler wait for every load in flight,
    // the next unit's included, before the first LDS read that follows. ----
    static_assert(kMaxGroups * 16 <= kWaves * 64, "one column per thread");
    auto load_prm = [&]() {
        if (tid < ng * 16) {
            const int n = min(group_of(tid >> 4) * 16 + (tid & 15), p.N - 1);
            if (p.bias)
                __builtin_amdgcn_global_load_lds((const glb_void_t *)(p.bias + n),
                                                 (lds_void_t *)&prm[0][wave * 64], 4, 0, 0);
            else
                prm[0][tid] = 0;
            __builtin_amdgcn_global_load_lds((const glb_void_t *)(p.mult + n),
                                             (lds_void_t *)&prm[1][wave * 64], 4, 0, 0);
            __builtin_amdgcn_global_load_lds((const glb_void_t *)(p.shift + n),
                                             (lds_void_t *)&prm[2][wave * 64], 4, 0, 0);
        }
    };
    // unit u: its bytes are in slot u&1 and its activations in `af`; the
    // next unit's loads (and activations, when K has several chunks) go out
    // right after the barrier
    v4i af0[kSteps], af1[kSteps];
    auto step = [&](int u, int slot, v4i(&af)[kSteps], v4i(&af_next)[kSteps]) {
        drain_and_barrier();
        if (u + 1 < nunits) {
            issue(u + 1, slot ^ 1);
            if (!ONE)
                load_acts((u + 1) % nchunks, af_next);
        }
        const int i = u / nchunks, c = u - i * nchunks;
        if (!ONE)
            fix_acts(c, af);
        if (c == 0 && i > 0) {
            reduce(i - 1);
            // two blocks share one buffer per block: its readers finish
            // before this group's partial sums overwrite it
            if constexpr (TB == 2)
                lds_barrier();
        }
        if (c == 0)
            acc = acc2 = (v4i){0, 0, 0, 0};
        consume(slot, af);
        if (c == nchunks - 1) {
            red[TB == 1 ? i & 1 : 0][wave][lane] = acc;
            if constexpr (TB == 2)
                red[1][wave][lane] = acc2;
        }
        // behind this unit's LDS reads: the compiler cannot tell the copy's
        // LDS range from the slot's and would wait for it before them
        if (u == 0)
            load_prm();
    };

    // ---- first activations.  A load in the MFMA layout touches 16 token
    // rows and 64 bytes of each, with neighbouring lanes on different rows;
    // loads in which neighbouring lanes read contiguous bytes pull the
    // 128 KB a CU needs 1 us faster per launch (measured).  Until the first
    // barrier, slot 1, the reduction buffer and the parameter and output
    // blocks (with the rest of the LDS) are unused: waves 0..5 copy
    // their 16 x 1 KB slices there with direct-to-LDS loads (token t's KB in
    // one instruction, lane L fetching granule L ^ t) and read them back in
    // the MFMA layout, granule G of token t at position G ^ t, which puts the
    // 16 lanes of every LDS read cycle on 16 different bank groups.  Waves
    // 6 and 7 load theirs directly.  A second token block goes through the
    // same regions in a second round.  K > kChunk keeps the direct loads. ----
    constexpr int kStagedWaves = 6;
    static_assert(4 * 16 * 1024 == kSlot && kPrmOff - kRedOff == 16 * 1024 &&
                      kLdsBytes - kPrmOff == 16 * 1024,
                  "staging regions: slot 1 for waves 0-3, the reduction buffer for wave 4, "
                  "the parameter and output blocks for wave 5");
    const bool staged = ONE && wave < kStagedWaves;
    const int stage_off = wave < 4 ? kSlot + wave * 16 * 1024 : wave == 4 ? kRedOff : kPrmOff;
    // One branch holds everything from the copies to the read-back: with two
    // tests of `staged`, the compiler assumed the other branch's direct
    // loads (into the same registers) pending and waited for every load,
    // the first unit's weights included, before the read-back.  A second
    // token block takes a second round through the same region once the
    // first round's reads are back (its wait also covers the weights, which
    // the first barrier needs anyway).
    if (staged) {
        const int kbase = wave * (kSteps * 64);
        // every workgroup copies the same activation bytes: each starts at
        // its own token, so that the workgroups of an XCD do not all read
        // the same L2 lines at once
        const int rot = (int)(blockIdx.x >> 3) & 15;
#pragma unroll
        for (int t0 = 0; t0 < 16; ++t0) {
            const int t = (t0 + rot) & 15;
            const int8_t *src = p.A + (int64_t)min(tok - col + t, p.M - 1) * p.lda +
                                min(kbase + 16 * (lane ^ t), p.K - 16);
            __builtin_amdgcn_global_load_lds((const glb_void_t *)src,
                                             (lds_void_t *)(lds + stage_off + t * 1024), 16, 0, 0);
        }
        issue(0, 0);
        // the copies above are done once at most kLoads later loads are out
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoads) : "memory");
#pragma unroll
        for (int s = 0; s < kSteps; ++s)
            af0[s] = *(const v4i *)(lds + stage_off + col * 1024 + (((kofs(s) >> 4) ^ col) << 4));
        if constexpr (TB == 2) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
            for (int t0 = 0; t0 < 16; ++t0) {
                const int t = (t0 + rot) & 15;
                const int8_t *src = p.A + (int64_t)min(tok - col + 16 + t, p.M - 1) * p.lda +
                                    min(kbase + 16 * (lane ^ t), p.K - 16);
                __builtin_amdgcn_global_load_lds((const glb_void_t *)src,
                                                 (lds_void_t *)(lds + stage_off + t * 1024), 16, 0, 0);
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
            for (int s = 0; s < kSteps; ++s)
                af2[s] = *(const v4i *)(lds + stage_off + col * 1024 + (((kofs(s) >> 4) ^ col) << 4));
        }
    } else {
        if constexpr (TB == 2)
            load_acts(0, af2, 1);
        load_acts(0, af0);
        issue(0, 0);
    }
    if (ONE)
        fix_acts(0, af0);
    if constexpr (TB == 2)
        fix_acts(0, af2);
    for (int u = 0; u < nunits; u += 2) {
        step(u, 0, af0, af1);
        if (u + 1 < nunits) {
            if (ONE)
                step(u + 1, 1, af0, af1);
            else
                step(u + 1, 1, af1, af0);
        }
    }
    drain_and_barrier();
    reduce(ng - 1);

    // ---- results: 16 tokens x 16 columns per group and token block, one
    // dword per lane (two blocks: outb rows 2i and 2i + 1, token-major) ----
    drain_and_barrier();
    if constexpr (TB == 2) {
        for (int j = tid >> 6; j < 2 * ng; j += kWaves) {
            const int i = j >> 1, t = tok - col + 16 * (j & 1) + (lane >> 2);
            const int n = group_of(i) * 16 + 4 * (lane & 3);
            if (t >= p.M || n >= p.N)
                continue;
            const unsigned v = outb[j][lane];
            int8_t *dst = p.C + (int64_t)t * p.ldc + n;
            if (n + 3 < p.N && (p.ldc & 3) == 0) {
                *(unsigned *)dst = v;
            } else {
                for (int e = 0; e < 4; ++e)
                    if (n + e < p.N)
                        dst[e] = (int8_t)(v >> (8 * e));
            }
        }
        return;
    }
    const bool tok_ok = tok < p.M;
    for (int i = wave; i < ng; i += kWaves) {
        const int n = group_of(i) * 16 + 4 * g;
        if (!tok_ok || n >= p.N)
            continue;
        const unsigned v = outb[i][lane];
        int8_t *dst = p.C + (int64_t)tok * p.ldc + n;
        if (n + 3 < p.N && (p.ldc & 3) == 0) {
            *(unsigned *)dst = v;
        } else {
            for (int e = 0; e < 4; ++e)
                if (n + e < p.N)
                    dst[e] = (int8_t)(v >> (8 * e));
        }
    }
}

}  // namespace

hipError_t launch_w4a8_skinny(const GemmDesc &d, hipStream_t s)
{
    SkinnyArgs a{};
    a.A = (const int8_t *)d.A;
    a.lda = d.lda_b;
    a.B = (const uint8_t *)d.B;
    a.ldb_b = d.ldb_b;
    a.bias = d.bias;
    a.mult = d.mult;
    a.shift = d.shift;
    a.C = (int8_t *)d.C;
    a.ldc = d.ldc;
    a.M = (int)d.M;
    a.N = (int)d.N;
    a.K = (int)d.K;
    a.ngroups = (int)((d.N + 15) / 16);
    // One workgroup per CU, but never more than kMaxGroups groups each.
    // Beyond 16 tokens with K within one chunk a workgroup takes two 16-token
    // blocks (32 tokens); the blocks of a grid row (grid_y > 1) share the CUs:
    // each gets a multiple of 8 workgroups, so that workgroups (x, y) and
    // (x, y') -- the same weight columns for different tokens, dispatched
    // round-robin over the 8 XCDs -- run at the same time on the same XCD,
    // and the weights come from HBM once and from that XCD's L2 for the
    // other blocks.
    const bool one = d.K <= kChunk;
    const int tb = one && d.M > 16 ? 2 : 1;
    const int grid_y = (int)((d.M + 16 * tb - 1) / (16 * tb));
    int grid_x = grid_y > 1 ? (d.cus / grid_y) & ~7 : d.cus;
    if (grid_x < 8)
        grid_x = 8;
    const int max_groups = tb == 2 ? kMaxGroups2 : kMaxGroups;
    if (grid_x * max_groups < a.ngroups)
        grid_x = (a.ngroups + max_groups - 1) / max_groups;
    if (grid_x > a.ngroups)
        grid_x = a.ngroups;
    const dim3 grid(grid_x, grid_y), block(kWaves * 64);
    if (tb == 2) {
        if (d.msb_first)
            hipLaunchKernelGGL((k_skinny_w4a8<true, true, 2>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((k_skinny_w4a8<true, false, 2>), grid, block, 0, s, a);
    } else if (d.msb_first) {
        if (one)
            hipLaunchKernelGGL((k_skinny_w4a8<true, true, 1>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((k_skinny_w4a8<false, true, 1>), grid, block, 0, s, a);
    } else {
        if (one)
            hipLaunchKernelGGL((k_skinny_w4a8<true, false, 1>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((k_skinny_w4a8<false, false, 1>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace qg
