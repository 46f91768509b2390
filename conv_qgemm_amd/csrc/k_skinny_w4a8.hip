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
// Layout of the work:
//   * a workgroup is 8 waves; K is cut into 8 slices, one per wave, of up
//     to 16 steps of 64 values, and the loop over K chunks of 8 slices
//     covers any K;
//   * each wave keeps its slice of the 16 activation rows in registers as
//     v_mfma_i32_16x16x64_i8 operands, loaded once per chunk (once in total
//     when K <= 8192) and byte-permuted to match the widened int4 order;
//   * the workgroup walks a strided list of 16-column groups; for each, every
//     wave streams its slice of the 16 weight rows with 16-byte loads (the
//     next group's loads are issued before this group's MFMAs), widens the
//     nibbles in registers and multiplies;
//   * the 8 partial 16x16 sums meet in LDS; one wave (rotating) adds them,
//     requantizes 4 adjacent columns per lane and stores one dword.
#include "dev_common.hpp"
#include "launch.hpp"

namespace qg {

namespace {

constexpr int kWaves = 8;
constexpr int kSteps = 16;               // MFMA K steps (64 values) per wave slice
constexpr int kLoads = kSteps / 2;       // 16-byte weight loads per lane per group
constexpr int kChunk = kWaves * kSteps * 64;  // K values per chunk (8192)

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

__global__ __launch_bounds__(kWaves * 64, 1) void k_skinny_w4a8(SkinnyArgs p)
{
    __shared__ __attribute__((aligned(16))) v4i red[2][kWaves][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 15;  // weight row within the group / token index
    const int g = lane >> 4;    // 16-value group within a 64-value K step
    const int t0 = blockIdx.y * 16;
    const int tok = t0 + col;
    const bool tok_ok = tok < p.M;
    const int nchunks = (p.K + kChunk - 1) / kChunk;
    const int KbB = p.K / 2;
    const v4i zero4 = {0, 0, 0, 0};

    // value offset of (step s, group g) inside a wave slice: loads cover two
    // steps, lane group g reading 32 consecutive values per load.
    auto kofs = [&](int s) { return (s >> 1) * 128 + g * 32 + (s & 1) * 16; };

    v4i af[kSteps];
    auto load_acts = [&](int chunk) {
        const int kbase = chunk * kChunk + wave * (kSteps * 64);
        const int8_t *arow = p.A + (int64_t)(tok_ok ? tok : 0) * p.lda;
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            const int k = kbase + kofs(s);
            v4i q = (tok_ok && k < p.K) ? *(const v4i *)(arow + k) : zero4;
            af[s] = even_odd_split(q);
        }
    };

    // weights of the group being multiplied, and of the next one in flight
    v4i wcur[kLoads], wnext[kLoads];
    auto load_weights = [&](int grp, int chunk, v4i (&dst)[kLoads]) {
        const int n = min(grp * 16 + col, p.N - 1);  // clamped columns are never stored
        const uint8_t *brow = p.B + (int64_t)n * p.ldb_b;
        const int kbase = chunk * kChunk + wave * (kSteps * 64);
#pragma unroll
        for (int l = 0; l < kLoads; ++l) {
            const int kb = (kbase + l * 128 + g * 32) / 2;  // packed byte offset
            dst[l] = kb < KbB ? *(const v4i *)(brow + kb) : zero4;
        }
    };

    if (nchunks == 1)
        load_acts(0);

    int it = 0;
    int grp = blockIdx.x;
    if (grp < p.ngroups)
        load_weights(grp, 0, wcur);
    for (; grp < p.ngroups; grp += gridDim.x, ++it) {
        v4i acc = zero4;
        for (int chunk = 0; chunk < nchunks; ++chunk) {
            if (nchunks > 1)
                load_acts(chunk);
            // prefetch the next (group, chunk) pair's weights
            int ngrp = grp, nchunk = chunk + 1;
            if (nchunk == nchunks) {
                ngrp = grp + gridDim.x;
                nchunk = 0;
            }
            if (ngrp < p.ngroups)
                load_weights(ngrp, nchunk, wnext);
#pragma unroll
            for (int l = 0; l < kLoads; ++l) {
                const v4i w = wcur[l];
                v2u lo = {(unsigned)w[0], (unsigned)w[1]};
                v2u hi = {(unsigned)w[2], (unsigned)w[3]};
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen_int4_x16(lo), af[2 * l], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen_int4_x16(hi), af[2 * l + 1], acc, 0, 0, 0);
            }
#pragma unroll
            for (int l = 0; l < kLoads; ++l)
                wcur[l] = wnext[l];
        }
        // lane holds token t0 + lane%16 and columns grp*16 + 4*(lane/16) + e
        red[it & 1][wave][lane] = acc;
        __syncthreads();
        if (wave == (it % kWaves)) {
            v4i sum = red[it & 1][0][lane];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) {
                v4i v = red[it & 1][w][lane];
                for (int e = 0; e < 4; ++e)
                    sum[e] += v[e];
            }
            const int n = grp * 16 + 4 * g;
            const bool vec = n + 3 < p.N && (p.ldc & 3) == 0;
            int y[4];
            for (int e = 0; e < 4; ++e) {
                const int nn = min(n + e, p.N - 1);
                const int b = p.bias ? p.bias[nn] : 0;
                const int m = p.mult[nn];
                const int s = p.shift[nn];
                y[e] = requant_one(sum[e] >> 4, b, m, s, 1ll << ((s - 1) & 63));
            }
            if (tok_ok && n < p.N) {
                int8_t *dst = p.C + (int64_t)tok * p.ldc + n;
                if (vec) {
                    *(unsigned *)dst = pack4_i8(y[0], y[1], y[2], y[3]);
                } else {
                    for (int e = 0; e < 4; ++e)
                        if (n + e < p.N)
                            dst[e] = (int8_t)y[e];
                }
            }
        }
    }
}

int num_cus()
{
    static int cached = 0;
    if (cached == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            n > 0)
            cached = n;
        else
            return 256;
    }
    return cached;
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
    const int grid_x = a.ngroups < num_cus() ? a.ngroups : num_cus();
    const int grid_y = (int)((d.M + 15) / 16);
    hipLaunchKernelGGL(k_skinny_w4a8, dim3(grid_x, grid_y), dim3(kWaves * 64), 0, s, a);
    return hipGetLastError();
}

}  // namespace qg
