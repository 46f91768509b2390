// vendor_hipblaslt.cpp -- comparison leg of the benchmark (libqgvendor.so,
// not part of the quantized GEMM library or its ABI).  It times AMD's
// hipBLASLt int8 GEMM on the same shape as the ring kernel's workload, over
// every solution the library offers for the problem, so that the kernel is
// set against the library's best and not only against the solution its
// heuristic picks.
//
// The product: C[M][N] = A[M][K] * B[N][K]^T with int8 operands and int32
// accumulation and output (no requantize), i.e. the column-major problem
// D(N x M) = op_T(B: K x N) * op_N(A: K x M).
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt-ext.hpp>
#include <hipblaslt/hipblaslt.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

void copy_name(const std::string &s, char *dst, int len)
{
    if (!dst || len <= 0)
        return;
    const size_t n = std::min(s.size(), (size_t)len - 1);
    memcpy(dst, s.data(), n);
    dst[n] = 0;
}

}  // namespace

extern "C" {

// Times every applicable hipBLASLt solution of the int8 problem above:
// 2 untimed calls, then `reps` calls each between two events on `stream`;
// the median per solution.  A, B, D are device memory (D: M*N int32), ws a
// device workspace of ws_bytes.  Outputs: the heuristic pick's median and
// the best median in microseconds, the number of solutions timed, and the
// two solutions' kernel names.  On return D holds the best solution's
// result.  Returns 0, or a negative code: -1 library set-up failed, -2 no
// solution applies, -3 a launch or timing call failed.
int qgv_int8_gemm_search(const void *A, const void *B, void *D, int64_t M, int64_t N, int64_t K,
                         void *ws, int64_t ws_bytes, int reps, void *stream, double *heuristic_us,
                         double *best_us, int *n_timed, char *best_name, int best_len,
                         char *heur_name, int heur_len)
{
    hipStream_t st = (hipStream_t)stream;
    hipblasLtHandle_t h = nullptr;
    if (hipblasLtCreate(&h) != HIPBLAS_STATUS_SUCCESS)
        return -1;
    int rc = 0;
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
    hipblasLtMatmulPreference_t pref = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    const int32_t alpha = 1, beta = 0;
    const hipblasOperation_t opa = HIPBLAS_OP_T, opb = HIPBLAS_OP_N;
    const uint64_t wmax = (uint64_t)ws_bytes;
    std::vector<hipblasLtMatmulHeuristicResult_t> all;
    hipblasLtMatmulHeuristicResult_t heur[1];
    int nh = 0;

    auto time_one = [&](hipblasLtMatmulAlgo_t &algo, double &us) -> bool {
        for (int i = 0; i < 2; ++i)
            if (hipblasLtMatmul(h, desc, &alpha, B, la, A, lb, &beta, D, lc, D, lc, &algo, ws,
                                (size_t)ws_bytes, st) != HIPBLAS_STATUS_SUCCESS)
                return false;
        std::vector<float> t;
        for (int r = 0; r < reps; ++r) {
            if (hipEventRecord(e0, st) != hipSuccess)
                return false;
            if (hipblasLtMatmul(h, desc, &alpha, B, la, A, lb, &beta, D, lc, D, lc, &algo, ws,
                                (size_t)ws_bytes, st) != HIPBLAS_STATUS_SUCCESS)
                return false;
            float ms = 0;
            if (hipEventRecord(e1, st) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                hipEventElapsedTime(&ms, e0, e1) != hipSuccess)
                return false;
            t.push_back(ms * 1000.0f);
        }
        std::sort(t.begin(), t.end());
        us = t[t.size() / 2];
        return true;
    };

    if (hipblasLtMatmulDescCreate(&desc, HIPBLAS_COMPUTE_32I, HIP_R_32I) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opa, sizeof(opa)) !=
            HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opb, sizeof(opb)) !=
            HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&la, HIP_R_8I, K, N, K) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&lb, HIP_R_8I, K, M, K) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&lc, HIP_R_32I, N, M, N) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wmax,
                                              sizeof(wmax)) != HIPBLAS_STATUS_SUCCESS ||
        hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
        rc = -1;
        goto done;
    }
    *heuristic_us = -1;
    if (hipblasLtMatmulAlgoGetHeuristic(h, desc, la, lb, lc, lc, pref, 1, heur, &nh) ==
            HIPBLAS_STATUS_SUCCESS &&
        nh > 0) {
        double us;
        if (!time_one(heur[0].algo, us)) {
            rc = -3;
            goto done;
        }
        *heuristic_us = us;
        copy_name(hipblaslt_ext::getKernelNameFromAlgo(h, heur[0].algo), heur_name, heur_len);
    }
    if (hipblaslt_ext::getAllAlgos(h, hipblaslt_ext::GemmType::HIPBLASLT_GEMM, opa, opb, HIP_R_8I,
                                   HIP_R_8I, HIP_R_32I, HIP_R_32I, HIPBLAS_COMPUTE_32I, all) !=
        HIPBLAS_STATUS_SUCCESS) {
        rc = -2;
        goto done;
    }
    {
        double best = -1;
        int ibest = -1, n = 0;
        for (size_t i = 0; i < all.size(); ++i) {
            size_t need = 0;
            if (hipblaslt_ext::matmulIsAlgoSupported(h, desc, &alpha, la, lb, &beta, lc, lc,
                                                     all[i].algo, need) != HIPBLAS_STATUS_SUCCESS ||
                need > (size_t)ws_bytes)
                continue;
            double us;
            if (!time_one(all[i].algo, us)) {
                rc = -3;
                goto done;
            }
            ++n;
            if (best < 0 || us < best) {
                best = us;
                ibest = (int)i;
            }
        }
        *n_timed = n;
        if (ibest < 0) {
            rc = -2;
            goto done;
        }
        *best_us = best;
        copy_name(hipblaslt_ext::getKernelNameFromAlgo(h, all[ibest].algo), best_name, best_len);
        // leave the best solution's result in D
        double us;
        if (!time_one(all[ibest].algo, us))
            rc = -3;
    }
done:
    if (e0)
        hipEventDestroy(e0);
    if (e1)
        hipEventDestroy(e1);
    if (pref)
        hipblasLtMatmulPreferenceDestroy(pref);
    if (lc)
        hipblasLtMatrixLayoutDestroy(lc);
    if (lb)
        hipblasLtMatrixLayoutDestroy(lb);
    if (la)
        hipblasLtMatrixLayoutDestroy(la);
    if (desc)
        hipblasLtMatmulDescDestroy(desc);
    hipblasLtDestroy(h);
    return rc;
}

}  // extern "C"
