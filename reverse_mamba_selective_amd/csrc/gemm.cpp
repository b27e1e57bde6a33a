// gemm.cpp -- the sidecar block's four projections as hipBLASLt GEMMs (MFMA
// kernels of the ROCm library; these are plain dense contractions, so the
// library's tuned kernels are used as they are).
//
// Row-major Y[M, N] = alpha * X[M, K] W[N, K]^T + beta * C is, column-major,
// Y^T = W X^T: A = W (stored K x N, transposed), B = X^T (K x M, as stored),
// the "TN" layout. One hipBLASLt handle per device and one algorithm per
// GEMM shape are kept for the life of the process (host memory only); the
// library's scratch is a slice of the caller's workspace.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "scan_internal.h"

namespace r2l {
namespace {

struct Shape {
    int device, dtype;
    int64_t M, N, K, ldx, ldw, ldc, ldy;
    bool beta;
    size_t ws;
    bool operator<(const Shape &o) const {
        return std::tie(device, dtype, M, N, K, ldx, ldw, ldc, ldy, beta, ws) <
               std::tie(o.device, o.dtype, o.M, o.N, o.K, o.ldx, o.ldw, o.ldc, o.ldy, o.beta, o.ws);
    }
};

struct Prepared {
    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr, d = nullptr;
    hipblasLtMatmulAlgo_t algo{};
    size_t ws = 0;
};

std::mutex g_mutex;
std::map<int, hipblasLtHandle_t> g_handles;
std::map<Shape, Prepared> g_plans;

const char *prepare(const Shape &s, hipblasLtHandle_t h, Prepared *out) {
    const hipDataType t = s.dtype == 1 ? HIP_R_16BF : HIP_R_32F;
    Prepared p;
    if (hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS)
        return "hipblasLtMatmulDescCreate failed";
    const int32_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
    hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof(opT));
    hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opN, sizeof(opN));
    if (hipblasLtMatrixLayoutCreate(&p.a, t, s.K, s.N, s.ldw) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&p.b, t, s.K, s.M, s.ldx) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&p.c, t, s.N, s.M, s.beta ? s.ldc : s.ldy) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&p.d, t, s.N, s.M, s.ldy) != HIPBLAS_STATUS_SUCCESS)
        return "hipblasLtMatrixLayoutCreate failed";
    hipblasLtMatmulPreference_t pref;
    if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS)
        return "hipblasLtMatmulPreferenceCreate failed";
    const uint64_t ws = s.ws;
    hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws,
                                          sizeof(ws));
    hipblasLtMatmulHeuristicResult_t res[1];
    int count = 0;
    const hipblasStatus_t st = hipblasLtMatmulAlgoGetHeuristic(h, p.desc, p.a, p.b, p.c, p.d, pref,
                                                               1, res, &count);
    hipblasLtMatmulPreferenceDestroy(pref);
    if (st != HIPBLAS_STATUS_SUCCESS || count < 1) return "hipBLASLt has no algorithm for this GEMM";
    p.algo = res[0].algo;
    p.ws = res[0].workspaceSize;
    *out = p;
    return nullptr;
}

}  // namespace

const char *run_gemm(int dtype, const GemmParams &g, hipStream_t stream) {
    if (g.M <= 0 || g.N <= 0) return nullptr;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return "hipGetDevice failed";
    const Shape s{dev, dtype, g.M, g.N, g.K, g.ldx, g.ldw, g.ldc, g.ldy, g.beta != 0.0f, g.ws_bytes};
    hipblasLtHandle_t h;
    Prepared p;
    {
        std::lock_guard<std::mutex> lock(g_mutex);
        auto hit = g_handles.find(dev);
        if (hit == g_handles.end()) {
            if (hipblasLtCreate(&h) != HIPBLAS_STATUS_SUCCESS) return "hipblasLtCreate failed";
            g_handles[dev] = h;
        } else {
            h = hit->second;
        }
        auto it = g_plans.find(s);
        if (it == g_plans.end()) {
            const char *err = prepare(s, h, &p);
            if (err) return err;
            g_plans[s] = p;
        } else {
            p = it->second;
        }
    }
    const float alpha = g.alpha, beta = g.beta;
    const hipblasStatus_t st = hipblasLtMatmul(h, p.desc, &alpha, g.W, p.a, g.X, p.b, &beta,
                                               g.beta != 0.0f ? g.C : g.Y, p.c, g.Y, p.d, &p.algo,
                                               p.ws ? g.ws : nullptr, p.ws, stream);
    return st == HIPBLAS_STATUS_SUCCESS ? nullptr : "hipblasLtMatmul failed";
}

}  // namespace r2l
