// gemm.cpp -- the sidecar block's four projections as hipBLASLt GEMMs (MFMA
// kernels of the ROCm library; these are plain dense contractions, so the
// library's tuned kernels are used as they are).
//
// Row-major Y[M, N] = alpha * X[M, K] W[N, K]^T + beta * C is, column-major,
// Y^T = W X^T: A = W (stored K x N, transposed), B = X^T (K x M, as stored),
// the "TN" layout. The hipBLASLt handle and the algorithm chosen for each GEMM
// shape live in a context that the caller creates and destroys
// (r2l_gemm_context_create / _destroy), one per device; nothing here is
// file-scope state. The library's scratch is a slice of the caller's
// workspace. The algorithm is the library's first heuristic choice unless a
// tuning call has timed its candidates for that shape and found one at least
// 5% faster.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <new>
#include <tuple>

#include "r2l_scan.h"
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

constexpr int kTuneCandidates = 16;

Shape shape_of(int dev, int dtype, const GemmParams &g) {
    return Shape{dev, dtype, g.M, g.N, g.K, g.ldx, g.ldw, g.ldc, g.ldy, g.beta != 0.0f, g.ws_bytes};
}

void release(Prepared &p) {
    if (p.a) hipblasLtMatrixLayoutDestroy(p.a);
    if (p.b) hipblasLtMatrixLayoutDestroy(p.b);
    if (p.c) hipblasLtMatrixLayoutDestroy(p.c);
    if (p.d) hipblasLtMatrixLayoutDestroy(p.d);
    if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
    p = Prepared{};
}

// The matmul and matrix descriptors of shape s.
const char *describe(const Shape &s, Prepared *p) {
    const hipDataType t = s.dtype == 1 ? HIP_R_16BF : HIP_R_32F;
    if (hipblasLtMatmulDescCreate(&p->desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS)
        return "hipblasLtMatmulDescCreate failed";
    const int32_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
    hipblasLtMatmulDescSetAttribute(p->desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof(opT));
    hipblasLtMatmulDescSetAttribute(p->desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opN, sizeof(opN));
    if (hipblasLtMatrixLayoutCreate(&p->a, t, s.K, s.N, s.ldw) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&p->b, t, s.K, s.M, s.ldx) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&p->c, t, s.N, s.M, s.beta ? s.ldc : s.ldy) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&p->d, t, s.N, s.M, s.ldy) != HIPBLAS_STATUS_SUCCESS)
        return "hipblasLtMatrixLayoutCreate failed";
    return nullptr;
}

// The library's candidates for shape s, best first by its own heuristic.
const char *candidates(const Shape &s, hipblasLtHandle_t h, const Prepared &p, int want,
                       hipblasLtMatmulHeuristicResult_t *res, int *count) {
    hipblasLtMatmulPreference_t pref;
    if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS)
        return "hipblasLtMatmulPreferenceCreate failed";
    const uint64_t ws = s.ws;
    hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws,
                                          sizeof(ws));
    *count = 0;
    const hipblasStatus_t st = hipblasLtMatmulAlgoGetHeuristic(h, p.desc, p.a, p.b, p.c, p.d, pref,
                                                               want, res, count);
    hipblasLtMatmulPreferenceDestroy(pref);
    if (st != HIPBLAS_STATUS_SUCCESS || *count < 1) return "hipBLASLt has no algorithm for this GEMM";
    return nullptr;
}

}  // namespace
}  // namespace r2l

// The context behind r2l_gemm_context: one device's hipBLASLt handle and the
// prepared GEMM of every shape used with it. The mutex guards the plan map
// (calls from several host threads may share a context).
struct r2l_gemm_context_s {
    static constexpr uint32_t kMagic = 0x52324c47u;   // "R2LG"
    uint32_t magic = kMagic;
    int device = -1;
    hipblasLtHandle_t handle = nullptr;
    std::mutex mutex;
    std::map<r2l::Shape, r2l::Prepared> plans;
};

namespace r2l {

const char *gemm_context_create(r2l_gemm_context *out) {
    *out = nullptr;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return "hipGetDevice failed (no device?)";
    r2l_gemm_context c = new (std::nothrow) r2l_gemm_context_s;
    if (!c) return "out of host memory";
    c->device = dev;
    if (hipblasLtCreate(&c->handle) != HIPBLAS_STATUS_SUCCESS) {
        delete c;
        return "hipblasLtCreate failed";
    }
    *out = c;
    return nullptr;
}

const char *gemm_context_check(r2l_gemm_context c) {
    if (!c) return "the GEMM context is NULL";
    if (c->magic != r2l_gemm_context_s::kMagic) return "not a live GEMM context";
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return "hipGetDevice failed";
    if (dev != c->device) return "the GEMM context belongs to another device";
    return nullptr;
}

const char *gemm_context_destroy(r2l_gemm_context c) {
    if (!c || c->magic != r2l_gemm_context_s::kMagic) return "not a live GEMM context";
    int cur = 0;
    const bool switch_dev = hipGetDevice(&cur) == hipSuccess && cur != c->device;
    if (switch_dev) (void)hipSetDevice(c->device);
    for (auto &kv : c->plans) release(kv.second);
    const bool ok = hipblasLtDestroy(c->handle) == HIPBLAS_STATUS_SUCCESS;
    if (switch_dev) (void)hipSetDevice(cur);
    c->magic = 0;
    delete c;
    return ok ? nullptr : "hipblasLtDestroy failed";
}

const char *tune_gemm(r2l_gemm_context ctx, int dtype, const GemmParams &g, void *y_scratch,
                      hipStream_t stream) {
    if (g.M <= 0 || g.N <= 0) return nullptr;
    const Shape s = shape_of(ctx->device, dtype, g);
    std::lock_guard<std::mutex> lock(ctx->mutex);
    const char *err = nullptr;
    hipblasLtHandle_t h = ctx->handle;
    Prepared p;
    err = describe(s, &p);
    if (err) {
        release(p);
        return err;
    }
    hipblasLtMatmulHeuristicResult_t res[kTuneCandidates];
    int count = 0;
    err = candidates(s, h, p, kTuneCandidates, res, &count);
    if (err) {
        release(p);
        return err;
    }
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) {
        release(p);
        return "hipEventCreate failed";
    }
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        release(p);
        return "hipEventCreate failed";
    }
    void *Y = y_scratch ? y_scratch : g.Y;
    const float alpha = g.alpha, beta = g.beta;
    float best = -1.0f;
    int pick = 0;
    for (int i = 0; i < count && !err; ++i) {
        if (res[i].state != HIPBLAS_STATUS_SUCCESS || res[i].workspaceSize > g.ws_bytes) continue;
        auto run = [&]() {
            return hipblasLtMatmul(h, p.desc, &alpha, g.W, p.a, g.X, p.b, &beta,
                                   g.beta != 0.0f ? g.C : Y, p.c, Y, p.d, &res[i].algo,
                                   res[i].workspaceSize ? g.ws : nullptr, res[i].workspaceSize,
                                   stream);
        };
        if (run() != HIPBLAS_STATUS_SUCCESS || run() != HIPBLAS_STATUS_SUCCESS)
            continue;                                            // warm-up, and a validity check
        constexpr int kReps = 20;
        bool ok = true;
        if (hipEventRecord(e0, stream) != hipSuccess) {
            err = "hipEventRecord failed";
            break;
        }
        for (int r = 0; r < kReps && ok; ++r) ok = run() == HIPBLAS_STATUS_SUCCESS;
        if (hipEventRecord(e1, stream) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) {
            err = "hipEventRecord or hipEventSynchronize failed";
            break;
        }
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
            err = "hipEventElapsedTime failed";
            break;
        }
        if (!ok) continue;
        // keep the library's first choice unless another is clearly faster
        if (best < 0.0f || (pick == 0 && i > 0 ? ms < 0.95f * best : ms < best)) {
            best = ms;
            pick = i;
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (!err && best < 0.0f) err = "no hipBLASLt candidate ran";
    if (err) {
        release(p);
        return err;
    }
    auto it = ctx->plans.find(s);
    if (it != ctx->plans.end()) {   // keep the existing descriptors of this shape
        it->second.algo = res[pick].algo;
        it->second.ws = res[pick].workspaceSize;
        release(p);
    } else {
        p.algo = res[pick].algo;
        p.ws = res[pick].workspaceSize;
        ctx->plans[s] = p;
    }
    return nullptr;
}

const char *run_gemm(r2l_gemm_context ctx, int dtype, const GemmParams &g, hipStream_t stream) {
    if (g.M <= 0 || g.N <= 0) return nullptr;
    const Shape s = shape_of(ctx->device, dtype, g);
    hipblasLtHandle_t h = ctx->handle;
    Prepared p;
    {
        std::lock_guard<std::mutex> lock(ctx->mutex);
        auto it = ctx->plans.find(s);
        if (it == ctx->plans.end()) {
            const char *err = describe(s, &p);
            if (err) {
                release(p);
                return err;
            }
            hipblasLtMatmulHeuristicResult_t res[1];
            int count = 0;
            err = candidates(s, h, p, 1, res, &count);
            if (err) {
                release(p);
                return err;
            }
            p.algo = res[0].algo;
            p.ws = res[0].workspaceSize;
            ctx->plans[s] = p;
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
