// r2l_api.cpp -- host side of libr2l_scan.so: argument checks, planning and
// launches for the entry points declared in include/r2l_scan.h.
//
// Every check runs before anything is queued, so a failed call leaves device
// memory untouched. The library allocates nothing: chunked plans use the
// caller's workspace, whose size r2l_workspace_size reports for the same plan.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "r2l_scan.h"
#include "scan_internal.h"
#include "bounds_check.h"
#include "scan_plan.h"

namespace {

using r2l::elem_size;
using r2l::eff_bstride;
using r2l::Launch;
using r2l::max_len_of;
using r2l::Op;
using r2l::Plan;
using r2l::tokens_of;
using r2l::wants_readout;

thread_local char g_last_error[512] = "";

r2l_status fail(r2l_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

r2l_status ok() {
    g_last_error[0] = '\0';
    return R2L_OK;
}

bool ragged(const r2l_scan_args *a) { return r2l::is_ragged(a); }

// ---- shape checks shared by planning and the entry points -------------------
r2l_status check_shape(const r2l_scan_args *a) {
    if (!a) return fail(R2L_ERR_INVALID_ARG, "args is NULL");
    if (a->batch < 0) return fail(R2L_ERR_INVALID_ARG, "batch < 0");
    if (a->dim < 1) return fail(R2L_ERR_INVALID_ARG, "dim < 1");
    if (a->dim > 65535 * 16) return fail(R2L_ERR_UNSUPPORTED, "dim above 1048560");
    if (a->batch > INT32_MAX) return fail(R2L_ERR_UNSUPPORTED, "batch above 2^31-1");
    if (a->dstate != r2l::kN)
        return fail(R2L_ERR_UNSUPPORTED, "dstate %d is not built (only %d)", a->dstate, r2l::kN);
    if (a->dtype != R2L_DTYPE_F32 && a->dtype != R2L_DTYPE_BF16)
        return fail(R2L_ERR_UNSUPPORTED, "dtype %d is not built", a->dtype);
    if (a->delta_softplus != 0 && a->delta_softplus != 1)
        return fail(R2L_ERR_INVALID_ARG, "delta_softplus must be 0 or 1");
    if (a->state_split != 0 && a->state_split != 1 && a->state_split != 2 && a->state_split != 4)
        return fail(R2L_ERR_INVALID_ARG, "state_split must be 0, 1, 2 or 4");
    if (ragged(a)) {
        if (a->total_tokens < 0) return fail(R2L_ERR_INVALID_ARG, "total_tokens < 0");
        if (a->max_seqlen < 0) return fail(R2L_ERR_INVALID_ARG, "max_seqlen < 0");
        if (a->total_tokens > INT32_MAX)
            return fail(R2L_ERR_UNSUPPORTED, "ragged layout limited to 2^31-1 tokens (int32 offsets)");
        if (a->batch > 0 && a->max_seqlen > a->total_tokens)
            return fail(R2L_ERR_INVALID_ARG, "max_seqlen %lld exceeds total_tokens %lld",
                        (long long)a->max_seqlen, (long long)a->total_tokens);
        if (a->batch == 0 && a->total_tokens != 0)
            return fail(R2L_ERR_INVALID_ARG, "batch 0 with total_tokens != 0");
    } else {
        if (a->seqlen < 0) return fail(R2L_ERR_INVALID_ARG, "seqlen < 0");
        if (a->seqlen > INT32_MAX) return fail(R2L_ERR_UNSUPPORTED, "seqlen above 2^31-1");
    }
    return R2L_OK;
}

// ---- buffer checks -----------------------------------------------------------
struct Range {
    const char *name;
    uintptr_t lo, hi;  // [lo, hi), empty when lo == hi
    bool is_output;
};

Range span(const char *name, const void *p, int64_t rows, int64_t stride, int64_t cols, int64_t es,
           bool out) {
    Range r{name, 0, 0, out};
    if (!p || rows <= 0 || cols <= 0) return r;
    r.lo = reinterpret_cast<uintptr_t>(p);
    r.hi = r.lo + static_cast<uintptr_t>(((rows - 1) * stride + cols) * es);
    return r;
}

// Address span of a token-major tensor [tokens, cols] (either layout).
Range token_span(const char *name, const r2l_scan_args *a, const void *p, int64_t stride,
                 int64_t bstride, int64_t cols, int64_t es, bool out) {
    Range r{name, 0, 0, out};
    const int64_t tok = tokens_of(a);
    if (!p || tok <= 0 || cols <= 0) return r;
    int64_t extent;
    if (ragged(a)) {
        extent = (tok - 1) * stride + cols;
    } else {
        extent = (a->batch - 1) * eff_bstride(a, bstride, stride) + (a->seqlen - 1) * stride + cols;
    }
    r.lo = reinterpret_cast<uintptr_t>(p);
    r.hi = r.lo + static_cast<uintptr_t>(extent * es);
    return r;
}

bool overlap(const Range &x, const Range &y) {
    return x.lo < x.hi && y.lo < y.hi && x.lo < y.hi && y.lo < x.hi;
}

bool aligned(const void *p, uintptr_t al) { return (reinterpret_cast<uintptr_t>(p) % al) == 0; }

r2l_status check_buffers(Op op, const r2l_scan_args *a, const Plan &pl) {
    const int64_t tok = tokens_of(a);
    const int64_t D = a->dim, N = r2l::kN, es = elem_size(a->dtype);
    const bool readout = wants_readout(op, a);

    if (ragged(a) && a->batch > 0 && !a->cu_seqlens)
        return fail(R2L_ERR_INVALID_ARG, "cu_seqlens is NULL");
    if (tok > 0) {
        if (!a->x) return fail(R2L_ERR_INVALID_ARG, "x is NULL");
        if (!a->dt) return fail(R2L_ERR_INVALID_ARG, "dt is NULL");
        if (!a->Bm) return fail(R2L_ERR_INVALID_ARG, "Bm is NULL");
        if (readout && !a->Cm) return fail(R2L_ERR_INVALID_ARG, "Cm is NULL (readout requested)");
        if (readout && !a->out) return fail(R2L_ERR_INVALID_ARG, "out is NULL");
        if (a->x_stride < D) return fail(R2L_ERR_INVALID_ARG, "x_stride < dim");
        if (a->dt_stride < D) return fail(R2L_ERR_INVALID_ARG, "dt_stride < dim");
        if (a->Bm_stride < N) return fail(R2L_ERR_INVALID_ARG, "Bm_stride < dstate");
        if (readout && a->Cm_stride < N) return fail(R2L_ERR_INVALID_ARG, "Cm_stride < dstate");
        if (readout && a->out_stride < D) return fail(R2L_ERR_INVALID_ARG, "out_stride < dim");
        if (a->res && a->res_stride < D) return fail(R2L_ERR_INVALID_ARG, "res_stride < dim");
        if (a->x_batch_stride < 0 || a->dt_batch_stride < 0 || a->Bm_batch_stride < 0 ||
            a->Cm_batch_stride < 0 || a->res_batch_stride < 0 || a->out_batch_stride < 0)
            return fail(R2L_ERR_INVALID_ARG, "negative batch stride");
        if (readout && !ragged(a) && a->batch > 1 &&
            eff_bstride(a, a->out_batch_stride, a->out_stride) < a->seqlen * a->out_stride)
            return fail(R2L_ERR_ALIAS, "out: sequences overlap (batch stride < seqlen * stride)");
        // The kernels address the rows of one sequence with 32-bit byte offsets.
        const int64_t L = max_len_of(a);
        const struct { int64_t st, cols; } rows[] = {
            {a->x_stride, D}, {a->dt_stride, D}, {a->res ? a->res_stride : 0, D},
            {readout ? a->out_stride : 0, D}, {a->Bm_stride, N}, {readout ? a->Cm_stride : 0, N}};
        for (const auto &r : rows)
            if (L > 0 && r.st > 0 && ((L - 1) * r.st + r.cols) * es > (int64_t)UINT32_MAX)
                return fail(R2L_ERR_UNSUPPORTED, "one sequence spans more than 4 GiB of a tensor");
    }
    if (a->batch > 0 && !a->A) return fail(R2L_ERR_INVALID_ARG, "A is NULL");
    if (op == Op::Prefix && !a->h_out && !a->out)
        return fail(R2L_ERR_INVALID_ARG, "prefix_scan_state needs h_out or out");
    if (op == Op::Commit) {
        if (!a->h_out) return fail(R2L_ERR_INVALID_ARG, "block_commit_state needs h_out (the state)");
        if (a->h_in && a->h_in != a->h_out)
            return fail(R2L_ERR_INVALID_ARG, "block_commit_state: h_in must be NULL or equal h_out");
    }

    // alignment
    const struct { const void *p; uintptr_t al; const char *n; } al[] = {
        {a->x, (uintptr_t)es, "x"},     {a->dt, (uintptr_t)es, "dt"},   {a->Bm, (uintptr_t)es, "Bm"},
        {a->Cm, (uintptr_t)es, "Cm"},   {a->res, (uintptr_t)es, "res"}, {a->out, (uintptr_t)es, "out"},
        {a->A, 16, "A"},                {a->Dskip, 4, "Dskip"},         {a->h_in, 16, "h_in"},
        {a->h_out, 16, "h_out"},        {a->cu_seqlens, 4, "cu_seqlens"},
        {a->workspace, 256, "workspace"}};
    for (const auto &e : al)
        if (e.p && !aligned(e.p, e.al))
            return fail(R2L_ERR_MISALIGNED, "%s is not %u-byte aligned", e.n, (unsigned)e.al);

    if (pl.chunked && (!a->workspace || a->workspace_bytes < pl.ws_bytes))
        return fail(R2L_ERR_WORKSPACE, "chunked plan needs %zu workspace bytes, got %zu",
                    pl.ws_bytes, a->workspace ? a->workspace_bytes : (size_t)0);

    // aliasing
    const bool commit_inplace = (op == Op::Commit);
    std::vector<Range> rs = {
        token_span("x", a, a->x, a->x_stride, a->x_batch_stride, D, es, false),
        token_span("dt", a, a->dt, a->dt_stride, a->dt_batch_stride, D, es, false),
        token_span("Bm", a, a->Bm, a->Bm_stride, a->Bm_batch_stride, N, es, false),
        token_span("Cm", a, readout ? a->Cm : nullptr, a->Cm_stride, a->Cm_batch_stride, N, es,
                   false),
        token_span("res", a, readout ? a->res : nullptr, a->res_stride, a->res_batch_stride, D, es,
                   false),
        span("A", a->A, D, N, N, 4, false),
        span("Dskip", readout ? a->Dskip : nullptr, 1, D, D, 4, false),
        span("cu_seqlens", a->cu_seqlens, 1, a->batch + 1, a->batch + 1, 4, false),
        span("h_in", commit_inplace ? nullptr : a->h_in, a->batch, D * N, D * N, 4, false),
        token_span("out", a, readout ? a->out : nullptr, a->out_stride, a->out_batch_stride, D, es,
                   true),
        span("h_out", a->h_out, a->batch, D * N, D * N, 4, true),
        span("workspace", pl.chunked ? a->workspace : nullptr, 1, (int64_t)pl.ws_bytes,
             (int64_t)pl.ws_bytes, 1, true),
    };
    for (size_t i = 0; i < rs.size(); ++i) {
        for (size_t j = i + 1; j < rs.size(); ++j) {
            const Range &u = rs[i], &v = rs[j];
            if (!(u.is_output || v.is_output) || !overlap(u, v)) continue;
            const Range &o = u.is_output ? u : v;
            const Range &other = u.is_output ? v : u;
            const char *on = o.name, *tn = other.name;
            // allowed exact aliases
            if (!strcmp(on, "out") && (!strcmp(tn, "x") || !strcmp(tn, "res"))) {
                const bool is_x = !strcmp(tn, "x");
                const void *tp = is_x ? a->x : a->res;
                const int64_t ts = is_x ? a->x_stride : a->res_stride;
                const int64_t tbs = is_x ? a->x_batch_stride : a->res_batch_stride;
                if (tp == a->out && ts == a->out_stride &&
                    eff_bstride(a, tbs, ts) == eff_bstride(a, a->out_batch_stride, a->out_stride))
                    continue;
            }
            if (!strcmp(on, "h_out") && !strcmp(tn, "h_in") && a->h_in == a->h_out) continue;
            return fail(R2L_ERR_ALIAS, "%s overlaps %s", on, tn);
        }
    }
    return R2L_OK;
}

// Optional host-side check of device offsets (R2L_CHECK_SEQLENS=1).
r2l_status check_seqlens_on_device(const r2l_scan_args *a) {
    const char *env = getenv("R2L_CHECK_SEQLENS");
    if (!env || strcmp(env, "1") != 0 || !ragged(a) || a->batch == 0) return R2L_OK;
    std::vector<int32_t> cu(static_cast<size_t>(a->batch) + 1);
    hipError_t e = hipMemcpy(cu.data(), a->cu_seqlens, cu.size() * sizeof(int32_t),
                             hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(R2L_ERR_HIP, "cu_seqlens copy: %s", hipGetErrorString(e));
    if (cu[0] != 0) return fail(R2L_ERR_INVALID_ARG, "cu_seqlens[0] != 0");
    for (int64_t b = 0; b < a->batch; ++b) {
        const int64_t L = static_cast<int64_t>(cu[b + 1]) - cu[b];
        if (L < 0) return fail(R2L_ERR_INVALID_ARG, "cu_seqlens decreases at %lld", (long long)b);
        if (L > a->max_seqlen)
            return fail(R2L_ERR_INVALID_ARG, "sequence %lld longer than max_seqlen", (long long)b);
    }
    if (cu[a->batch] != a->total_tokens)
        return fail(R2L_ERR_INVALID_ARG, "cu_seqlens[batch] != total_tokens");
    return R2L_OK;
}

// ---- launching ----------------------------------------------------------------
r2l_status hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(R2L_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

r2l_status execute(const Launch *ls, int n, hipStream_t stream) {
    for (int i = 0; i < n; ++i) {
        const Launch &l = ls[i];
        hipError_t e = hipSuccess;
        const char *what = "segment scan launch";
        switch (l.kind) {
            case Launch::Segment:
                if (l.mode & r2l::kModeBias)
                    e = r2l::launch_sidecar_segment(l.dtype, l.mode, l.seg, stream);
                else if ((l.mode & r2l::kModeOutMask) == r2l::kModeWs || (l.mode & r2l::kModeAdd))
                    e = r2l::launch_bidir_segment(l.reverse, l.dtype, l.mode, l.seg, stream);
                else
                    e = r2l::launch_segment_scan(l.reverse, l.dtype, l.G, l.mode, l.seg, stream);
                break;
            case Launch::Conv:
                e = r2l::launch_conv(l.dtype, l.conv, stream);
                what = "sidecar conv launch";
                break;
            case Launch::Gemm: {
                const char *err = r2l::run_gemm(l.gemm.ctx, l.dtype, l.gemm, stream);
                if (err) return fail(R2L_ERR_HIP, "sidecar projection: %s", err);
                break;
            }
            case Launch::Bidir:
                e = r2l::launch_bidir_fused(l.dtype, l.mode & r2l::kModeOutMask,
                                            (l.mode & r2l::kModeLds) != 0, l.seg, l.seg2,
                                            stream);
                what = "bidirectional scan launch";
                break;
            case Launch::Carry:
                e = r2l::launch_carry(l.carry, stream);
                what = "carry launch";
                break;
            case Launch::Copy:
                e = r2l::launch_copy(l.dtype, l.copy, stream);
                what = "residual copy launch";
                break;
            case Launch::Backward:
                e = r2l::launch_backward(l.reverse, l.dtype, l.G, l.bwd, stream);
                what = "backward launch";
                break;
            case Launch::Sum:
                e = r2l::launch_sums(l.sums, stream);
                what = "gradient sum launch";
                break;
        }
        r2l_status st = hip_status(e, what);
        if (st != R2L_OK) return st;
    }
    return ok();
}

r2l_status run(Op op, const r2l_scan_args *a, hipStream_t stream, bool device_check = true) {
    r2l_status st = check_shape(a);
    if (st != R2L_OK) return st;
    const Plan pl = r2l::make_plan(op, a);
    st = check_buffers(op, a, pl);
    if (st != R2L_OK) return st;
    if (device_check) {
        st = check_seqlens_on_device(a);
        if (st != R2L_OK) return st;
    }
    if (a->batch * pl.nchunks * pl.tiles > INT32_MAX - 8)
        return fail(R2L_ERR_UNSUPPORTED, "grid too large");

    Launch ls[3];
    const int n = r2l::build_launches(op, a, pl, ls);
    return execute(ls, n, stream);
}

// ---- saved checkpoints ------------------------------------------------------------
// The checkpoint buffer is one more output of the forward (and an input of the
// backward): 16-byte aligned, large enough, overlapping no other buffer.
r2l_status check_ckpt(const r2l_scan_args *a, const void *ckpt, size_t bytes, bool is_output,
                      const void *workspace, size_t ws_bytes) {
    const size_t need = r2l::checkpoint_bytes(a);
    if (need == 0) return R2L_OK;
    if (!ckpt) return fail(R2L_ERR_INVALID_ARG, "ckpt is NULL");
    if (!aligned(ckpt, 16)) return fail(R2L_ERR_MISALIGNED, "ckpt is not 16-byte aligned");
    if (bytes < need)
        return fail(R2L_ERR_WORKSPACE, "the checkpoints need %zu bytes, got %zu", need, bytes);
    const int64_t D = a->dim, N = r2l::kN, es = elem_size(a->dtype), B = a->batch;
    const Range c{"ckpt", reinterpret_cast<uintptr_t>(ckpt), reinterpret_cast<uintptr_t>(ckpt) + need,
                  is_output};
    const Range others[] = {
        token_span("x", a, a->x, a->x_stride, a->x_batch_stride, D, es, false),
        token_span("dt", a, a->dt, a->dt_stride, a->dt_batch_stride, D, es, false),
        token_span("Bm", a, a->Bm, a->Bm_stride, a->Bm_batch_stride, N, es, false),
        token_span("Cm", a, a->Cm, a->Cm_stride, a->Cm_batch_stride, N, es, false),
        token_span("res", a, a->res, a->res_stride, a->res_batch_stride, D, es, false),
        token_span("out", a, a->out, a->out_stride, a->out_batch_stride, D, es, true),
        span("A", a->A, D, N, N, 4, false),
        span("Dskip", a->Dskip, 1, D, D, 4, false),
        span("h_in", a->h_in, B, D * N, D * N, 4, false),
        span("h_out", a->h_out, B, D * N, D * N, 4, true),
        span("cu_seqlens", a->cu_seqlens, 1, B + 1, B + 1, 4, false),
        span("workspace", workspace, 1, (int64_t)ws_bytes, (int64_t)ws_bytes, 1, true)};
    for (const Range &o : others)
        if ((is_output || o.is_output) && overlap(c, o))
            return fail(R2L_ERR_ALIAS, "ckpt overlaps %s", o.name);
    return R2L_OK;
}

// op: Scan (r2l_scan_save) or Prefix (prefix_scan_save)
r2l_status prepare_save(Op op, const r2l_scan_args *a, r2l_scan_args *v, Plan *pl) {
    r2l_status st = check_shape(a);
    if (st != R2L_OK) return st;
    if (a->state_split > 1)
        return fail(R2L_ERR_UNSUPPORTED, "%s runs one lane per channel (state_split 0 or 1)",
                    op == Op::Scan ? "r2l_scan_save" : "prefix_scan_save");
    *v = *a;
    v->state_split = 1;
    *pl = r2l::make_plan(op, v, true);
    st = check_buffers(op, v, *pl);
    if (st != R2L_OK) return st;
    if (v->batch * pl->nchunks * pl->tiles > INT32_MAX - 8)
        return fail(R2L_ERR_UNSUPPORTED, "grid too large");
    return R2L_OK;
}

r2l_status run_save(Op op, const r2l_scan_args *a, float *ckpt, size_t ckpt_bytes,
                    hipStream_t stream) {
    r2l_scan_args v;
    Plan pl;
    r2l_status st = prepare_save(op, a, &v, &pl);
    if (st != R2L_OK) return st;
    st = check_ckpt(&v, ckpt, ckpt_bytes, true, pl.chunked ? v.workspace : nullptr,
                    pl.chunked ? pl.ws_bytes : 0);
    if (st != R2L_OK) return st;
    st = check_seqlens_on_device(&v);
    if (st != R2L_OK) return st;
    Launch ls[r2l::kMaxSaveLaunches];
    const int n = r2l::build_save_launches(op, &v, pl, ckpt, ls);
    return execute(ls, n, stream);
}

// ---- bidirectional scan -----------------------------------------------------------
// Each direction is checked as a scan with readout into out: the forward one
// with the call's residual and states, the reverse one with its own
// parameters and neither residual nor state (so that out may be
// exactly x but overlaps nothing else of either direction), both without the
// workspace, which is then checked against every buffer of both.
r2l_status check_bidir(const r2l_scan_args *a, const r2l_dir_args *rev, const r2l::BidirPlan &bp) {
    if (a->state_split > 1)
        return fail(R2L_ERR_UNSUPPORTED, "bidir_scan runs one lane per channel (state_split 0 or 1)");
    const int64_t tok = tokens_of(a);
    if (tok > 0 && !a->out) return fail(R2L_ERR_INVALID_ARG, "out is NULL");
    Plan bare = bp.pl;
    bare.chunked = false;
    r2l_scan_args f = *a;
    f.workspace = nullptr;
    f.workspace_bytes = 0;
    r2l_status st = check_buffers(Op::Scan, &f, bare);   // (a readout is always wanted)
    if (st != R2L_OK) return st;
    r2l_scan_args r = r2l::reverse_view(&f, rev);
    st = check_buffers(Op::Scan, &r, bare);
    if (st != R2L_OK) return st;
    if (bp.readout && a->dim * r2l::max_len_of(a) * 4 > (int64_t)UINT32_MAX)
        return fail(R2L_ERR_UNSUPPORTED, "one sequence's fp32 rows span more than 4 GiB");
    if (bp.ws_bytes == 0) return R2L_OK;
    if (!a->workspace || a->workspace_bytes < bp.ws_bytes)
        return fail(R2L_ERR_WORKSPACE, "bidir_scan needs %zu workspace bytes, got %zu", bp.ws_bytes,
                    a->workspace ? a->workspace_bytes : (size_t)0);
    if (!aligned(a->workspace, 256)) return fail(R2L_ERR_MISALIGNED, "workspace is not 256-byte aligned");
    const int64_t D = a->dim, N = r2l::kN, es = elem_size(a->dtype);
    const Range ws = span("workspace", a->workspace, 1, (int64_t)bp.ws_bytes, (int64_t)bp.ws_bytes, 1, true);
    const Range others[] = {
        token_span("x", a, a->x, a->x_stride, a->x_batch_stride, D, es, false),
        token_span("dt", a, a->dt, a->dt_stride, a->dt_batch_stride, D, es, false),
        token_span("Bm", a, a->Bm, a->Bm_stride, a->Bm_batch_stride, N, es, false),
        token_span("Cm", a, a->Cm, a->Cm_stride, a->Cm_batch_stride, N, es, false),
        token_span("reverse dt", a, r.dt, r.dt_stride, r.dt_batch_stride, D, es, false),
        token_span("reverse Bm", a, r.Bm, r.Bm_stride, r.Bm_batch_stride, N, es, false),
        token_span("reverse Cm", a, r.Cm, r.Cm_stride, r.Cm_batch_stride, N, es, false),
        token_span("res", a, a->res, a->res_stride, a->res_batch_stride, D, es, false),
        token_span("out", a, a->out, a->out_stride, a->out_batch_stride, D, es, false),
        span("A", a->A, D, N, N, 4, false),
        span("reverse A", r.A, D, N, N, 4, false),
        span("Dskip", a->Dskip, 1, D, D, 4, false),
        span("reverse Dskip", r.Dskip, 1, D, D, 4, false),
        span("cu_seqlens", a->cu_seqlens, 1, a->batch + 1, a->batch + 1, 4, false),
        span("h_in", a->h_in, a->batch, D * N, D * N, 4, false),
        span("h_out", a->h_out, a->batch, D * N, D * N, 4, false),
    };
    for (const Range &o : others)
        if (overlap(ws, o)) return fail(R2L_ERR_ALIAS, "workspace overlaps %s", o.name);
    return R2L_OK;
}

r2l_status prepare_bidir(const r2l_scan_args *a, const r2l_dir_args *rev, r2l::BidirPlan *bp) {
    r2l_status st = check_shape(a);
    if (st != R2L_OK) return st;
    *bp = r2l::make_bidir_plan(a);
    st = check_bidir(a, rev, *bp);
    if (st != R2L_OK) return st;
    if (a->batch * bp->pl.nchunks * bp->pl.tiles > INT32_MAX - 8)
        return fail(R2L_ERR_UNSUPPORTED, "grid too large");
    return R2L_OK;
}

r2l_status run_bidir(const r2l_scan_args *a, const r2l_dir_args *rev, hipStream_t stream) {
    r2l::BidirPlan bp;
    r2l_status st = prepare_bidir(a, rev, &bp);
    if (st != R2L_OK) return st;
    st = check_seqlens_on_device(a);
    if (st != R2L_OK) return st;
    Launch ls[r2l::kMaxBidirLaunches];
    const int n = r2l::build_bidir_launches(a, rev, bp, ls);
    return execute(ls, n, stream);
}

// ---- sidecar block ------------------------------------------------------------------
r2l_status check_sidecar(const r2l_sidecar_args *a, const r2l::SidecarPlan &sp) {
    const int64_t tok = sp.tokens, di = a->d_inner, dm = a->d_model;
    const int64_t es = elem_size(a->dtype);
    if (a->d_model < 1 || a->d_inner < 1) return fail(R2L_ERR_INVALID_ARG, "d_model and d_inner must be >= 1");
    if (a->d_model % 8 || a->d_inner % 8)
        return fail(R2L_ERR_UNSUPPORTED, "d_model and d_inner must be multiples of 8");
    if (a->dt_rank < 1) return fail(R2L_ERR_INVALID_ARG, "dt_rank < 1");
    if (a->dt_rank % 8) return fail(R2L_ERR_UNSUPPORTED, "dt_rank must be a multiple of 8");
    if (a->d_conv < 1 || a->d_conv > r2l::kConvMaxTaps)
        return fail(R2L_ERR_UNSUPPORTED, "d_conv must be 1..%d", r2l::kConvMaxTaps);
    if (tok == 0) return R2L_OK;
    const struct { const void *p; const char *n; bool need; } req[] = {
        {a->hidden, "hidden", true}, {a->out, "out", true}, {a->W_in, "W_in", sp.runs},
        {a->conv_w, "conv_w", sp.runs}, {a->W_x, "W_x", sp.runs}, {a->W_dt, "W_dt", sp.runs},
        {a->A, "A", sp.runs}, {a->W_out, "W_out", sp.runs}};
    for (const auto &r : req)
        if (r.need && !r.p) return fail(R2L_ERR_INVALID_ARG, "%s is NULL", r.n);
    if (a->hidden_stride < dm || a->out_stride < dm)
        return fail(R2L_ERR_INVALID_ARG, "hidden or out stride < d_model");
    // the GEMM operands: 16-byte aligned rows
    const struct { const void *p; int64_t ld; const char *n; } al[] = {
        {a->hidden, a->hidden_stride, "hidden"}, {a->out, a->out_stride, "out"},
        {a->W_in, dm, "W_in"}, {a->W_x, di, "W_x"}, {a->W_dt, a->dt_rank, "W_dt"},
        {a->W_out, di, "W_out"}};
    for (const auto &e : al)
        if (e.p && (!aligned(e.p, 16) || (e.ld * es) % 16))
            return fail(R2L_ERR_MISALIGNED, "%s: rows must start on 16-byte boundaries", e.n);
    const struct { const void *p; const char *n; } f4[] = {
        {a->conv_w, "conv_w"}, {a->conv_b, "conv_b"}, {a->dt_bias, "dt_bias"}, {a->A, "A"},
        {a->Dskip, "Dskip"}, {a->cu_seqlens, "cu_seqlens"}};
    for (const auto &e : f4)
        if (e.p && !aligned(e.p, 4)) return fail(R2L_ERR_MISALIGNED, "%s is not 4-byte aligned", e.n);
    if (!sp.runs && !(a->out == a->hidden && a->out_stride == a->hidden_stride)) {
        const Range h = span("hidden", a->hidden, tok, a->hidden_stride, dm, es, false);
        const Range o = span("out", a->out, tok, a->out_stride, dm, es, true);
        if (overlap(h, o)) return fail(R2L_ERR_ALIAS, "out overlaps hidden");
    }
    if (!sp.runs) return R2L_OK;
    if (!a->gemm) return fail(R2L_ERR_INVALID_ARG, "gemm (the GEMM context) is NULL");
    if (!a->workspace || a->workspace_bytes < sp.ws_bytes)
        return fail(R2L_ERR_WORKSPACE, "the sidecar needs %zu workspace bytes, got %zu", sp.ws_bytes,
                    a->workspace ? a->workspace_bytes : (size_t)0);
    if (!aligned(a->workspace, 256)) return fail(R2L_ERR_MISALIGNED, "workspace is not 256-byte aligned");
    const int64_t R = a->dt_rank, N = r2l::kN;
    std::vector<Range> rs = {
        span("hidden", a->hidden, tok, a->hidden_stride, dm, es, false),
        span("W_in", a->W_in, 2 * di, dm, dm, es, false),
        span("conv_w", a->conv_w, di, a->d_conv, a->d_conv, 4, false),
        span("conv_b", a->conv_b, 1, di, di, 4, false),
        span("W_x", a->W_x, R + 2 * N, di, di, es, false),
        span("W_dt", a->W_dt, di, R, R, es, false),
        span("dt_bias", a->dt_bias, 1, di, di, 4, false),
        span("A", a->A, di, N, N, 4, false),
        span("Dskip", a->Dskip, 1, di, di, 4, false),
        span("W_out", a->W_out, dm, di, di, es, false),
        span("cu_seqlens", a->cu_seqlens, 1, a->batch + 1, a->batch + 1, 4, false),
        span("out", a->out, tok, a->out_stride, dm, es, true),
        span("workspace", a->workspace, 1, (int64_t)sp.ws_bytes, (int64_t)sp.ws_bytes, 1, true),
    };
    for (size_t i = 0; i < rs.size(); ++i)
        for (size_t j = i + 1; j < rs.size(); ++j) {
            if (!(rs[i].is_output || rs[j].is_output) || !overlap(rs[i], rs[j])) continue;
            const bool out_hidden = (!strcmp(rs[i].name, "hidden") && !strcmp(rs[j].name, "out"));
            if (out_hidden && a->out == a->hidden && a->out_stride == a->hidden_stride) continue;
            return fail(R2L_ERR_ALIAS, "%s overlaps %s", rs[j].is_output ? rs[j].name : rs[i].name,
                        rs[j].is_output ? rs[i].name : rs[j].name);
        }
    // the scan on the workspace, as r2l_scan would check it
    const r2l_scan_args v = r2l::sidecar_scan_view(a, sp);
    return check_buffers(Op::Scan, &v, sp.pl);
}

r2l_status prepare_sidecar(const r2l_sidecar_args *a, r2l::SidecarPlan *sp) {
    if (!a) return fail(R2L_ERR_INVALID_ARG, "args is NULL");
    *sp = r2l::make_sidecar_plan(a);
    const r2l_scan_args v = r2l::sidecar_scan_view(a, *sp);
    r2l_status st = check_shape(&v);
    if (st != R2L_OK) return st;
    if (a->d_model > 65535 * 16) return fail(R2L_ERR_UNSUPPORTED, "d_model above 1048560");
    st = check_sidecar(a, *sp);
    if (st != R2L_OK) return st;
    const int64_t maxlen = ragged(&v) ? v.max_seqlen : v.seqlen;
    const int64_t conv_blocks = a->batch * ((maxlen + r2l::kConvTokens - 1) / r2l::kConvTokens + 1) *
                                ((a->d_inner + r2l::kWG - 1) / r2l::kWG);
    if (a->batch * sp->pl.nchunks * sp->pl.tiles > INT32_MAX - 8 || conv_blocks > INT32_MAX - 8)
        return fail(R2L_ERR_UNSUPPORTED, "grid too large");
    return R2L_OK;
}

// The GEMM context of a call that runs: live, and made for the current device.
r2l_status check_gemm_context(const r2l_sidecar_args *a, const r2l::SidecarPlan &sp) {
    if (!sp.runs || sp.tokens == 0) return R2L_OK;
    const char *err = r2l::gemm_context_check(a->gemm);
    if (err) return fail(R2L_ERR_INVALID_ARG, "gemm: %s", err);
    return R2L_OK;
}

r2l_status run_sidecar(const r2l_sidecar_args *a, hipStream_t stream) {
    r2l::SidecarPlan sp;
    r2l_status st = prepare_sidecar(a, &sp);
    if (st != R2L_OK) return st;
    st = check_gemm_context(a, sp);
    if (st != R2L_OK) return st;
    const r2l_scan_args v = r2l::sidecar_scan_view(a, sp);
    st = check_seqlens_on_device(&v);
    if (st != R2L_OK) return st;
    Launch ls[r2l::kMaxSidecarLaunches];
    const int n = r2l::build_sidecar_launches(a, sp, ls);
    return execute(ls, n, stream);
}

// Host offsets handed to an access replay: they must describe the call.
r2l_status check_host_offsets(const r2l_scan_args *a, const int32_t *cu) {
    if (!ragged(a) || a->batch == 0) return R2L_OK;
    if (!cu) return fail(R2L_ERR_INVALID_ARG, "cu_seqlens_host is NULL");
    if (cu[0] != 0 || cu[a->batch] != a->total_tokens)
        return fail(R2L_ERR_INVALID_ARG, "cu_seqlens_host does not span total_tokens");
    for (int64_t b = 0; b < a->batch; ++b) {
        const int64_t L = static_cast<int64_t>(cu[b + 1]) - cu[b];
        if (L < 0 || L > a->max_seqlen)
            return fail(R2L_ERR_INVALID_ARG, "cu_seqlens_host: bad length at %lld", (long long)b);
    }
    return R2L_OK;
}

// ---- backward -------------------------------------------------------------------
r2l_status check_backward(const r2l_scan_args *a, const r2l_grad_args *g, const r2l::BwdPlan &pl) {
    if (!g) return fail(R2L_ERR_INVALID_ARG, "grad is NULL");
    const int64_t tok = tokens_of(a);
    const int64_t D = a->dim, N = r2l::kN, es = elem_size(a->dtype);
    if (ragged(a) && a->batch > 0 && !a->cu_seqlens)
        return fail(R2L_ERR_INVALID_ARG, "cu_seqlens is NULL");
    if (a->batch > 0 && !a->A) return fail(R2L_ERR_INVALID_ARG, "A is NULL");
    if (tok > 0) {
        const struct { const void *p; const char *n; } req[] = {
            {a->x, "x"}, {a->dt, "dt"}, {a->Bm, "Bm"}, {a->Cm, "Cm"}, {g->dout, "dout"}};
        for (const auto &r : req)
            if (!r.p) return fail(R2L_ERR_INVALID_ARG, "%s is NULL", r.n);
        if (a->x_stride < D || a->dt_stride < D || g->dout_stride < D)
            return fail(R2L_ERR_INVALID_ARG, "x, dt or dout stride < dim");
        if (a->Bm_stride < N || a->Cm_stride < N)
            return fail(R2L_ERR_INVALID_ARG, "Bm or Cm stride < dstate");
        if ((g->dx && g->dx_stride < D) || (g->ddt && g->ddt_stride < D))
            return fail(R2L_ERR_INVALID_ARG, "dx or ddt stride < dim");
        if (a->res && a->res_stride < D) return fail(R2L_ERR_INVALID_ARG, "res_stride < dim");
        if (a->x_batch_stride < 0 || a->dt_batch_stride < 0 || a->Bm_batch_stride < 0 ||
            a->Cm_batch_stride < 0 || g->dout_batch_stride < 0 || g->dx_batch_stride < 0 ||
            g->ddt_batch_stride < 0)
            return fail(R2L_ERR_INVALID_ARG, "negative batch stride");
        const int64_t L = max_len_of(a);
        const struct { int64_t st, cols; } rows[] = {
            {a->x_stride, D}, {a->dt_stride, D}, {g->dout_stride, D}, {g->dx ? g->dx_stride : 0, D},
            {g->ddt ? g->ddt_stride : 0, D}, {a->Bm_stride, N}, {a->Cm_stride, N}};
        for (const auto &r : rows)
            if (L > 0 && r.st > 0 && ((L - 1) * r.st + r.cols) * es > (int64_t)UINT32_MAX)
                return fail(R2L_ERR_UNSUPPORTED, "one sequence spans more than 4 GiB of a tensor");
        if (!ragged(a) && a->batch > 1) {
            if (g->dx && eff_bstride(a, g->dx_batch_stride, g->dx_stride) < a->seqlen * g->dx_stride)
                return fail(R2L_ERR_ALIAS, "dx: sequences overlap");
            if (g->ddt && eff_bstride(a, g->ddt_batch_stride, g->ddt_stride) < a->seqlen * g->ddt_stride)
                return fail(R2L_ERR_ALIAS, "ddt: sequences overlap");
        }
    }
    // (with no token there is nothing to tell an empty residual from none: ds is 0)
    if (g->ds && !a->res && tok > 0)
        return fail(R2L_ERR_INVALID_ARG, "ds needs a residual (out = y has no gate)");
    if (pl.ws_bytes > 0 && (!g->workspace || g->workspace_bytes < pl.ws_bytes))
        return fail(R2L_ERR_WORKSPACE, "backward needs %zu workspace bytes, got %zu", pl.ws_bytes,
                    g->workspace ? g->workspace_bytes : (size_t)0);
    if (a->batch * pl.tiles > INT32_MAX - 8 || a->batch * pl.nchunks * pl.fwd_tiles > INT32_MAX - 8)
        return fail(R2L_ERR_UNSUPPORTED, "grid too large");

    const struct { const void *p; uintptr_t al; const char *n; } al[] = {
        {a->x, (uintptr_t)es, "x"},       {a->dt, (uintptr_t)es, "dt"},     {a->Bm, (uintptr_t)es, "Bm"},
        {a->Cm, (uintptr_t)es, "Cm"},     {g->dout, (uintptr_t)es, "dout"}, {g->dx, (uintptr_t)es, "dx"},
        {g->ddt, (uintptr_t)es, "ddt"},   {a->A, 16, "A"},                  {a->Dskip, 4, "Dskip"},
        {a->h_in, 16, "h_in"},            {g->dh_out, 16, "dh_out"},        {g->dh_in, 16, "dh_in"},
        {g->dBm, 4, "dBm"},               {g->dCm, 4, "dCm"},               {g->dA, 4, "dA"},
        {g->dDskip, 4, "dDskip"},         {g->ds, 4, "ds"},                 {a->cu_seqlens, 4, "cu_seqlens"},
        {g->workspace, 256, "workspace"}};
    for (const auto &e : al)
        if (e.p && !aligned(e.p, e.al))
            return fail(R2L_ERR_MISALIGNED, "%s is not %u-byte aligned", e.n, (unsigned)e.al);

    // no output may overlap an input or another output
    const int64_t B = a->batch;
    std::vector<Range> rs = {
        token_span("x", a, a->x, a->x_stride, a->x_batch_stride, D, es, false),
        token_span("dt", a, a->dt, a->dt_stride, a->dt_batch_stride, D, es, false),
        token_span("Bm", a, a->Bm, a->Bm_stride, a->Bm_batch_stride, N, es, false),
        token_span("Cm", a, a->Cm, a->Cm_stride, a->Cm_batch_stride, N, es, false),
        token_span("res", a, a->res, a->res_stride, a->res_batch_stride, D, es, false),
        token_span("dout", a, g->dout, g->dout_stride, g->dout_batch_stride, D, es, false),
        span("A", a->A, D, N, N, 4, false),
        span("Dskip", a->Dskip, 1, D, D, 4, false),
        span("h_in", a->h_in, B, D * N, D * N, 4, false),
        span("dh_out", g->dh_out, B, D * N, D * N, 4, false),
        span("cu_seqlens", a->cu_seqlens, 1, B + 1, B + 1, 4, false),
        token_span("dx", a, g->dx, g->dx_stride, g->dx_batch_stride, D, es, true),
        token_span("ddt", a, g->ddt, g->ddt_stride, g->ddt_batch_stride, D, es, true),
        span("dBm", g->dBm, tok, N, N, 4, true),
        span("dCm", g->dCm, tok, N, N, 4, true),
        span("dA", g->dA, D, N, N, 4, true),
        span("dDskip", g->dDskip, 1, D, D, 4, true),
        span("dh_in", g->dh_in, B, D * N, D * N, 4, true),
        span("ds", g->ds, 1, 1, 1, 4, true),
        span("workspace", pl.ws_bytes ? g->workspace : nullptr, 1, (int64_t)pl.ws_bytes,
             (int64_t)pl.ws_bytes, 1, true)};
    for (size_t i = 0; i < rs.size(); ++i)
        for (size_t j = i + 1; j < rs.size(); ++j)
            if ((rs[i].is_output || rs[j].is_output) && overlap(rs[i], rs[j]))
                return fail(R2L_ERR_ALIAS, "%s overlaps %s", rs[i].is_output ? rs[i].name : rs[j].name,
                            rs[i].is_output ? rs[j].name : rs[i].name);
    return R2L_OK;
}

// The checkpoints a backward reads: sized and aligned, overlapping no output of
// the forward's arguments nor any gradient output.
r2l_status check_saved(const r2l_scan_args *fwd, const r2l_grad_args *grad, const r2l::BwdPlan &pl,
                       const float *saved, size_t saved_bytes) {
    r2l_status st = check_ckpt(fwd, saved, saved_bytes, false, grad->workspace, pl.ws_bytes);
    if (st != R2L_OK) return st;
    const size_t need = r2l::checkpoint_bytes(fwd);
    if (need == 0) return R2L_OK;
    const int64_t T = tokens_of(fwd), D = fwd->dim, N = r2l::kN, es = elem_size(fwd->dtype);
    const Range c{"ckpt", reinterpret_cast<uintptr_t>(saved), reinterpret_cast<uintptr_t>(saved) + need,
                  false};
    const Range outs[] = {
        token_span("dx", fwd, grad->dx, grad->dx_stride, grad->dx_batch_stride, D, es, true),
        token_span("ddt", fwd, grad->ddt, grad->ddt_stride, grad->ddt_batch_stride, D, es, true),
        span("dBm", grad->dBm, T, N, N, 4, true), span("dCm", grad->dCm, T, N, N, 4, true),
        span("dA", grad->dA, D, N, N, 4, true), span("dDskip", grad->dDskip, 1, D, D, 4, true),
        span("dh_in", grad->dh_in, fwd->batch, D * N, D * N, 4, true),
        span("ds", grad->ds, 1, 1, 1, 4, true)};
    for (const Range &o : outs)
        if (overlap(c, o)) return fail(R2L_ERR_ALIAS, "%s overlaps ckpt", o.name);
    return R2L_OK;
}

// use_saved: the checkpoints come from r2l_scan_save (saved, saved_bytes)
r2l_status run_backward(bool reverse, const r2l_scan_args *fwd, const r2l_grad_args *grad,
                        hipStream_t stream, bool use_saved = false, const float *saved = nullptr,
                        size_t saved_bytes = 0) {
    r2l_status st = check_shape(fwd);
    if (st != R2L_OK) return st;
    if (!grad) return fail(R2L_ERR_INVALID_ARG, "grad is NULL");
    const r2l::BwdPlan pl = r2l::make_bwd_plan(fwd, grad, use_saved);
    st = check_backward(fwd, grad, pl);
    if (st != R2L_OK) return st;
    if (use_saved) {
        st = check_saved(fwd, grad, pl, saved, saved_bytes);
        if (st != R2L_OK) return st;
    }
    st = check_seqlens_on_device(fwd);
    if (st != R2L_OK) return st;
    Launch ls[r2l::kMaxBwdLaunches];
    const int n = r2l::build_bwd_launches(reverse, fwd, grad, pl, ls, saved);
    return execute(ls, n, stream);
}

}  // namespace

extern "C" {

r2l_status r2l_scan_backward(const r2l_scan_args *fwd, const r2l_grad_args *grad, void *stream) {
    return run_backward(true, fwd, grad, static_cast<hipStream_t>(stream));
}

r2l_status prefix_scan_backward(const r2l_scan_args *fwd, const r2l_grad_args *grad, void *stream) {
    return run_backward(false, fwd, grad, static_cast<hipStream_t>(stream));
}

r2l_status r2l_checkpoint_size(const r2l_scan_args *a, size_t *bytes) {
    if (!bytes) return fail(R2L_ERR_INVALID_ARG, "bytes is NULL");
    r2l_status st = check_shape(a);
    if (st != R2L_OK) return st;
    *bytes = r2l::checkpoint_bytes(a);
    return ok();
}

r2l_status r2l_scan_save(const r2l_scan_args *a, float *ckpt, size_t ckpt_bytes, void *stream) {
    return run_save(Op::Scan, a, ckpt, ckpt_bytes, static_cast<hipStream_t>(stream));
}

r2l_status r2l_scan_backward_saved(const r2l_scan_args *fwd, const r2l_grad_args *grad,
                                   const float *ckpt, size_t ckpt_bytes, void *stream) {
    return run_backward(true, fwd, grad, static_cast<hipStream_t>(stream), true, ckpt, ckpt_bytes);
}

r2l_status prefix_scan_save(const r2l_scan_args *a, float *ckpt, size_t ckpt_bytes, void *stream) {
    return run_save(Op::Prefix, a, ckpt, ckpt_bytes, static_cast<hipStream_t>(stream));
}

r2l_status prefix_scan_backward_saved(const r2l_scan_args *fwd, const r2l_grad_args *grad,
                                      const float *ckpt, size_t ckpt_bytes, void *stream) {
    return run_backward(false, fwd, grad, static_cast<hipStream_t>(stream), true, ckpt, ckpt_bytes);
}

r2l_status r2l_check_access_backward(int32_t reverse, const r2l_scan_args *fwd,
                                     const r2l_grad_args *grad, const int32_t *cu_seqlens_host,
                                     r2l_access_report *report) {
    if (!report) return fail(R2L_ERR_INVALID_ARG, "report is NULL");
    report->launches = report->accesses = report->vector_staging = 0;
    report->message[0] = '\0';
    r2l_status st = check_shape(fwd);
    if (st != R2L_OK) return st;
    if (!grad) return fail(R2L_ERR_INVALID_ARG, "grad is NULL");
    const r2l::BwdPlan pl = r2l::make_bwd_plan(fwd, grad);
    st = check_backward(fwd, grad, pl);
    if (st != R2L_OK) return st;
    if (ragged(fwd) && fwd->batch > 0) {
        if (!cu_seqlens_host) return fail(R2L_ERR_INVALID_ARG, "cu_seqlens_host is NULL");
        if (cu_seqlens_host[0] != 0 || cu_seqlens_host[fwd->batch] != fwd->total_tokens)
            return fail(R2L_ERR_INVALID_ARG, "cu_seqlens_host does not span total_tokens");
    }
    st = r2l::check_backward_accesses(reverse != 0, fwd, grad, pl, cu_seqlens_host, report);
    if (st != R2L_OK && report->message[0]) fail(st, "%s", report->message);
    return st == R2L_OK ? ok() : st;
}

r2l_status r2l_backward_workspace_size(const r2l_scan_args *fwd, const r2l_grad_args *grad,
                                       size_t *bytes) {
    if (!bytes) return fail(R2L_ERR_INVALID_ARG, "bytes is NULL");
    r2l_status st = check_shape(fwd);
    if (st != R2L_OK) return st;
    if (!grad) return fail(R2L_ERR_INVALID_ARG, "grad is NULL");
    *bytes = r2l::make_bwd_plan(fwd, grad).ws_bytes;
    return ok();
}


r2l_status bidir_scan(const r2l_scan_args *a, const r2l_dir_args *rev, void *stream) {
    return run_bidir(a, rev, static_cast<hipStream_t>(stream));
}

r2l_status r2l_check_access_bidir(const r2l_scan_args *a, const r2l_dir_args *rev,
                                  const int32_t *cu_seqlens_host, r2l_access_report *report) {
    if (!report) return fail(R2L_ERR_INVALID_ARG, "report is NULL");
    report->launches = report->accesses = report->vector_staging = 0;
    report->message[0] = '\0';
    r2l::BidirPlan bp;
    r2l_status st = prepare_bidir(a, rev, &bp);
    if (st != R2L_OK) return st;
    st = check_host_offsets(a, cu_seqlens_host);
    if (st != R2L_OK) return st;
    st = r2l::check_bidir_accesses(a, rev, bp, cu_seqlens_host, report);
    if (st != R2L_OK) return fail(st, "%s", report->message);
    return ok();
}

r2l_status r2l_sidecar_forward(const r2l_sidecar_args *a, void *stream) {
    return run_sidecar(a, static_cast<hipStream_t>(stream));
}

r2l_status r2l_gemm_context_create(r2l_gemm_context *ctx) {
    if (!ctx) return fail(R2L_ERR_INVALID_ARG, "ctx is NULL");
    *ctx = nullptr;
    const char *err = r2l::gemm_context_create(ctx);
    if (err) return fail(R2L_ERR_HIP, "r2l_gemm_context_create: %s", err);
    return ok();
}

r2l_status r2l_gemm_context_destroy(r2l_gemm_context ctx) {
    if (!ctx) return fail(R2L_ERR_INVALID_ARG, "ctx is NULL");
    const char *err = r2l::gemm_context_destroy(ctx);
    if (err) return fail(strstr(err, "live") ? R2L_ERR_INVALID_ARG : R2L_ERR_HIP,
                         "r2l_gemm_context_destroy: %s", err);
    return ok();
}

r2l_status r2l_sidecar_tune(const r2l_sidecar_args *a, void *stream) {
    r2l::SidecarPlan sp;
    r2l_status st = prepare_sidecar(a, &sp);
    if (st != R2L_OK) return st;
    st = check_gemm_context(a, sp);
    if (st != R2L_OK) return st;
    Launch ls[r2l::kMaxSidecarLaunches];
    const int n = r2l::build_sidecar_launches(a, sp, ls);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t es = elem_size(a->dtype);
    for (int i = 0; i < n; ++i) {
        if (ls[i].kind != Launch::Gemm) continue;
        const r2l::GemmParams &g = ls[i].gemm;
        void *scratch = nullptr;
        if (g.Y == a->out) {
            // the out-projection: time it into the x|z rows (dead by then), never into out
            const size_t need = static_cast<size_t>(((g.M - 1) * g.ldy + g.N) * es);
            if (need <= sp.off_u - sp.off_xz)
                scratch = static_cast<char *>(a->workspace) + sp.off_xz;
            else if (a->out == a->hidden)
                continue;   // in place and no room: keep the library's first choice
        }
        const char *err = r2l::tune_gemm(a->gemm, a->dtype, g, scratch, s);
        if (err) return fail(R2L_ERR_HIP, "sidecar projection tuning: %s", err);
    }
    return ok();
}

r2l_status r2l_sidecar_workspace_size(const r2l_sidecar_args *a, size_t *bytes) {
    if (!bytes) return fail(R2L_ERR_INVALID_ARG, "bytes is NULL");
    if (!a) return fail(R2L_ERR_INVALID_ARG, "args is NULL");
    const r2l::SidecarPlan sp = r2l::make_sidecar_plan(a);
    const r2l_scan_args v = r2l::sidecar_scan_view(a, sp);
    r2l_status st = check_shape(&v);
    if (st != R2L_OK) return st;
    *bytes = sp.ws_bytes;
    return ok();
}

r2l_status r2l_check_access_sidecar(const r2l_sidecar_args *a, const int32_t *cu_seqlens_host,
                                    r2l_access_report *report) {
    if (!report) return fail(R2L_ERR_INVALID_ARG, "report is NULL");
    report->launches = report->accesses = report->vector_staging = 0;
    report->message[0] = '\0';
    r2l::SidecarPlan sp;
    r2l_status st = prepare_sidecar(a, &sp);
    if (st != R2L_OK) return st;
    const r2l_scan_args v = r2l::sidecar_scan_view(a, sp);
    st = check_host_offsets(&v, cu_seqlens_host);
    if (st != R2L_OK) return st;
    st = r2l::check_sidecar_accesses(a, sp, cu_seqlens_host, report);
    if (st != R2L_OK) return fail(st, "%s", report->message);
    return ok();
}

r2l_status r2l_scan(const r2l_scan_args *a, void *stream) {
    return run(Op::Scan, a, static_cast<hipStream_t>(stream));
}

static_assert(r2l::kNoallocScratchBytes == R2L_NOALLOC_SCRATCH_BYTES,
              "the scratch size in the header");

r2l_status r2l_scan_noalloc(const r2l_scan_args *a, void *stream) {
    r2l_status st = check_shape(a);
    if (st != R2L_OK) return st;
    r2l_scan_args v = *a;
    v.workspace = nullptr;
    v.workspace_bytes = 0;
    const Plan pl = r2l::make_plan(Op::Scan, &v);
    if (pl.ws_bytes > r2l::kNoallocScratchBytes)
        return fail(R2L_ERR_WORKSPACE,
                    "the plan needs %zu bytes of scratch, more than the %zu that "
                    "r2l_scan_noalloc holds (use r2l_scan with a workspace)",
                    pl.ws_bytes, r2l::kNoallocScratchBytes);
    if (pl.ws_bytes > 0) {
        void *p = nullptr;
        st = hip_status(r2l::noalloc_scratch(&p), "scratch address lookup");
        if (st != R2L_OK) return st;
        v.workspace = p;
        v.workspace_bytes = r2l::kNoallocScratchBytes;
    }
    return run(Op::Scan, &v, static_cast<hipStream_t>(stream), false);
}

r2l_status prefix_scan_state(const r2l_scan_args *a, void *stream) {
    return run(Op::Prefix, a, static_cast<hipStream_t>(stream));
}

r2l_status block_commit_state(const r2l_scan_args *a, void *stream) {
    return run(Op::Commit, a, static_cast<hipStream_t>(stream));
}

r2l_status r2l_workspace_size(int32_t op, const r2l_scan_args *a, size_t *bytes) {
    if (!bytes) return fail(R2L_ERR_INVALID_ARG, "bytes is NULL");
    if (op != R2L_OP_SCAN && op != R2L_OP_PREFIX && op != R2L_OP_COMMIT && op != R2L_OP_BIDIR &&
        op != R2L_OP_SAVE && op != R2L_OP_PREFIX_SAVE)
        return fail(R2L_ERR_INVALID_ARG, "unknown op %d", op);
    r2l_status st = check_shape(a);
    if (st != R2L_OK) return st;
    if (op == R2L_OP_BIDIR) {
        *bytes = r2l::make_bidir_plan(a).ws_bytes;
        return ok();
    }
    if (op == R2L_OP_SAVE || op == R2L_OP_PREFIX_SAVE) {
        r2l_scan_args v = *a;
        v.state_split = 1;
        *bytes = r2l::make_plan(op == R2L_OP_SAVE ? Op::Scan : Op::Prefix, &v, true).ws_bytes;
        return ok();
    }
    const Op o = op == R2L_OP_SCAN ? Op::Scan : (op == R2L_OP_PREFIX ? Op::Prefix : Op::Commit);
    *bytes = r2l::make_plan(o, a).ws_bytes;
    return ok();
}

r2l_status r2l_check_access(int32_t op, const r2l_scan_args *a, const int32_t *cu_seqlens_host,
                            r2l_access_report *report) {
    if (!report) return fail(R2L_ERR_INVALID_ARG, "report is NULL");
    report->launches = report->accesses = report->vector_staging = 0;
    report->message[0] = '\0';
    if (op != R2L_OP_SCAN && op != R2L_OP_PREFIX && op != R2L_OP_COMMIT)
        return fail(R2L_ERR_INVALID_ARG, "unknown op %d", op);
    r2l_status st = check_shape(a);
    if (st != R2L_OK) return st;
    const Op o = op == R2L_OP_SCAN ? Op::Scan : (op == R2L_OP_PREFIX ? Op::Prefix : Op::Commit);
    const Plan pl = r2l::make_plan(o, a);
    st = check_buffers(o, a, pl);
    if (st != R2L_OK) return st;
    if (ragged(a) && a->batch > 0) {
        if (!cu_seqlens_host) return fail(R2L_ERR_INVALID_ARG, "cu_seqlens_host is NULL");
        if (cu_seqlens_host[0] != 0 || cu_seqlens_host[a->batch] != a->total_tokens)
            return fail(R2L_ERR_INVALID_ARG, "cu_seqlens_host does not span total_tokens");
        for (int64_t b = 0; b < a->batch; ++b) {
            const int64_t L = static_cast<int64_t>(cu_seqlens_host[b + 1]) - cu_seqlens_host[b];
            if (L < 0 || L > a->max_seqlen)
                return fail(R2L_ERR_INVALID_ARG, "cu_seqlens_host: bad length at %lld", (long long)b);
        }
    }
    st = r2l::check_accesses(o, a, pl, cu_seqlens_host, report);
    if (st != R2L_OK) return fail(st, "%s", report->message);
    return ok();
}

r2l_status r2l_check_access_save(int32_t reverse, const r2l_scan_args *a, const float *ckpt,
                                 size_t ckpt_bytes, const int32_t *cu_seqlens_host,
                                 r2l_access_report *report) {
    if (!report) return fail(R2L_ERR_INVALID_ARG, "report is NULL");
    report->launches = report->accesses = report->vector_staging = 0;
    report->message[0] = '\0';
    const Op op = reverse ? Op::Scan : Op::Prefix;
    r2l_scan_args v;
    Plan pl;
    r2l_status st = prepare_save(op, a, &v, &pl);
    if (st != R2L_OK) return st;
    st = check_ckpt(&v, ckpt, ckpt_bytes, true, pl.chunked ? v.workspace : nullptr,
                    pl.chunked ? pl.ws_bytes : 0);
    if (st != R2L_OK) return st;
    st = check_host_offsets(&v, cu_seqlens_host);
    if (st != R2L_OK) return st;
    st = r2l::check_accesses(op, &v, pl, cu_seqlens_host, report, const_cast<float *>(ckpt),
                             ckpt_bytes);
    if (st != R2L_OK) return fail(st, "%s", report->message);
    return ok();
}

r2l_status r2l_check_access_backward_saved(int32_t reverse, const r2l_scan_args *fwd,
                                           const r2l_grad_args *grad,
                                           const float *ckpt, size_t ckpt_bytes,
                                           const int32_t *cu_seqlens_host,
                                           r2l_access_report *report) {
    if (!report) return fail(R2L_ERR_INVALID_ARG, "report is NULL");
    report->launches = report->accesses = report->vector_staging = 0;
    report->message[0] = '\0';
    r2l_status st = check_shape(fwd);
    if (st != R2L_OK) return st;
    if (!grad) return fail(R2L_ERR_INVALID_ARG, "grad is NULL");
    const r2l::BwdPlan pl = r2l::make_bwd_plan(fwd, grad, true);
    st = check_backward(fwd, grad, pl);
    if (st != R2L_OK) return st;
    st = check_saved(fwd, grad, pl, ckpt, ckpt_bytes);
    if (st != R2L_OK) return st;
    st = check_host_offsets(fwd, cu_seqlens_host);
    if (st != R2L_OK) return st;
    st = r2l::check_backward_accesses(reverse != 0, fwd, grad, pl, cu_seqlens_host, report, ckpt,
                                      ckpt_bytes);
    if (st != R2L_OK && report->message[0]) fail(st, "%s", report->message);
    return st == R2L_OK ? ok() : st;
}

r2l_status r2l_describe_plan(int32_t op, const r2l_scan_args *a, r2l_plan_info *info) {
    if (!info) return fail(R2L_ERR_INVALID_ARG, "info is NULL");
    if (op != R2L_OP_SCAN && op != R2L_OP_PREFIX && op != R2L_OP_COMMIT && op != R2L_OP_BIDIR)
        return fail(R2L_ERR_INVALID_ARG, "unknown op %d", op);
    r2l_status st = check_shape(a);
    if (st != R2L_OK) return st;
    if (op == R2L_OP_BIDIR) {
        const r2l::BidirPlan bp = r2l::make_bidir_plan(a);
        info->lanes_per_channel = 1;
        info->chunked = bp.pl.chunked ? 1 : 0;
        info->chunk_tokens = bp.pl.chunk_len;
        info->chunks = bp.pl.nchunks;
        info->workspace_bytes = static_cast<int64_t>(bp.ws_bytes);
        Launch ls[r2l::kMaxBidirLaunches];
        info->launches = r2l::build_bidir_launches(a, nullptr, bp, ls);
        return ok();
    }
    const Op o = op == R2L_OP_SCAN ? Op::Scan : (op == R2L_OP_PREFIX ? Op::Prefix : Op::Commit);
    const Plan pl = r2l::make_plan(o, a);
    info->lanes_per_channel = pl.G;
    info->chunked = pl.chunked ? 1 : 0;
    info->chunk_tokens = pl.chunk_len;
    info->chunks = pl.nchunks;
    info->workspace_bytes = static_cast<int64_t>(pl.ws_bytes);
    Launch ls[3];
    info->launches = r2l::build_launches(o, a, pl, ls);
    return ok();
}

const char *r2l_status_string(r2l_status s) {
    switch (s) {
        case R2L_OK: return "ok";
        case R2L_ERR_INVALID_ARG: return "invalid argument";
        case R2L_ERR_UNSUPPORTED: return "unsupported dtype or size";
        case R2L_ERR_ALIAS: return "buffers overlap";
        case R2L_ERR_MISALIGNED: return "misaligned pointer";
        case R2L_ERR_WORKSPACE: return "workspace missing or too small";
        case R2L_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char *r2l_last_error(void) { return g_last_error; }

int32_t r2l_abi_version(void) { return R2L_ABI_VERSION; }

}  // extern "C"
