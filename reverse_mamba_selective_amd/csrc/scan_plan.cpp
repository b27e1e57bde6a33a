// scan_plan.cpp -- planning (lanes per channel, chunking, workspace layout)
// and the launch list of one entry-point call.
#include "scan_plan.h"

#include <algorithm>

#include "scan_geometry.h"

namespace r2l {
namespace {

// Measured on MI355X (bf16, N = 16): one lane per channel runs the token loop
// at ~90% of the VALU issue rate once a few waves share each SIMD, while
// splitting a channel's states over 2 or 4 lanes costs more instructions per
// token (softplus repeated, a cross-lane sum) than its extra waves win back.
// So the planner keeps one lane per channel and, when a shape has too few
// channels to fill the machine, cuts sequences into chunks instead:
//  * state-only scans chunk for free (the carry is one fma per chunk);
//  * readout scans pay a second, state-only pass over the chunks after the
//    first (about 1.65x the vector work of one pass at 9 chunks) and still
//    come out ahead below ~4096 waves. Each of their two passes runs one chunk
//    fewer than the plan has (the chunk pass skips the last chunk when no
//    final state is wanted, the readout pass the first), so they take one
//    chunk more than the machine needs: 8 x 4096 x 4096 runs in 0.78 ms with
//    9 chunks, 0.84 ms with 8, 1.01 ms with 4 lanes per channel and 1.64 ms
//    with one wave per channel tile and no chunking.
constexpr int64_t kTargetLanes = 4096 * 64;
// Longest chunk a state-only plan keeps, so that ragged prefixes of very
// different lengths balance across the machine.
constexpr int64_t kMaxStateChunk = 1024;
// Shortest chunk worth a carry pass.
constexpr int64_t kMinChunk = 256;

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

SegParams base_params(const r2l_scan_args *a, const Plan &pl) {
    SegParams p{};
    p.seqlen = is_ragged(a) ? 0 : a->seqlen;
    p.cu_seqlens = a->cu_seqlens;
    p.D = a->dim;
    p.chunk_len = static_cast<int32_t>(pl.chunk_len);
    p.nchunks = static_cast<int32_t>(pl.nchunks);
    p.tiles = static_cast<int32_t>(pl.tiles);
    p.nblocks = a->batch * pl.nchunks * pl.tiles;
    p.x = a->x;   p.xs = a->x_stride;  p.xbs = eff_bstride(a, a->x_batch_stride, a->x_stride);
    p.dt = a->dt; p.dts = a->dt_stride; p.dtbs = eff_bstride(a, a->dt_batch_stride, a->dt_stride);
    p.Bm = a->Bm; p.Bs = a->Bm_stride;  p.Bbs = eff_bstride(a, a->Bm_batch_stride, a->Bm_stride);
    p.Cm = a->Cm; p.Cs = a->Cm_stride;  p.Cbs = eff_bstride(a, a->Cm_batch_stride, a->Cm_stride);
    p.A = a->A;
    p.Dskip = a->Dskip;
    p.softplus = a->delta_softplus;
    p.res = a->res; p.rs = a->res_stride;
    p.rbs = eff_bstride(a, a->res_batch_stride, a->res_stride);
    p.s = a->s;
    p.out = a->out; p.os = a->out_stride;
    p.obs = eff_bstride(a, a->out_batch_stride, a->out_stride);
    return p;
}

// Whether every Bm (and, when staged, Cm) row starts on the alignment the
// staging's vector loads need: base pointer, row stride and batch stride.
bool bc_vector_ok(const r2l_scan_args *a, bool readout) {
    const int64_t es = elem_size(a->dtype);
    const int64_t al = stage_align(readout ? 2 * kN : kN, static_cast<int>(es));
    auto ok = [&](const void *p, int64_t st, int64_t bst) {
        return reinterpret_cast<uintptr_t>(p) % al == 0 && (st * es) % al == 0 &&
               (eff_bstride(a, bst, st) * es) % al == 0;
    };
    return ok(a->Bm, a->Bm_stride, a->Bm_batch_stride) &&
           (!readout || ok(a->Cm, a->Cm_stride, a->Cm_batch_stride));
}

// What the readout writes: y, or the gated residual reading x itself (when
// res is exactly x) or a separate residual tensor.
int out_mode(const r2l_scan_args *a, const SegParams &p) {
    if (!a->res) return kModeY;
    if (a->res == a->x && a->res_stride == a->x_stride && p.rbs == p.xbs) return kModeResX;
    return kModeRes;
}

}  // namespace

Plan make_plan(Op op, const r2l_scan_args *a, bool ckpt) {
    Plan pl;
    const int64_t channels = a->batch * a->dim;
    const int64_t maxlen = max_len_of(a);
    pl.G = a->state_split ? a->state_split : 1;
    const bool readout = runs_readout(op, a);
    int64_t chunk = 0;
    if (!runs_scan(op, a)) {
        // nothing is scanned: no chunks, no workspace
    } else if (a->chunk_tokens > 0) {
        chunk = a->chunk_tokens;
    } else if (a->chunk_tokens == 0 && maxlen > 0) {
        const int64_t lanes = std::max<int64_t>(channels * pl.G, 1);
        const int64_t fill = (kTargetLanes + lanes - 1) / lanes;  // chunks to fill the machine
        const int64_t want = readout ? (fill > 1 ? fill + 1 : 1)
                                     : std::max<int64_t>(fill, (maxlen + kMaxStateChunk - 1) /
                                                                   kMaxStateChunk);
        if (want > 1) chunk = std::max<int64_t>(kMinChunk, (maxlen + want - 1) / want);
        // a readout plan of two chunks runs one chunk per pass: no gain
        if (readout && chunk > 0 && (maxlen + chunk - 1) / chunk < 3) chunk = 0;
    }
    if (ckpt) chunk = (chunk + kCkptTokens - 1) / kCkptTokens * kCkptTokens;
    if (chunk > 0 && chunk < maxlen) {
        pl.chunked = true;
        pl.chunk_len = chunk;
        pl.nchunks = (maxlen + chunk - 1) / chunk;
    } else {
        pl.chunked = false;
        pl.chunk_len = std::max<int64_t>(maxlen, 1);
        pl.nchunks = 1;
    }
    pl.tiles = (a->dim * pl.G + kWG - 1) / kWG;
    if (pl.chunked) {
        const size_t q = static_cast<size_t>(a->batch) * pl.nchunks * a->dim * kN * 4;
        const size_t s = static_cast<size_t>(a->batch) * pl.nchunks * a->dim * 4;
        pl.off_S = align256(q);
        pl.off_H = pl.off_S + align256(s);
        pl.ws_bytes = pl.off_H + (readout ? align256(q) : 0);
    }
    return pl;
}

namespace {

// The residual copied to out when the gate is closed (nothing when out is
// the residual itself).
int copy_launch(const r2l_scan_args *a, Launch *out) {
    const int64_t rbs = eff_bstride(a, a->res_batch_stride, a->res_stride);
    const int64_t obs = eff_bstride(a, a->out_batch_stride, a->out_stride);
    if (a->out == a->res && a->out_stride == a->res_stride && obs == rbs) return 0;
    if (tokens_of(a) == 0) return 0;
    Launch l{};
    l.kind = Launch::Copy;
    l.dtype = a->dtype;
    l.copy.rows = tokens_of(a);
    l.copy.seqlen = is_ragged(a) ? 0 : a->seqlen;
    l.copy.D = a->dim;
    l.copy.src = a->res; l.copy.ss = a->res_stride; l.copy.sbs = rbs;
    l.copy.dst = a->out; l.copy.ds = a->out_stride; l.copy.dbs = obs;
    *out = l;
    return 1;
}

int build_scan_launches(Op op, const r2l_scan_args *a, const Plan &pl, Launch out[3]);

}  // namespace

int build_launches(Op op, const r2l_scan_args *a, const Plan &pl, Launch out[3]) {
    if (a->batch == 0) return 0;
    int n = runs_scan(op, a) ? build_scan_launches(op, a, pl, out) : 0;
    // after the scan, which may read x when out is x
    if (gate_closed(op, a)) n += copy_launch(a, out + n);
    return n;
}

namespace {

int build_scan_launches(Op op, const r2l_scan_args *a, const Plan &pl, Launch out[3]) {
    const bool reverse = (op == Op::Scan);
    const bool readout = runs_readout(op, a);
    const int64_t DN = a->dim * kN;
    // block_commit_state reads the state it updates from h_out
    const float *h_init = (op == Op::Commit) ? a->h_out : a->h_in;

    auto seg = [&](const SegParams &p, int mode) {
        Launch l{};
        l.kind = Launch::Segment;
        l.reverse = reverse;
        l.dtype = a->dtype;
        l.G = pl.G;
        l.mode = mode;
        l.seg = p;
        l.seg.bc_vec = bc_vector_ok(a, mode != kModeState) ? 1 : 0;
        return l;
    };

    if (!pl.chunked) {
        if (tokens_of(a) == 0 && !a->h_out) return 0;
        SegParams p = base_params(a, pl);
        p.hin = h_init; p.hin_b = DN; p.hin_c = 0;
        p.hfin = a->h_out; p.hfin_b = DN; p.hfin_c = 0;
        out[0] = seg(p, readout ? out_mode(a, p) : kModeState);
        return 1;
    }

    char *ws = static_cast<char *>(a->workspace);
    float *Q = reinterpret_cast<float *>(ws);
    float *S = reinterpret_cast<float *>(ws + pl.off_S);
    float *H = readout ? reinterpret_cast<float *>(ws + pl.off_H) : nullptr;

    // 1. every chunk from a zero state: local final state Q and Delta sum S.
    // Readout plans: chunk 0 starts from the call's own initial state, so this
    // pass already writes its outputs, and the readout pass skips it; without
    // h_out nothing reads the last chunk's Q and S, so this pass skips it.
    SegParams p1 = base_params(a, pl);
    p1.hfin = Q; p1.hfin_b = pl.nchunks * DN; p1.hfin_c = DN;
    p1.sdelta = S; p1.sd_b = pl.nchunks * a->dim; p1.sd_c = a->dim;
    if (readout) {
        p1.hin = h_init; p1.hin_b = DN; p1.hin_c = 0;
        p1.split_c0 = 1;
        p1.skip_last = a->h_out ? 0 : 1;
        out[0] = seg(p1, out_mode(a, p1));
    } else {
        p1.hin = nullptr;
        p1.res = nullptr;
        p1.out = nullptr;
        out[0] = seg(p1, kModeState);
    }

    // 2. chain the chunks: the state entering each chunk, and the final state
    Launch c{};
    c.kind = Launch::Carry;
    c.reverse = reverse;
    c.dtype = a->dtype;
    c.carry.batch = a->batch;
    c.carry.seqlen = is_ragged(a) ? 0 : a->seqlen;
    c.carry.cu_seqlens = a->cu_seqlens;
    c.carry.D = a->dim;
    c.carry.chunk_len = static_cast<int32_t>(pl.chunk_len);
    c.carry.nchunks = static_cast<int32_t>(pl.nchunks);
    c.carry.A = a->A;
    c.carry.hin = readout ? nullptr : h_init;
    c.carry.c0_seeded = readout ? 1 : 0;
    c.carry.Q = Q;
    c.carry.S = S;
    c.carry.Hc = H;
    c.carry.hout = a->h_out;
    out[1] = c;
    if (!readout) return 2;

    // 3. readout: rescan every chunk but the first from the state that enters it
    SegParams p3 = base_params(a, pl);
    p3.hin = H; p3.hin_b = pl.nchunks * DN; p3.hin_c = DN;
    p3.hfin = nullptr;
    p3.skip_c0 = 1;
    out[2] = seg(p3, out_mode(a, p3));
    return 3;
}

}  // namespace

// ---- checkpoints ------------------------------------------------------------------
size_t checkpoint_bytes(const r2l_scan_args *a) {
    const int64_t T = tokens_of(a);
    if (T <= 0) return 0;
    return static_cast<size_t>(ckpt_rows(T, a->batch)) * static_cast<size_t>(a->dim) * kN * 4;
}

namespace {

// One unchunked state-only scan over every sequence from h_in, one lane per
// channel, storing the checkpoints (the true states).
Launch ckpt_state_launch(bool reverse, const r2l_scan_args *a, int64_t fwd_tiles, float *ck) {
    Plan fp;
    fp.G = 1;
    fp.chunk_len = std::max<int64_t>(max_len_of(a), 1);
    fp.nchunks = 1;
    fp.tiles = fwd_tiles;
    SegParams p = base_params(a, fp);
    p.res = nullptr;
    p.out = nullptr;
    p.ckpt = ck;
    p.bc_vec = bc_vector_ok(a, false) ? 1 : 0;
    p.hin = a->h_in; p.hin_b = a->dim * kN; p.hin_c = 0;
    Launch l{};
    l.kind = Launch::Segment;
    l.reverse = reverse;
    l.dtype = a->dtype;
    l.G = 1;
    l.mode = kModeState | kModeCkpt;
    l.seg = p;
    return l;
}

}  // namespace

int build_save_launches(Op op, const r2l_scan_args *a, const Plan &pl, float *ckpt,
                        Launch out[kMaxSaveLaunches]) {
    int n = build_launches(op, a, pl, out);
    bool stored = false;
    for (int i = 0; i < n; ++i)
        if (out[i].kind == Launch::Segment && (out[i].mode & kModeOutMask) != kModeState) {
            out[i].mode |= kModeCkpt;
            out[i].seg.ckpt = ckpt;
            stored = true;
        }
    if (!stored && tokens_of(a) > 0 && a->batch > 0) {
        // before the residual copy, which may overwrite x (out == x with a
        // separate residual): the checkpoints are the states of the x given
        int at = n;
        while (at > 0 && out[at - 1].kind == Launch::Copy) --at;
        for (int i = n; i > at; --i) out[i] = out[i - 1];
        out[at] = ckpt_state_launch(op == Op::Scan, a, (a->dim + kWG - 1) / kWG, ckpt);
        ++n;
    }
    return n;
}

// ---- bidirectional scan ------------------------------------------------------------
BidirPlan make_bidir_plan(const r2l_scan_args *a) {
    BidirPlan bp;
    r2l_scan_args v = *a;
    v.state_split = 1;
    bp.readout = runs_readout(Op::Prefix, &v);
    bp.pl = make_plan(Op::Prefix, &v);
    if (!bp.readout) {
        bp.ws_bytes = bp.pl.ws_bytes;
        return bp;
    }
    bp.fused = !bp.pl.chunked;
    bp.off_chunk = align256(static_cast<size_t>(tokens_of(a)) * static_cast<size_t>(a->dim) * 4);
    bp.ws_bytes = bp.off_chunk + bp.pl.ws_bytes;
    return bp;
}

r2l_scan_args reverse_view(const r2l_scan_args *a, const r2l_dir_args *rev) {
    r2l_scan_args r = *a;
    if (rev) {
        if (rev->dt) { r.dt = rev->dt; r.dt_stride = rev->dt_stride; r.dt_batch_stride = rev->dt_batch_stride; }
        if (rev->Bm) { r.Bm = rev->Bm; r.Bm_stride = rev->Bm_stride; r.Bm_batch_stride = rev->Bm_batch_stride; }
        if (rev->Cm) { r.Cm = rev->Cm; r.Cm_stride = rev->Cm_stride; r.Cm_batch_stride = rev->Cm_batch_stride; }
        if (rev->A) r.A = rev->A;
        if (rev->Dskip) r.Dskip = rev->Dskip;
    }
    r.res = nullptr; r.res_stride = 0; r.res_batch_stride = 0;
    r.s = 0.0f;
    r.h_in = nullptr;
    r.h_out = nullptr;
    r.state_split = 1;
    return r;
}

int build_bidir_launches(const r2l_scan_args *a, const r2l_dir_args *rev, const BidirPlan &bp,
                         Launch out[kMaxBidirLaunches]) {
    if (a->batch == 0) return 0;
    r2l_scan_args f = *a;
    f.state_split = 1;
    if (!bp.readout) return build_launches(Op::Prefix, &f, bp.pl, out);
    if (tokens_of(a) == 0 && !a->h_out) return 0;

    char *ws = static_cast<char *>(a->workspace);
    float *rows = reinterpret_cast<float *>(ws);
    r2l_scan_args r = reverse_view(a, rev);
    r.workspace = ws + bp.off_chunk;
    r.workspace_bytes = bp.pl.ws_bytes;
    f.workspace = ws + bp.off_chunk;
    f.workspace_bytes = bp.pl.ws_bytes;
    const int64_t DN = a->dim * kN;

    if (bp.fused) {
        SegParams pr = base_params(&r, bp.pl);
        pr.out = nullptr;
        pr.yws = rows;
        pr.bc_vec = bc_vector_ok(&r, true) ? 1 : 0;
        SegParams pf = base_params(&f, bp.pl);
        pf.hin = a->h_in; pf.hin_b = DN; pf.hin_c = 0;
        pf.hfin = a->h_out; pf.hfin_b = DN; pf.hfin_c = 0;
        pf.yadd = rows;
        pf.bc_vec = bc_vector_ok(&f, true) ? 1 : 0;
        Launch l{};
        l.kind = Launch::Bidir;
        l.dtype = a->dtype;
        l.G = 1;
        l.mode = kModeAdd | out_mode(&f, pf);
        if (bp.pl.chunk_len <= kBidirLdsTokens) l.mode |= kModeLds;   // the rows stay in LDS
        l.seg = pr;
        l.seg2 = pf;
        out[0] = l;
        return 1;
    }
    // chunked: each direction's own plan, the readout launches retargeted
    int n = build_scan_launches(Op::Scan, &r, bp.pl, out);
    for (int i = 0; i < n; ++i)
        if (out[i].kind == Launch::Segment && out[i].mode != kModeState) {
            out[i].mode = kModeWs;
            out[i].seg.out = nullptr;
            out[i].seg.yws = rows;
        }
    const int m = build_scan_launches(Op::Prefix, &f, bp.pl, out + n);
    for (int i = n; i < n + m; ++i)
        if (out[i].kind == Launch::Segment && out[i].mode != kModeState) {
            out[i].mode |= kModeAdd;
            out[i].seg.yadd = rows;
        }
    return n + m;
}

// ---- sidecar block -----------------------------------------------------------------
SidecarPlan make_sidecar_plan(const r2l_sidecar_args *a) {
    SidecarPlan sp;
    sp.tokens = a->cu_seqlens ? a->total_tokens : a->batch * a->seqlen;
    sp.runs = a->s != 0.0f;
    if (!sp.runs) return sp;
    const size_t T = static_cast<size_t>(sp.tokens), di = static_cast<size_t>(a->d_inner);
    const size_t es = a->dtype == R2L_DTYPE_BF16 ? 2 : 4;
    sp.ldx = ((a->dt_rank + 2 * kN) + 7) / 8 * 8;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align256(bytes);
        return at;
    };
    sp.off_xz = take(T * 2 * di * es);
    sp.off_u = take(T * di * es);
    sp.off_xdbl = take(T * static_cast<size_t>(sp.ldx) * es);
    sp.off_dt = take(T * di * es);
    sp.off_g = take(T * di * es);
    sp.off_chunk = off;
    sp.ws_bytes = off;   // for the view below
    const r2l_scan_args v = sidecar_scan_view(a, sp);
    sp.pl = make_plan(Op::Scan, &v);
    sp.off_chunk = take(sp.pl.ws_bytes);
    sp.off_gemm = take(kGemmWorkspace);
    sp.ws_bytes = off;
    return sp;
}

r2l_scan_args sidecar_scan_view(const r2l_sidecar_args *a, const SidecarPlan &sp) {
    r2l_scan_args v{};
    v.batch = a->batch;
    v.seqlen = a->seqlen;
    v.cu_seqlens = a->cu_seqlens;
    v.total_tokens = a->total_tokens;
    v.max_seqlen = a->max_seqlen;
    v.dim = a->d_inner;
    v.dstate = a->dstate;
    v.dtype = a->dtype;
    const int64_t es = a->dtype == R2L_DTYPE_BF16 ? 2 : 4, di = a->d_inner;
    char *ws = static_cast<char *>(a->workspace);
    auto at = [&](size_t off, int64_t elems) { return ws ? ws + off + elems * es : nullptr; };
    v.x = at(sp.off_u, 0);          v.x_stride = di;
    v.dt = at(sp.off_dt, 0);        v.dt_stride = di;
    v.Bm = at(sp.off_xdbl, a->dt_rank);        v.Bm_stride = sp.ldx;
    v.Cm = at(sp.off_xdbl, a->dt_rank + kN);   v.Cm_stride = sp.ldx;
    v.A = a->A;
    v.Dskip = a->Dskip;
    v.delta_softplus = 1;
    v.res = at(sp.off_xz, di);      v.res_stride = 2 * di;    // z
    v.s = 1.0f;
    v.out = at(sp.off_g, 0);        v.out_stride = di;
    v.workspace = at(sp.off_chunk, 0);
    v.workspace_bytes = sp.pl.ws_bytes;
    return v;
}

int build_sidecar_launches(const r2l_sidecar_args *a, const SidecarPlan &sp,
                           Launch out[kMaxSidecarLaunches]) {
    const int64_t T = sp.tokens, di = a->d_inner, dm = a->d_model;
    if (a->batch == 0 || T == 0) return 0;
    if (!sp.runs) {   // s == 0: out is hidden
        if (a->out == a->hidden && a->out_stride == a->hidden_stride) return 0;
        Launch l{};
        l.kind = Launch::Copy;
        l.dtype = a->dtype;
        l.copy.rows = T;
        l.copy.seqlen = 0;
        l.copy.D = dm;
        l.copy.src = a->hidden; l.copy.ss = a->hidden_stride; l.copy.sbs = 0;
        l.copy.dst = a->out;    l.copy.ds = a->out_stride;    l.copy.dbs = 0;
        out[0] = l;
        return 1;
    }
    char *ws = static_cast<char *>(a->workspace);
    void *xz = ws + sp.off_xz, *u = ws + sp.off_u, *xdbl = ws + sp.off_xdbl;
    void *dtb = ws + sp.off_dt, *g = ws + sp.off_g, *gws = ws + sp.off_gemm;
    int n = 0;
    auto gemm = [&](int64_t N, int64_t K, const void *X, int64_t ldx, const void *W, void *Y,
                    int64_t ldy, const void *C, int64_t ldc, float alpha, float beta) {
        Launch l{};
        l.kind = Launch::Gemm;
        l.dtype = a->dtype;
        l.gemm = GemmParams{a->gemm, T, N, K, X, ldx, W, K, C, ldc, Y, ldy, alpha, beta, gws,
                            kGemmWorkspace};
        out[n++] = l;
    };
    // 1. [x | z] = hidden W_in^T
    gemm(2 * di, dm, a->hidden, a->hidden_stride, a->W_in, xz, 2 * di, nullptr, 0, 1.0f, 0.0f);
    // 2. u = SiLU(conv(x))
    {
        Launch l{};
        l.kind = Launch::Conv;
        l.dtype = a->dtype;
        ConvParams &c = l.conv;
        c.seqlen = a->cu_seqlens ? 0 : a->seqlen;
        c.cu_seqlens = a->cu_seqlens;
        c.D = di;
        c.K = a->d_conv;
        const int64_t maxlen = a->cu_seqlens ? a->max_seqlen : a->seqlen;
        c.nchunks = static_cast<int32_t>(std::max<int64_t>((maxlen + kConvTokens - 1) / kConvTokens, 1));
        const int64_t lane_ch = conv_lane_channels(a->dtype == R2L_DTYPE_BF16 ? 2 : 4);
        c.tiles = static_cast<int32_t>((di + kWG * lane_ch - 1) / (kWG * lane_ch));
        c.nblocks = a->batch * c.nchunks * c.tiles;
        c.x = xz; c.xs = 2 * di;
        c.w = a->conv_w;
        c.b = a->conv_b;
        c.u = u; c.us = di;
        out[n++] = l;
    }
    // 3. [r | B | C] = u W_x^T
    gemm(a->dt_rank + 2 * kN, di, u, di, a->W_x, xdbl, sp.ldx, nullptr, 0, 1.0f, 0.0f);
    // 4. r W_dt^T (the bias is added in the scan)
    gemm(di, a->dt_rank, xdbl, sp.ldx, a->W_dt, dtb, di, nullptr, 0, 1.0f, 0.0f);
    // 5. the gated R2L scan
    const r2l_scan_args v = sidecar_scan_view(a, sp);
    Launch ls[3];
    const int m = build_launches(Op::Scan, &v, sp.pl, ls);
    for (int i = 0; i < m; ++i) {
        if (ls[i].kind == Launch::Segment) {
            ls[i].mode = ls[i].mode == kModeState ? (kModeState | kModeBias) : (kModeGate | kModeBias);
            ls[i].seg.dt_bias = a->dt_bias;
        }
        out[n++] = ls[i];
    }
    // 6. out = hidden + s * g W_out^T
    gemm(dm, di, g, di, a->W_out, a->out, a->out_stride, a->hidden, a->hidden_stride, a->s, 1.0f);
    return n;
}

// ---- backward ------------------------------------------------------------------
BwdPlan make_bwd_plan(const r2l_scan_args *a, const r2l_grad_args *g, bool saved) {
    BwdPlan pl;
    pl.G = 4;
    pl.tiles = (a->dim * pl.G + kWG - 1) / kWG;
    pl.fwd_tiles = (a->dim + kWG - 1) / kWG;
    pl.tokens = tokens_of(a);
    pl.ck_rows = ckpt_rows(pl.tokens, a->batch);
    // Phase 1 runs one lane per channel; a shape with too few channels to
    // fill the machine scans chunks from zero in parallel (chunks are whole
    // checkpoint groups) and phase 2 adds each chunk's entry state to its
    // checkpoints. Phase 2 itself is not chunked.
    const int64_t maxlen = max_len_of(a);
    int64_t chunk = 0;
    if (a->chunk_tokens > 0) {
        chunk = a->chunk_tokens;
    } else if (a->chunk_tokens == 0 && maxlen > 0) {
        const int64_t lanes = std::max<int64_t>(a->batch * a->dim, 1);
        const int64_t fill = (kTargetLanes + lanes - 1) / lanes;
        if (fill > 1) chunk = std::max<int64_t>(kMinChunk, (maxlen + fill - 1) / fill);
    }
    chunk = (chunk + kCkptTokens - 1) / kCkptTokens * kCkptTokens;
    if (!saved && chunk > 0 && chunk < maxlen) {
        pl.chunked = true;
        pl.chunk_len = chunk;
        pl.nchunks = (maxlen + chunk - 1) / chunk;
    } else {
        pl.chunk_len = std::max<int64_t>(maxlen, 1);
        pl.nchunks = 1;
    }
    pl.saved = saved;
    if (a->res) {
        const bool is_x = a->res == a->x && a->res_stride == a->x_stride &&
                          eff_bstride(a, a->res_batch_stride, a->res_stride) ==
                              eff_bstride(a, a->x_batch_stride, a->x_stride);
        pl.res_kind = is_x ? 1 : 2;
    }
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align256(bytes);
        return at;
    };
    const size_t D = static_cast<size_t>(a->dim), B = static_cast<size_t>(a->batch);
    const size_t T = static_cast<size_t>(pl.tokens), tiles = static_cast<size_t>(pl.tiles);
    pl.off_ck = take(pl.tokens > 0 && !saved ? static_cast<size_t>(pl.ck_rows) * D * kN * 4 : 0);
    pl.off_B = take(g->dBm ? tiles * T * kN * 4 : 0);
    pl.off_C = take(g->dCm ? tiles * T * kN * 4 : 0);
    pl.off_A = take(g->dA ? B * D * kN * 4 : 0);
    pl.off_D = take(g->dDskip ? B * D * 4 : 0);
    pl.off_S = take(g->ds ? B * tiles * 4 : 0);
    if (pl.chunked) {
        const size_t nc = static_cast<size_t>(pl.nchunks);
        pl.off_Q = take(B * nc * D * kN * 4);
        pl.off_Sc = take(B * nc * D * 4);
        pl.off_H = take(B * nc * D * kN * 4);
        pl.off_cks = take(static_cast<size_t>(pl.ck_rows) * D * 4);
    }
    pl.ws_bytes = off;
    return pl;
}

int build_bwd_launches(bool reverse, const r2l_scan_args *a, const r2l_grad_args *g,
                       const BwdPlan &pl, Launch out[kMaxBwdLaunches], const float *saved_ckpt) {
    char *ws = static_cast<char *>(g->workspace);
    auto at = [&](size_t off, bool want) { return want ? reinterpret_cast<float *>(ws + off) : nullptr; };
    float *ck = pl.saved ? nullptr : at(pl.off_ck, pl.tokens > 0);
    float *pB = at(pl.off_B, g->dBm != nullptr), *pC = at(pl.off_C, g->dCm != nullptr);
    float *pA = at(pl.off_A, g->dA != nullptr), *pD = at(pl.off_D, g->dDskip != nullptr);
    float *pS = at(pl.off_S, g->ds != nullptr);
    const bool chunked = pl.chunked && pl.tokens > 0;
    float *Q = at(pl.off_Q, chunked), *Sc = at(pl.off_Sc, chunked);
    float *H = at(pl.off_H, chunked), *cks = at(pl.off_cks, chunked);
    const int64_t D = a->dim;
    int n = 0;

    if (a->batch > 0) {
        // phase 1: the forward state scan, one lane per channel, with checkpoints
        // (none when the forward saved them)
        if (pl.tokens > 0 && !pl.saved) {
            Plan fp;
            fp.G = 1;
            fp.chunk_len = pl.chunk_len;
            fp.nchunks = pl.nchunks;
            fp.tiles = pl.fwd_tiles;
            SegParams p = base_params(a, fp);
            p.res = nullptr;
            p.out = nullptr;
            p.ckpt = ck;
            p.bc_vec = bc_vector_ok(a, false) ? 1 : 0;
            if (chunked) {   // every chunk from zero: local checkpoints, Q, Delta sums
                p.hin = nullptr;
                p.hfin = Q; p.hfin_b = pl.nchunks * D * kN; p.hfin_c = D * kN;
                p.sdelta = Sc; p.sd_b = pl.nchunks * D; p.sd_c = D;
                p.ckpt_s = cks;
            } else {
                p.hin = a->h_in; p.hin_b = D * kN; p.hin_c = 0;
            }
            Launch l{};
            l.kind = Launch::Segment;
            l.reverse = reverse;
            l.dtype = a->dtype;
            l.G = 1;
            l.mode = kModeState | kModeCkpt;
            l.seg = p;
            out[n++] = l;
        }
        if (chunked) {   // the state entering every chunk (h_in before chunk 0)
            Launch c{};
            c.kind = Launch::Carry;
            c.reverse = reverse;
            c.dtype = a->dtype;
            c.carry.batch = a->batch;
            c.carry.seqlen = is_ragged(a) ? 0 : a->seqlen;
            c.carry.cu_seqlens = a->cu_seqlens;
            c.carry.D = D;
            c.carry.chunk_len = static_cast<int32_t>(pl.chunk_len);
            c.carry.nchunks = static_cast<int32_t>(pl.nchunks);
            c.carry.A = a->A;
            c.carry.hin = a->h_in;
            c.carry.c0_seeded = 0;
            c.carry.Q = Q;
            c.carry.S = Sc;
            c.carry.Hc = H;
            c.carry.hout = nullptr;
            out[n++] = c;
        }
        // phase 2: the adjoint
        BwdParams q{};
        q.seqlen = is_ragged(a) ? 0 : a->seqlen;
        q.cu_seqlens = a->cu_seqlens;
        q.D = D;
        q.tiles = static_cast<int32_t>(pl.tiles);
        q.nblocks = a->batch * pl.tiles;
        q.tokens = pl.tokens;
        q.x = a->x;   q.xs = a->x_stride;   q.xbs = eff_bstride(a, a->x_batch_stride, a->x_stride);
        q.dt = a->dt; q.dts = a->dt_stride; q.dtbs = eff_bstride(a, a->dt_batch_stride, a->dt_stride);
        q.Bm = a->Bm; q.Bs = a->Bm_stride;  q.Bbs = eff_bstride(a, a->Bm_batch_stride, a->Bm_stride);
        q.Cm = a->Cm; q.Cs = a->Cm_stride;  q.Cbs = eff_bstride(a, a->Cm_batch_stride, a->Cm_stride);
        q.bc_vec = bc_vector_ok(a, true) ? 1 : 0;
        q.A = a->A;
        q.Dskip = a->Dskip;
        q.softplus = a->delta_softplus;
        q.dyscale = pl.res_kind ? a->s : 1.0f;
        q.dxres = pl.res_kind == 1 ? 1.0f : 0.0f;
        q.want_ds = g->ds ? 1 : 0;
        q.ckpt = pl.saved ? saved_ckpt : ck;
        if (chunked) {
            q.chunk_len = static_cast<int32_t>(pl.chunk_len);
            q.nchunks = static_cast<int32_t>(pl.nchunks);
            q.Hc = H;
            q.ckpt_s = cks;
        }
        q.dout = g->dout; q.gs = g->dout_stride;
        q.gbs = eff_bstride(a, g->dout_batch_stride, g->dout_stride);
        q.dh_out = g->dh_out;
        q.dx = g->dx;   q.dxs = g->dx_stride;   q.dxbs = eff_bstride(a, g->dx_batch_stride, g->dx_stride);
        q.ddt = g->ddt; q.dds = g->ddt_stride;  q.ddbs = eff_bstride(a, g->ddt_batch_stride, g->ddt_stride);
        q.dh_in = g->dh_in;
        q.partB = pB; q.partC = pC; q.partA = pA; q.partD = pD; q.partS = pS;
        Launch l{};
        l.kind = Launch::Backward;
        l.reverse = reverse;
        l.dtype = a->dtype;
        l.G = pl.G;
        l.bwd = q;
        out[n++] = l;
    }
    // the ordered sums, one launch (with no sequence they write zeros)
    Launch l{};
    l.kind = Launch::Sum;
    auto sum = [&](const float *src, int64_t P, int64_t pstride, int64_t cnt, float *dst) {
        l.sums.seg[l.sums.count++] = SumParams{src, P, pstride, cnt, dst};
    };
    const int64_t T = pl.tokens;
    if (g->dBm && T > 0) sum(pB, pl.tiles, T * kN, T * kN, g->dBm);
    if (g->dCm && T > 0) sum(pC, pl.tiles, T * kN, T * kN, g->dCm);
    if (g->dA) sum(pA, a->batch, D * kN, D * kN, g->dA);
    if (g->dDskip) sum(pD, a->batch, D, D, g->dDskip);
    if (g->ds) sum(pS, a->batch * pl.tiles, 1, 1, g->ds);
    if (l.sums.count) out[n++] = l;
    return n;
}

}  // namespace r2l
