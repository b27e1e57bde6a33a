// scan_plan.h -- how one entry-point call becomes kernel launches. Used by the
// entry points (r2l_api.cpp) and by the host-side access checker
// (bounds_check.cpp), so both see the same launches with the same parameters.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "r2l_scan.h"
#include "scan_internal.h"

namespace r2l {

enum class Op { Scan, Prefix, Commit };

struct Plan {
    int G = 1;               // lanes per channel
    bool chunked = false;
    int64_t chunk_len = 0;   // tokens per chunk (visiting order)
    int64_t nchunks = 1;
    int64_t tiles = 0;       // channel tiles per segment
    size_t ws_bytes = 0;     // Q, S (+ H for readout plans), each 256-byte aligned
    size_t off_S = 0, off_H = 0;
};

struct Launch {
    enum Kind { Segment, Carry, Copy, Backward, Sum, Bidir, Conv, Gemm } kind;
    bool reverse;
    int dtype;
    int G;
    int mode;                // kMode* (segment launches)
    SegParams seg;           // (Bidir: the reverse pass)
    SegParams seg2;          // Bidir: the forward pass
    CarryParams carry;
    CopyParams copy;
    BwdParams bwd;
    SumBatch sums;
    ConvParams conv;
    GemmParams gemm;
};

// The backward of r2l_scan: phase 1 (state-only segment scan writing
// checkpoints; when chunked, from zero per chunk, then the carry of the
// chunk entry states), phase 2 (the adjoint) and one launch of ordered sums.
constexpr int kMaxBwdLaunches = 4;
struct BwdPlan {
    int G = 4;               // lanes per channel in phase 2
    int64_t tiles = 0;       // phase-2 channel tiles per sequence
    int64_t fwd_tiles = 0;   // phase-1 tiles (one lane per channel)
    int64_t tokens = 0;
    int64_t ck_rows = 0;
    bool chunked = false;    // phase 1 cut into chunks (a multiple of kCkptTokens)
    bool saved = false;      // the checkpoints were saved by the forward: no phase 1
    int64_t chunk_len = 0, nchunks = 1;
    size_t ws_bytes = 0;
    size_t off_ck = 0, off_B = 0, off_C = 0, off_A = 0, off_D = 0, off_S = 0;
    // chunked phase 1: local final states Q, Delta sums, entry states H
    // ([batch][nchunks][D](x kN)) and the checkpoints' Delta sums [ck_rows][D]
    size_t off_Q = 0, off_Sc = 0, off_H = 0, off_cks = 0;
    int res_kind = 0;        // 0: none, 1: the residual is x, 2: a separate residual
};

// saved: the checkpoints come from r2l_scan_save (no phase 1, no checkpoint area)
BwdPlan make_bwd_plan(const r2l_scan_args *a, const r2l_grad_args *g, bool saved = false);
// reverse: the backward of r2l_scan (true) or of the forward-direction readout (false)
int build_bwd_launches(bool reverse, const r2l_scan_args *a, const r2l_grad_args *g,
                       const BwdPlan &pl, Launch out[kMaxBwdLaunches],
                       const float *saved_ckpt = nullptr);

inline bool is_ragged(const r2l_scan_args *a) { return a->cu_seqlens != nullptr; }
inline int64_t tokens_of(const r2l_scan_args *a) {
    return is_ragged(a) ? a->total_tokens : a->batch * a->seqlen;
}
inline int64_t max_len_of(const r2l_scan_args *a) {
    return is_ragged(a) ? a->max_seqlen : a->seqlen;
}
inline bool wants_readout(Op op, const r2l_scan_args *a) {
    return op == Op::Scan || a->out != nullptr;
}
// A readout call whose gate s is 0 outputs its residual bit for bit: no
// readout runs; the residual is copied to out (or already is out), and the
// state is scanned only when h_out is wanted.
inline bool gate_closed(Op op, const r2l_scan_args *a) {
    return wants_readout(op, a) && a->res != nullptr && a->s == 0.0f;
}
inline bool runs_readout(Op op, const r2l_scan_args *a) {
    return wants_readout(op, a) && !gate_closed(op, a);
}
// Whether any segment scan runs at all.
inline bool runs_scan(Op op, const r2l_scan_args *a) {
    return !gate_closed(op, a) || a->h_out != nullptr;
}
inline int64_t elem_size(int32_t dtype) { return dtype == R2L_DTYPE_BF16 ? 2 : 4; }

// Batch stride actually used by a token-major tensor in the dense layout.
inline int64_t eff_bstride(const r2l_scan_args *a, int64_t bstride, int64_t stride) {
    if (is_ragged(a)) return 0;
    return bstride ? bstride : a->seqlen * stride;
}

// ckpt: the plan of a scan that saves the backward's checkpoints (chunks are
// whole checkpoint groups)
Plan make_plan(Op op, const r2l_scan_args *a, bool ckpt = false);

// The bidirectional scan (bidir_scan): the reverse direction's readout into
// fp32 workspace rows, then the forward direction's readout adding them; one
// fused launch when the plan does not chunk. Both directions share one plan
// (same shape, one lane per channel).
constexpr int kMaxBidirLaunches = 6;
struct BidirPlan {
    Plan pl;                 // either direction's plan (the forward's alone when the gate is closed)
    bool readout = false;    // false: s == 0 with a residual (out = res, forward state only)
    bool fused = false;
    size_t off_chunk = 0;    // the plans' carry workspace after the fp32 rows
    size_t ws_bytes = 0;
};
BidirPlan make_bidir_plan(const r2l_scan_args *a);
// The reverse direction's arguments: x and the shape from `a`, the parameters
// from `rev` (NULL pointers: the forward's), no residual, state or output.
r2l_scan_args reverse_view(const r2l_scan_args *a, const r2l_dir_args *rev);
int build_bidir_launches(const r2l_scan_args *a, const r2l_dir_args *rev, const BidirPlan &bp,
                         Launch out[kMaxBidirLaunches]);

// The sidecar block (r2l_sidecar_forward): in-projection GEMM, conv + SiLU,
// x-projection GEMM, dt-projection GEMM, the gated R2L scan (its own plan),
// out-projection GEMM with the residual; or only the residual copy when s == 0.
constexpr int kMaxSidecarLaunches = 8;
constexpr size_t kGemmWorkspace = size_t(32) << 20;   // hipBLASLt scratch
struct SidecarPlan {
    bool runs = false;       // false: s == 0 (out = hidden)
    Plan pl;                 // the scan's plan
    int64_t tokens = 0;
    int64_t ldx = 0;         // elements per [r | B | C] row (dt_rank + 2 N, rounded up to 8)
    size_t off_xz = 0, off_u = 0, off_xdbl = 0, off_dt = 0, off_g = 0, off_chunk = 0,
           off_gemm = 0, ws_bytes = 0;
};
SidecarPlan make_sidecar_plan(const r2l_sidecar_args *a);
// The scan of the block as an r2l_scan call on the workspace: x = u, dt,
// Bm, Cm = the columns of [r | B | C], the residual slot = z, out = the gated y.
r2l_scan_args sidecar_scan_view(const r2l_sidecar_args *a, const SidecarPlan &sp);
int build_sidecar_launches(const r2l_sidecar_args *a, const SidecarPlan &sp,
                           Launch out[kMaxSidecarLaunches]);

// The launches of a call, in order (at most 3). Arguments must have passed
// the entry point's checks. Returns the count.
int build_launches(Op op, const r2l_scan_args *a, const Plan &pl, Launch out[3]);

// r2l_scan_save (op Scan) and prefix_scan_save (op Prefix): the launches of
// the call (plan made with ckpt = true, one lane per channel) whose readout
// scans also store the checkpoints at ckpt; when no readout runs (s == 0, or
// a prefix call without one), one more state-only scan stores them.
constexpr int kMaxSaveLaunches = 4;
int build_save_launches(Op op, const r2l_scan_args *a, const Plan &pl, float *ckpt,
                        Launch out[kMaxSaveLaunches]);
// Bytes of the checkpoints of a call: ckpt_rows(tokens, batch) x D x kN fp32.
size_t checkpoint_bytes(const r2l_scan_args *a);

}  // namespace r2l
