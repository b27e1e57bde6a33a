// scan_kernels.hip -- gfx950 kernels of the R2L / forward selective scans.
//
// The operation (see include/r2l_scan.h for the full contract and its sources):
// per sequence, channel d and state n, tokens visited right to left (the R2L
// stream of "Bifocal Diffusion Language Models", section 2) or left to right
// (the forward-only boundary states of "Training Hybrid Block Diffusion
// Language Models with Partial Bidirectionality", "Methodology" item 1):
//     Delta = softplus(dt);  h_n = exp(Delta*A[d,n])*h_n + Delta*Bm[t,n]*x[t,d]
//     y = sum_n Cm[t,n]*h_n + Dskip[d]*x[t,d];  out = res + s*y  (s == 0: res)
//
// Mapping onto CDNA4. This is a recurrence over tokens with one exp per
// (token, channel, state): vector ALU work, no dense contraction, so no MFMA.
//  * Lanes run over channels: G lanes (1, 2 or 4) own one channel and hold its
//    N/G fp32 states in VGPRs for the whole segment. A wave reads 64/G
//    consecutive channels of a token row: one coalesced 64/G*sizeof(T) span
//    per tensor and token.
//  * Bm/Cm rows are shared by every channel. A workgroup stages kTile rows of
//    them in LDS as fp32 (converted once), and every wave reads them back as
//    broadcasts.
//  * The reversal is only the sign of the token step in the address math; the
//    output goes back to the token's own row, so nothing is flipped in memory.
//  * Softplus and the decay are computed in-kernel with the hardware base-2
//    exponential and logarithm (v_exp_f32 / v_log_f32), log2(e) being folded
//    into A once per lane.
//  * The gated residual res + s*y is fused into the store; bf16 outputs use
//    the hardware round-to-nearest-even conversion. (With s == 0 the output is
//    the residual bit for bit: the planner copies it, or leaves it in place,
//    and runs no readout.)
//  * Long sequences can be cut into chunks scanned from a zero state in
//    parallel; the carry kernel then chains the chunk results. Because the
//    recurrence is linear, a chunk's contribution to the state after it is its
//    local final state Q plus exp(A * sum(Delta)) times the state entering it.
//  * Block ids are remapped so that the tiles of one segment, which read the
//    same Bm/Cm rows, are dispatched to the same XCD (blocks go round-robin
//    over the 8 XCDs, each with its own L2).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scan_device.h"
#include "scan_geometry.h"
#include "scan_internal.h"

namespace r2l {
namespace {

using namespace dev;

// ---- the segment scan ------------------------------------------------------
// One workgroup scans one segment (a chunk of one sequence) for kWG/G channels.
// Per lane and token: Delta, then for each of its NS states one exp, the state
// update and (READOUT) the readout term; the G partial readouts are summed
// across the lane group; then the skip term and the gated residual.
//
// Latency hiding: x / dt / res of the token PF positions ahead are loaded into
// a register ring before the current token is computed, and the Bm/Cm rows of
// the next kTile tokens are fetched into registers during the current tile and
// written to the other half of a double-buffered LDS area at its end (one
// barrier per tile). Row addresses are uniform (scalar) and the lane adds a
// 32-bit channel offset.
template <bool REV, typename T, int G, int MODE, bool SP>
__device__ __forceinline__ void scan_segment(const SegParams &p, float *lds, const BlockGeom &bg,
                                             const SeqGeom &sq, const SegGeom &sg,
                                             const float *hin) {
    constexpr bool READOUT = MODE != kModeState;
    constexpr int NS = kN / G;                   // states per lane
    constexpr int NBC = READOUT ? 2 * kN : kN;   // staged floats per token (B, then C)
    constexpr int STAGE = stage_cols(NBC);       // staged elements per thread per tile
    constexpr int SW = STAGE * static_cast<int>(sizeof(T)) / 4;   // ... as 32-bit words
    constexpr int PF = kPrefetch;
    static_assert(kTile * NBC == STAGE * kWG && kN % STAGE == 0 && STAGE % 4 == 0 &&
                  kTile % PF == 0, "tile shape");
    float (*lds_bc)[kTile * NBC] = reinterpret_cast<float (*)[kTile * NBC]>(lds);
    using E = Elem<T>;
    using R = typename E::raw_t;

    const int64_t b = bg.b;
    const int c = bg.c;
    const int ntok = sg.ntok;

    const LaneGeom lg = lane_geom(bg.tile, threadIdx.x, G, p.D);
    const uint32_t dl = lg.d;
    const int sub = lg.sub;

    float a2[NS], h[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) a2[j] = p.A[dl * kN + sub * NS + j] * kLog2e;
    if (hin) {
        const float *hp = hin + dl * kN + sub * NS;
#pragma unroll
        for (int j = 0; j < NS; ++j) h[j] = hp[j];
    } else {
#pragma unroll
        for (int j = 0; j < NS; ++j) h[j] = 0.0f;
    }
    const float dskip = (READOUT && p.Dskip) ? p.Dskip[dl] : 0.0f;
    float dsum = 0.0f;

    // Per-token rows go through raw buffer resources based at the sequence's
    // first row: the row offset is a scalar (row * row bytes) and the lane
    // adds its fixed 32-bit channel offset. The resource bound only checks the
    // lane offset, so every row used below is one of the segment's own rows;
    // the host guarantees that one sequence of one tensor spans < 4 GiB.
    const uint32_t es = static_cast<uint32_t>(sizeof(T));
    const uint32_t doff = dl * es;
    const uint32_t xrb = static_cast<uint32_t>(p.xs) * es, drb = static_cast<uint32_t>(p.dts) * es;
    const uint32_t rrb = static_cast<uint32_t>(p.rs) * es, orb = static_cast<uint32_t>(p.os) * es;
    const auto rx = make_rsrc(static_cast<const T *>(p.x) + sq.xo,
                              seq_span_bytes(sq.len, p.xs, p.D, es));
    const auto rd = make_rsrc(static_cast<const T *>(p.dt) + sq.dto,
                              seq_span_bytes(sq.len, p.dts, p.D, es));
    const auto rr_ = make_rsrc(MODE == kModeRes ? static_cast<const T *>(p.res) + sq.ro : nullptr,
                               MODE == kModeRes ? seq_span_bytes(sq.len, p.rs, p.D, es) : 0);
    const auto ro_ = make_rsrc(READOUT ? static_cast<T *>(p.out) + sq.oo : nullptr,
                               READOUT ? seq_span_bytes(sq.len, p.os, p.D, es) : 0);
    // Staging: this thread's matrix (uniform per wave) as one resource.
    const StageSlot ss = stage_slot(threadIdx.x, NBC);
    const bool stage_c = READOUT && __builtin_amdgcn_readfirstlane(ss.mat) != 0;
    const auto rbc = stage_c
        ? make_rsrc(static_cast<const T *>(p.Cm) + sq.Co, seq_span_bytes(sq.len, p.Cs, kN, es))
        : make_rsrc(static_cast<const T *>(p.Bm) + sq.Bo, seq_span_bytes(sq.len, p.Bs, kN, es));
    const uint32_t bcrb = static_cast<uint32_t>(stage_c ? p.Cs : p.Bs) * es;
    const uint32_t bccol = static_cast<uint32_t>(ss.col0) * es;
    const bool bc_vec = p.bc_vec != 0;
    const float gate = p.s;   // never 0 in the residual modes

    // ---- register ring of per-token inputs (slot = position % PF)
    R xq[PF], dq[PF], rq[PF];
    auto load_pos = [&](int k, int slot) {       // k: a visited position of this segment
        const uint32_t row = static_cast<uint32_t>(seg_row(sg, k));
        xq[slot] = E::bload(rx, doff, row * xrb);
        dq[slot] = E::bload(rd, doff, row * drb);
        if constexpr (MODE == kModeRes) rq[slot] = E::bload(rr_, doff, row * rrb);
    };

    // ---- Bm/Cm staging of one tile of kTile tokens
    uint32_t stw[SW];
    auto stage_load = [&](int tbase, int tcnt) {   // tcnt >= 1
        const uint32_t row = static_cast<uint32_t>(seg_row(sg, tbase + stage_pos(ss.k, tcnt)));
        const uint32_t voff = row * bcrb + bccol;
        if (bc_vec)
            bload_words<SW>(rbc, voff, stw);
        else
            E::template bload_elems<STAGE>(rbc, voff, stw);
    };
    auto stage_store = [&](int buf) {
        float4 *dst = reinterpret_cast<float4 *>(&lds_bc[buf][ss.k * NBC + ss.mat * kN + ss.col0]);
#pragma unroll
        for (int q = 0; q < STAGE / 4; ++q)
            dst[q] = make_float4(E::word_elem(stw, 4 * q), E::word_elem(stw, 4 * q + 1),
                                 E::word_elem(stw, 4 * q + 2), E::word_elem(stw, 4 * q + 3));
    };

    // One visited position k: consume ring slot `slot`, refill it with the
    // position PF ahead, update the state and store the output row.
    // Delta of the next visited position is computed one token ahead, off
    // the critical path of the current token (its dt is already in the ring).
    float dnext = 0.0f;
    auto delta_of = [&](R dr) {
        const float dv = E::widen(dr);
        if constexpr (SP)
            return softplus(dv);
        else
            return dv;
    };
    auto token = [&](int k, const float *bcrow, int slot) {
        const R xr = xq[slot], rr = rq[slot];
        const float delta = dnext;
        dnext = delta_of(dq[(slot + 1) % PF]);
        load_pos(prefetch_pos(k + PF, ntok), slot);
        const float xv = E::widen(xr);
        if constexpr (!READOUT) dsum += delta;
        const float dx = delta * xv;
        const float *row = bcrow + sub * NS;
        // the readout sums even and odd states separately: two short
        // dependency chains instead of one of NS fmas
        float y0 = 0.0f, y1 = 0.0f;
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            const float abar = __builtin_amdgcn_exp2f(delta * a2[n]);
            h[n] = fmaf(abar, h[n], row[n] * dx);
            if constexpr (READOUT) {
                if (n & 1)
                    y1 = fmaf(row[kN + n], h[n], y1);
                else
                    y0 = fmaf(row[kN + n], h[n], y0);
            }
        }
        if constexpr (READOUT) {
            float y = group_sum<G>(y0 + y1);
            y = fmaf(dskip, xv, y);
            // Every lane stores: the G lanes of a channel, and idle lanes
            // shadowing the last channel, hold bit-identical values for the
            // same address.
            R o;
            if constexpr (MODE == kModeY) {
                o = E::pack(y);
            } else {
                const R rbits = MODE == kModeRes ? rr : xr;
                o = E::pack(fmaf(gate, y, E::widen(rbits)));
            }
            const uint32_t orow = static_cast<uint32_t>(seg_row(sg, k));
            E::bstore(o, ro_, doff, orow * orb);
        }
    };

    // Backward phase 1: the state entering each group of kCkptTokens visited
    // positions (the groups are the prefetch groups).
    static_assert(PF == kCkptTokens, "checkpoint groups are the prefetch groups");
    auto checkpoint = [&](int pos) {
        if (!p.ckpt || !lg.active) return;
        float *cp = p.ckpt + (ckpt_row(b, sq.s0p, pos) * p.D + dl) * kN + sub * NS;
#pragma unroll
        for (int j = 0; j < NS; ++j) cp[j] = h[j];
    };

    // Start-up: the first tile's Bm/Cm rows are requested first (they gate
    // the barrier), then the first PF tokens of x/dt/res.
    const int ntiles = (ntok + kTile - 1) / kTile;
    const int cnt0 = ntok < kTile ? ntok : kTile;
    if (ntok > 0) stage_load(0, cnt0);
#pragma unroll
    for (int j = 0; j < PF; ++j) rq[j] = 0;
    if (ntok > 0) {
#pragma unroll
        for (int j = 0; j < PF; ++j) load_pos(prefetch_pos(j, ntok), j);
        stage_store(0);
        dnext = delta_of(dq[0]);
    }
    __syncthreads();

    for (int ti = 0; ti < ntiles; ++ti) {
        const int base = ti * kTile;
        const int cnt = ntok - base < kTile ? ntok - base : kTile;
        const bool more = ti + 1 < ntiles;
        const int ncnt = more ? (ntok - base - kTile < kTile ? ntok - base - kTile : kTile) : 0;
        if (more) stage_load(base + kTile, ncnt);
        const float *bc = lds_bc[ti & 1];

        const int full = cnt - cnt % PF;
        for (int k0 = 0; k0 < full; k0 += PF) {
            if constexpr (!READOUT) checkpoint(base + k0);
#pragma unroll
            for (int j = 0; j < PF; ++j) token(base + k0 + j, bc + (k0 + j) * NBC, j);
        }
        if constexpr (!READOUT)
            if (full < cnt) checkpoint(base + full);
#pragma unroll
        for (int j = 0; j < PF; ++j)            // the last tile's partial group
            if (full + j < cnt) token(base + full + j, bc + (full + j) * NBC, j);

        if (more) stage_store((ti + 1) & 1);
        __syncthreads();
    }

    if (p.hfin && lg.active) {
        float *hp = p.hfin + b * p.hfin_b + c * p.hfin_c + dl * kN + sub * NS;
#pragma unroll
        for (int j = 0; j < NS; ++j) hp[j] = h[j];
    }
    if (!READOUT && p.sdelta && lg.active && sub == 0) p.sdelta[b * p.sd_b + c * p.sd_c + dl] = dsum;
}

// One workgroup per (sequence b, chunk c, channel tile). Chunk passes of
// readout plans (split_c0) run the readout on chunk 0, which starts from the
// call's own initial state, and the state-only scan from zero on the others.
template <bool REV, typename T, int G, int MODE, bool SP>
__global__ __launch_bounds__(kWG) void segment_scan_kernel(const SegParams p) {
    constexpr int NBC_MAX = MODE != kModeState ? 2 * kN : kN;
    __shared__ __align__(16) float lds[2 * kTile * NBC_MAX];

    const BlockGeom bg = block_geom(p.nblocks, p.tiles, p.nchunks, blockIdx.x);
    if (!bg.valid) return;
    const int64_t b = bg.b;
    const int c = bg.c;
    const int64_t s0 = p.cu_seqlens ? p.cu_seqlens[b] : 0;
    const int64_t s1 = p.cu_seqlens ? p.cu_seqlens[b + 1] : 0;
    const SeqGeom sq = seq_geom(p, b, s0, s1);
    const SegGeom sg = seg_geom(REV, c, p.chunk_len, sq.len);
    if (!segment_runs(p, sg, c)) return;
    const float *hin = segment_hin(p, b, c);
    if constexpr (MODE != kModeState) {
        if (p.split_c0 && c > 0) {
            scan_segment<REV, T, G, kModeState, SP>(p, lds, bg, sq, sg, hin);
            return;
        }
    }
    scan_segment<REV, T, G, MODE, SP>(p, lds, bg, sq, sg, hin);
}

// ---- the carry over chunks -------------------------------------------------
// One lane per (sequence, channel, state); the chunk loop is short and its
// loads do not depend on the carried value, so they pipeline.
__global__ __launch_bounds__(kCarryThreads) void carry_kernel(const CarryParams p) {
    const CarryGeom g = carry_geom(p.D, blockIdx.x, blockIdx.y, threadIdx.x);
    if (!g.valid) return;
    const int64_t len = p.cu_seqlens
        ? static_cast<int64_t>(p.cu_seqlens[g.b + 1]) - p.cu_seqlens[g.b] : p.seqlen;
    const int nc = carry_chunks(len, p.chunk_len, p.nchunks);
    const float a2 = p.A[g.d * kN + g.n] * kLog2e;
    // seeded: chunk 0 was scanned from the call's initial state, so its
    // local final state is already the true state after it
    float H = p.c0_seeded ? p.Q[(g.b * p.nchunks * p.D + g.d) * kN + g.n]
                          : (p.hin ? p.hin[(g.b * p.D + g.d) * kN + g.n] : 0.0f);
    for (int c = p.c0_seeded ? 1 : 0; c < nc; ++c) {
        const int64_t sc = (g.b * p.nchunks + c) * p.D + g.d;
        if (p.Hc) p.Hc[sc * kN + g.n] = H;
        if (c == nc - 1 && !p.hout) break;   // the last chunk's local results are not needed
        const float P = __builtin_amdgcn_exp2f(a2 * p.S[sc]);
        H = fmaf(P, H, p.Q[sc * kN + g.n]);
    }
    if (p.hout) p.hout[(g.b * p.D + g.d) * kN + g.n] = H;
}

// ---- copy of token rows (the output of a call with s == 0 is the residual) -
template <typename R>
__global__ __launch_bounds__(kCopyThreads) void copy_rows_kernel(const CopyParams p) {
    const int64_t col = static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x;
    if (col >= p.D) return;
    const R *src = static_cast<const R *>(p.src);
    R *dst = static_cast<R *>(p.dst);
    for (int64_t r = blockIdx.y; r < p.rows; r += gridDim.y) {
        const CopyRow cr = copy_row(p, r);
        dst[cr.dst + col] = src[cr.src + col];
    }
}

template <bool REV, typename T, int MODE, bool SP>
hipError_t launch_g(int G, const SegParams &p, hipStream_t stream) {
    const int64_t grid = padded_grid(p.nblocks);
    switch (G) {
        case 1:
            hipLaunchKernelGGL((segment_scan_kernel<REV, T, 1, MODE, SP>), dim3(grid), dim3(kWG),
                               0, stream, p);
            break;
        case 2:
            hipLaunchKernelGGL((segment_scan_kernel<REV, T, 2, MODE, SP>), dim3(grid), dim3(kWG),
                               0, stream, p);
            break;
        case 4:
            hipLaunchKernelGGL((segment_scan_kernel<REV, T, 4, MODE, SP>), dim3(grid), dim3(kWG),
                               0, stream, p);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool REV, typename T, bool SP>
hipError_t launch_m(int mode, int G, const SegParams &p, hipStream_t stream) {
    switch (mode) {
        case kModeState: return launch_g<REV, T, kModeState, SP>(G, p, stream);
        case kModeY: return launch_g<REV, T, kModeY, SP>(G, p, stream);
        case kModeResX: return launch_g<REV, T, kModeResX, SP>(G, p, stream);
        case kModeRes: return launch_g<REV, T, kModeRes, SP>(G, p, stream);
        default: return hipErrorInvalidValue;
    }
}

template <bool REV, typename T>
hipError_t launch_s(int mode, int G, const SegParams &p, hipStream_t stream) {
    return p.softplus ? launch_m<REV, T, true>(mode, G, p, stream)
                      : launch_m<REV, T, false>(mode, G, p, stream);
}

}  // namespace

hipError_t launch_segment_scan(bool reverse, int dtype, int G, int mode, const SegParams &p,
                               hipStream_t stream) {
    if (reverse)
        return dtype == 1 ? launch_s<true, uint16_t>(mode, G, p, stream)
                          : launch_s<true, float>(mode, G, p, stream);
    return dtype == 1 ? launch_s<false, uint16_t>(mode, G, p, stream)
                      : launch_s<false, float>(mode, G, p, stream);
}

hipError_t launch_copy(int dtype, const CopyParams &p, hipStream_t stream) {
    if (p.rows <= 0 || p.D <= 0) return hipSuccess;
    const dim3 grid(static_cast<uint32_t>((p.D + kCopyThreads - 1) / kCopyThreads),
                    static_cast<uint32_t>(p.rows < kCopyMaxRowBlocks ? p.rows : kCopyMaxRowBlocks));
    if (dtype == 1)
        hipLaunchKernelGGL(copy_rows_kernel<uint16_t>, grid, dim3(kCopyThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(copy_rows_kernel<uint32_t>, grid, dim3(kCopyThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_carry(const CarryParams &p, hipStream_t stream) {
    const dim3 grid(static_cast<uint32_t>(p.batch), static_cast<uint32_t>(carry_tiles(p.D)));
    hipLaunchKernelGGL(carry_kernel, grid, dim3(kCarryThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace r2l
