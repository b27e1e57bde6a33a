// scan_segment.h -- the segment scan of the gfx950 selective-scan kernels
// (device code, included by the .hip files that instantiate it: the scans of
// the three entry points in scan_kernels.hip, the bidirectional scan's in
// bidir_kernels.hip). See scan_kernels.hip for how it maps onto CDNA4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scan_device.h"
#include "scan_geometry.h"
#include "scan_internal.h"

namespace r2l {
namespace {

using namespace dev;

// Waves that share a SIMD run the same code; with equal priority the older
// one issues first and finishes early, leaving the others to run their last
// tokens with fewer waves to hide latency. So the two waves of a SIMD take
// turns, group by group, at the higher of two levels (by the parity of their
// slot on the SIMD), both dropping to the lower pair for their last group:
// denoising hook 20.4 -> 19.7 us, prefill unchanged, against a ladder that
// only lowered a wave's priority over its last three groups (which had gained
// 2.5% on the prefill's 456-token chunks; builds alternated on one box).
__device__ __forceinline__ void set_prio(int p) {
    if (p >= 3)
        __builtin_amdgcn_s_setprio(3);
    else if (p == 2)
        __builtin_amdgcn_s_setprio(2);
    else if (p == 1)
        __builtin_amdgcn_s_setprio(1);
    else
        __builtin_amdgcn_s_setprio(0);
}
__device__ __forceinline__ void wave_priority_by_work_left(int tokens_left, int alt) {
    const int q = (tokens_left - 1) / kPrefetch;   // groups left after this one
    set_prio((q >= 1 ? 2 : 0) + ((alt + q) & 1));
}

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
                                             const float *hin, float *ylds = nullptr) {
    constexpr int OUT = MODE & kModeOutMask;     // what the readout writes
    constexpr bool ADD = (MODE & kModeAdd) != 0;  // y += an fp32 addend per token
    // the fp32 rows (kModeWs / kModeAdd) at ylds[row * kWG + thread] in LDS
    constexpr bool LROWS = (MODE & kModeLds) != 0;
    constexpr bool CK = (MODE & kModeCkpt) != 0;   // store checkpoints
    constexpr bool BIAS = (MODE & kModeBias) != 0;  // dt += dt_bias[d] before softplus
    constexpr bool READS_RES = OUT == kModeRes || OUT == kModeGate;
    constexpr bool READOUT = OUT != kModeState;
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

    // A * log2(e), the state and Dskip: read at start-up, after the first
    // rows are requested (below)
    float a2[NS], h[NS];
    float dskip = 0.0f;
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
    const auto rr_ = make_rsrc(READS_RES ? static_cast<const T *>(p.res) + sq.ro : nullptr,
                               READS_RES ? seq_span_bytes(sq.len, p.rs, p.D, es) : 0);
    constexpr bool TO_OUT = READOUT && OUT != kModeWs;
    const auto ro_ = make_rsrc(TO_OUT ? static_cast<T *>(p.out) + sq.oo : nullptr,
                               TO_OUT ? seq_span_bytes(sq.len, p.os, p.D, es) : 0);
    // fp32 rows [packed token, D] of the workspace: y written (kModeWs) or the
    // addend read (kModeAdd), at the sequence's packed rows
    const uint32_t wrb = static_cast<uint32_t>(p.D) * 4u, woff = dl * 4u;
    const auto rw_ = make_rsrc(OUT == kModeWs && !LROWS ? p.yws + sq.s0p * p.D : nullptr,
                               OUT == kModeWs && !LROWS ? seq_span_bytes(sq.len, p.D, p.D, 4) : 0);
    const auto ra_ = make_rsrc(ADD && !LROWS ? p.yadd + sq.s0p * p.D : nullptr,
                               ADD && !LROWS ? seq_span_bytes(sq.len, p.D, p.D, 4) : 0);
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
    uint32_t aq[PF];
    auto load_pos = [&](int k, int slot) {       // k: a visited position of this segment
        const uint32_t row = static_cast<uint32_t>(seg_row(sg, k));
        xq[slot] = E::bload(rx, doff, row * xrb);
        dq[slot] = E::bload(rd, doff, row * drb);
        if constexpr (READS_RES) rq[slot] = E::bload(rr_, doff, row * rrb);
        if constexpr (ADD && !LROWS) aq[slot] = __builtin_amdgcn_raw_buffer_load_b32(ra_, woff, row * wrb, 0);
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
    const float dtb = (BIAS && p.dt_bias) ? p.dt_bias[dl] : 0.0f;
    auto delta_of = [&](R dr) {
        const float dv = BIAS ? E::widen(dr) + dtb : E::widen(dr);
        if constexpr (SP)
            return softplus(dv);
        else
            return dv;
    };
    auto token = [&](int k, const float *bcrow, int slot) {
        const R xr = xq[slot], rr = rq[slot];
        const uint32_t addend = aq[slot];
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
            const uint32_t orow = static_cast<uint32_t>(seg_row(sg, k));
            // LDS row, clamped: a sequence longer than the plan's maximum (a
            // broken max_seqlen) stays inside the array
            const uint32_t lrow = orow < kBidirLdsTokens ? orow : kBidirLdsTokens - 1;
            if constexpr (ADD) {
                if constexpr (LROWS)
                    y += ylds[lrow * kWG + threadIdx.x];
                else
                    y += __uint_as_float(addend);
            }
            if constexpr (OUT == kModeWs) {
                if constexpr (LROWS)
                    ylds[lrow * kWG + threadIdx.x] = y;
                else
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), rw_, woff, orow * wrb, 0);
            } else {
                R o;
                if constexpr (OUT == kModeY) {
                    o = E::pack(y);
                } else if constexpr (OUT == kModeGate) {
                    const float zv = E::widen(rr);   // y * SiLU(z) = y * z / (1 + e^-z)
                    o = E::pack(y * zv * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zv * kLog2e)));
                } else {
                    const R rbits = OUT == kModeRes ? rr : xr;
                    o = E::pack(fmaf(gate, y, E::widen(rbits)));
                }
                E::bstore(o, ro_, doff, orow * orb);
            }
        }
    };

    // Checkpoints (kModeCkpt): the state entering each group of kCkptTokens
    // visited positions (the groups are the prefetch groups; chunks are whole
    // groups) and, in the backward's chunked phase 1, the chunk's Delta sum
    // up to it.
    static_assert(PF == kCkptTokens, "checkpoint groups are the prefetch groups");
    auto checkpoint = [&](int pos) {
        if (!p.ckpt || !lg.active) return;
        const int64_t row = ckpt_row(b, sq.s0p, static_cast<int64_t>(c) * p.chunk_len + pos);
        static_assert(NS % 4 == 0, "checkpoints are stored by quads of states");
#pragma unroll
        for (int q = 0; q < NS / 4; ++q)
            *reinterpret_cast<float4 *>(p.ckpt + ckpt_quad(row, p.D, dl, sub * (NS / 4) + q)) =
                make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
        if constexpr (!READOUT)
            if (p.ckpt_s && sub == 0) p.ckpt_s[row * p.D + dl] = dsum;
    };

    // Start-up: the first tile's Bm/Cm rows are requested first (they gate
    // the barrier), then the first PF tokens of x/dt/res.
    const int ntiles = (ntok + kTile - 1) / kTile;
    const int cnt0 = ntok < kTile ? ntok : kTile;
    if (ntok > 0) stage_load(0, cnt0);
#pragma unroll
    for (int j = 0; j < PF; ++j) {
        rq[j] = 0;
        aq[j] = 0;
    }
    if (ntok > 0) {
#pragma unroll
        for (int j = 0; j < PF; ++j) load_pos(prefetch_pos(j, ntok), j);
    }
    // the per-lane constants after the rows, so that their round trip to
    // memory overlaps the rows' instead of preceding it
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
    if (READOUT && p.Dskip) dskip = p.Dskip[dl];
    if (ntok > 0) {
        stage_store(0);
        dnext = delta_of(dq[0]);
    }
    __syncthreads();

    // the wave's slot on its SIMD (HW_ID bits 3:0): two waves sharing a SIMD
    // take turns at the higher priority
    const int alt = static_cast<int>(__builtin_amdgcn_s_getreg((3 << 11) | 4) & 1);
    for (int ti = 0; ti < ntiles; ++ti) {
        const int base = ti * kTile;
        const int cnt = ntok - base < kTile ? ntok - base : kTile;
        const bool more = ti + 1 < ntiles;
        const int ncnt = more ? (ntok - base - kTile < kTile ? ntok - base - kTile : kTile) : 0;
        if (more) stage_load(base + kTile, ncnt);
        const float *bc = lds_bc[ti & 1];

        const int full = cnt - cnt % PF;
        for (int k0 = 0; k0 < full; k0 += PF) {
            wave_priority_by_work_left(ntok - base - k0, alt);
            if constexpr (CK) checkpoint(base + k0);
#pragma unroll
            for (int j = 0; j < PF; ++j) token(base + k0 + j, bc + (k0 + j) * NBC, j);
        }
        if constexpr (CK)
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
    constexpr int NBC_MAX = (MODE & kModeOutMask) != kModeState ? 2 * kN : kN;
    __shared__ __align__(16) float lds[2 * kTile * NBC_MAX];

    // The set-up reads these arguments behind its branches (block validity,
    // layout, chunk role); loaded where they are first used, each would cost a
    // dependent round trip to memory before the first row is requested. An
    // empty asm statement that takes them as scalar operands makes the
    // compiler fetch them all at once, here.
    asm volatile("" ::"s"(p.nblocks), "s"(p.tiles), "s"(p.nchunks), "s"(p.chunk_len),
                 "s"(p.seqlen), "s"(p.cu_seqlens), "s"(p.D), "s"(p.split_c0), "s"(p.skip_c0),
                 "s"(p.skip_last), "s"(p.hin));
    asm volatile("" ::"s"(p.x), "s"(p.xs), "s"(p.xbs), "s"(p.dt), "s"(p.dts), "s"(p.dtbs),
                 "s"(p.Bm), "s"(p.Bs), "s"(p.Bbs), "s"(p.Cm), "s"(p.Cs), "s"(p.Cbs),
                 "s"(p.bc_vec));
    asm volatile("" ::"s"(p.A), "s"(p.Dskip), "s"(p.res), "s"(p.rs), "s"(p.rbs), "s"(p.s),
                 "s"(p.out), "s"(p.os), "s"(p.obs));
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
    if constexpr ((MODE & kModeOutMask) != kModeState) {
        if (p.split_c0 && c > 0) {
            scan_segment<REV, T, G, kModeState | (MODE & kModeBias), SP>(p, lds, bg, sq, sg, hin);
            return;
        }
    }
    scan_segment<REV, T, G, MODE, SP>(p, lds, bg, sq, sg, hin);
}

}  // namespace
}  // namespace r2l
