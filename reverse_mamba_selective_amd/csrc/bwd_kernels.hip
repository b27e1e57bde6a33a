// bwd_kernels.hip -- gfx950 kernels of the backward of a selective scan with
// readout: the gradients that training the R2L stream needs ("Bifocal
// Diffusion Language Models" trains the sidecar jointly, or only the sidecar
// and s in the plug-in variant).
//
// With dy = dyscale * dout and g the gradient with respect to the state,
// visiting the tokens in the opposite order of the forward scan:
//     g += dy * Cm[t]             dCm[t] += dy * h_t        (over channels)
//     dDelta = sum_n g_n (Bm[t,n] x + A_n abar_n h_prev_n)
//     dA += g Delta abar h_prev   dBm[t] += g Delta x       (over channels)
//     dx = dy Dskip + Delta sum_n g_n Bm[t,n] (+ dout if the residual is x)
//     g *= abar;  ddt = dDelta * sigmoid(dt) (softplus on)
// and at the end dh_in = g.
//
// Mapping onto CDNA4:
//  * Phase 1 (the forward segment kernel, state only) stored the state
//    entering every group of kCkptTokens visited positions. When the shape has
//    too few channels to fill the machine, phase 1 scans chunks of the
//    sequence from zero in parallel; by linearity the true state entering a
//    group is its chunk-local checkpoint plus exp(A * sum of Delta since the
//    chunk's start) times the state entering the chunk. Here one workgroup
//    owns (sequence, tile of kWG / G channels), G lanes per channel holding
//    kN / G states each, and walks the groups backwards: it recomputes the
//    group's states in registers from its checkpoint, then runs the adjoint
//    over the group in reverse.
//  * dBm and dCm are sums over channels of per-lane products: each 16-lane
//    row of a wave adds its 16 / G channels with DPP row rotations (VALU adds,
//    no lane permutes through LDS), the block's 16 rows add up in LDS, and the
//    block writes one partial row per token and tile; the sums over tiles, over sequences
//    (dA, dDskip) and over blocks (ds) are separate launches in a fixed order,
//    so the result is deterministic (no atomics).
//  * Bm / Cm rows are staged in LDS per tile of kTile tokens (double-buffered,
//    walking the tiles backwards) as in the forward kernel.
//  * softplus(dt) and its derivative are per channel: each of a channel's G
//    lanes takes them for K / G of the group's tokens and quad broadcasts
//    (DPP) hand Delta and sigmoid to the other lanes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scan_device.h"
#include "scan_geometry.h"
#include "scan_internal.h"

namespace r2l {
namespace {

using namespace dev;

// 1 / (1 + e^-v): the derivative of softplus. v_exp_f32 saturates to 0 or
// +inf, which gives 1 or 0.
__device__ __forceinline__ float sigmoid(float v) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-v * kLog2e));
}

// Lane l's value of each quad, to all four lanes of that quad (l is a constant
// once the caller's loop is unrolled).
template <int L>
__device__ __forceinline__ float quad_lane(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), L * 0x55, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_bcast(float v, int l) {
    switch (l) {
        case 0: return quad_lane<0>(v);
        case 1: return quad_lane<1>(v);
        case 2: return quad_lane<2>(v);
        default: return quad_lane<3>(v);
    }
}

// Sum of v[] over the channels of each 16-lane row of a wave: the lanes of
// a row that hold the same states (same lane % G) are the orbit of rotations
// by G, 2G, 4G, ... within the row, so adding DPP row rotations of G, 2G, ...
// leaves every lane with its row's totals of its own NS states (lanes of one
// orbit hold equal values). One VALU add per value and step; no selects, no
// LDS permutes.
template <int R, int NS>
__device__ __forceinline__ void add_row_ror(float (&v)[NS]) {
    // kept as a plain add: fused into the product that made v, the rotated
    // copy would be the fma's addend, which DPP cannot supply (mov + fma)
#pragma clang fp contract(off)
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int o = __builtin_amdgcn_mov_dpp(__float_as_int(v[i]), 0x120 + R, 0xF, 0xF, true);
        v[i] += __int_as_float(o);   // v + (v of the lane R places along the row)
    }
}

template <int G>
__device__ __forceinline__ void row_channel_sum(float (&v)[kN / G]) {
    constexpr int NS = kN / G;
    if constexpr (G <= 1) add_row_ror<1, NS>(v);
    if constexpr (G <= 2) add_row_ror<2, NS>(v);
    if constexpr (G <= 4) add_row_ror<4, NS>(v);
    add_row_ror<8, NS>(v);
}

// DS: also ds = sum over tokens and channels of dout * y. With the readout's
// partials dout * h and dDskip's dout * x taken before the gate's factor s
// (which is applied to their sums), ds is their contraction with what they
// multiply: the sum of Cm * dCm over the group's tokens, made where the block
// sums its channels, and of Dskip * dDskip over its channels; y itself is
// never recomputed, and s = 0 is no special case.
template <bool REV, typename T, int G, bool SP, bool DS>
__global__ __launch_bounds__(kWG) void bwd_kernel(const BwdParams p) {
    constexpr int NS = kN / G;
    constexpr int K = kCkptTokens;
    constexpr int NBC = 2 * kN;                  // staged floats per token (Bm, then Cm)
    constexpr int STAGE = stage_cols(NBC);
    constexpr int SW = STAGE * static_cast<int>(sizeof(T)) / 4;
    constexpr int WAVES = kWG / 64;
    static_assert(K * NBC == kWG, "one thread per (group token, column) in the block sum");
    __shared__ __align__(16) float lds_bc[2][kTile * NBC];
    constexpr int ROWS = WAVES * 4;              // 16-lane rows per block
    // row partials of a group, double-buffered: a group's block sum overlaps
    // the next group's adjoint (one barrier per group)
    __shared__ float red[2][ROWS][K][NBC];
    __shared__ float red_s[WAVES];
    using E = Elem<T>;
    using R = typename E::raw_t;

    const BlockGeom bg = block_geom(p.nblocks, p.tiles, 1, blockIdx.x);
    if (!bg.valid) return;
    const int64_t b = bg.b;
    const int64_t s0 = p.cu_seqlens ? p.cu_seqlens[b] : 0;
    const int64_t s1 = p.cu_seqlens ? p.cu_seqlens[b + 1] : 0;
    const BwdSeqGeom sq = bwd_seq_geom(p, b, s0, s1);
    const SegGeom sg = seg_geom(REV, 0, sq.len > 0 ? sq.len : 1, sq.len);
    const int ntok = sg.ntok;
    const LaneGeom lg = lane_geom(bg.tile, threadIdx.x, G, p.D);
    const uint32_t dl = lg.d;
    const int sub = lg.sub;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

    float An[NS], a2[NS], g[NS], dA[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        An[j] = p.A[dl * kN + sub * NS + j];
        a2[j] = An[j] * kLog2e;
        dA[j] = 0.0f;
        g[j] = (p.dh_out && lg.active) ? p.dh_out[(b * p.D + dl) * kN + sub * NS + j] : 0.0f;
    }
    const float dsk = p.Dskip ? p.Dskip[dl] : 0.0f;
    // lanes past the last channel shadow it; they must add nothing to any sum
    const float dys = lg.active ? p.dyscale : 0.0f;
    const float dxr = lg.active ? p.dxres : 0.0f;
    const float act = lg.active ? 1.0f : 0.0f;
    float dD = 0.0f, dsum = 0.0f;

    // per-token rows through raw buffer resources based at the sequence's first
    // row (scalar row offset, 32-bit lane offset), as in the forward kernel
    const uint32_t es = static_cast<uint32_t>(sizeof(T));
    const uint32_t doff = dl * es;
    const uint32_t xrb = static_cast<uint32_t>(p.xs) * es, drb = static_cast<uint32_t>(p.dts) * es;
    const uint32_t grb = static_cast<uint32_t>(p.gs) * es;
    const uint32_t dxrb = static_cast<uint32_t>(p.dxs) * es, ddrb = static_cast<uint32_t>(p.dds) * es;
    const auto rx = make_rsrc(static_cast<const T *>(p.x) + sq.xo, seq_span_bytes(sq.len, p.xs, p.D, es));
    const auto rd = make_rsrc(static_cast<const T *>(p.dt) + sq.dto, seq_span_bytes(sq.len, p.dts, p.D, es));
    const auto rg = make_rsrc(static_cast<const T *>(p.dout) + sq.go, seq_span_bytes(sq.len, p.gs, p.D, es));
    const auto rdx = make_rsrc(p.dx ? static_cast<T *>(p.dx) + sq.dxo : nullptr,
                               p.dx ? seq_span_bytes(sq.len, p.dxs, p.D, es) : 0);
    const auto rdd = make_rsrc(p.ddt ? static_cast<T *>(p.ddt) + sq.ddo : nullptr,
                               p.ddt ? seq_span_bytes(sq.len, p.dds, p.D, es) : 0);

    // Bm / Cm staging: threads 0..127 fetch Bm runs, 128..255 Cm runs
    const StageSlot ss = stage_slot(threadIdx.x, NBC);
    const bool stage_c = __builtin_amdgcn_readfirstlane(ss.mat) != 0;
    const auto rbc = stage_c
        ? make_rsrc(static_cast<const T *>(p.Cm) + sq.Co, seq_span_bytes(sq.len, p.Cs, kN, es))
        : make_rsrc(static_cast<const T *>(p.Bm) + sq.Bo, seq_span_bytes(sq.len, p.Bs, kN, es));
    const uint32_t bcrb = static_cast<uint32_t>(stage_c ? p.Cs : p.Bs) * es;
    const uint32_t bccol = static_cast<uint32_t>(ss.col0) * es;
    uint32_t stw[SW];
    auto stage_load = [&](int tbase, int tcnt) {   // tcnt >= 1
        const uint32_t row = static_cast<uint32_t>(seg_row(sg, tbase + stage_pos(ss.k, tcnt)));
        const uint32_t voff = row * bcrb + bccol;
        if (p.bc_vec)
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

    // per-token inputs of one group (positions past its end repeat its last
    // one) and the state entering it (its checkpoint; chunked phase 1: the
    // chunk-local checkpoint, the chunk's Delta sum up to it and the state
    // entering the chunk, combined when the group is consumed)
    // SP: each of a channel's G lanes loads dt only for the group's tokens j
    // with j % G == sub and computes softplus and its derivative for them; the
    // group's Delta and sigmoid rows then reach every lane of the channel by
    // quad broadcasts (DPP), instead of all G lanes computing all K tokens
    constexpr int OWN = SP ? K / G : 1;          // dt values per lane (SP)
    static_assert(!SP || K % G == 0, "a group splits evenly over the channel's lanes");
    R nx[K], nd[SP ? OWN : K], ng[K];
    float nck[NS], nH[NS], nS = 0.0f;
    const bool chunked = p.Hc != nullptr;
#pragma unroll
    for (int n = 0; n < NS; ++n) nH[n] = 0.0f;
    auto load_group = [&](int gpos, int gcnt) {
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const uint32_t row = static_cast<uint32_t>(seg_row(sg, gpos + (j < gcnt ? j : gcnt - 1)));
            nx[j] = E::bload(rx, doff, row * xrb);
            if constexpr (!SP) nd[j] = E::bload(rd, doff, row * drb);
            ng[j] = E::bload(rg, doff, row * grb);
        }
        if constexpr (SP) {
#pragma unroll
            for (int k = 0; k < OWN; ++k) {   // this lane's tokens sub, sub + G, ...
                const int jo = sub + G * k;
                const uint32_t row = static_cast<uint32_t>(seg_row(sg, gpos + (jo < gcnt ? jo : gcnt - 1)));
                nd[k] = E::bload(rd, doff + row * drb, 0);
            }
        }
        const int64_t ckr = ckpt_row(b, sq.s0p, gpos);
        static_assert(NS == 4, "one checkpoint quad per lane");
        const float *cp = p.ckpt + ckpt_quad(ckr, p.D, dl, sub);
#pragma unroll
        for (int n = 0; n < NS; ++n) nck[n] = cp[n];
        if (chunked) {
            const int64_t c = gpos / p.chunk_len;
            const float *hp = p.Hc + ((b * p.nchunks + c) * p.D + dl) * kN + sub * NS;
#pragma unroll
            for (int n = 0; n < NS; ++n) nH[n] = hp[n];
            nS = p.ckpt_s[ckr * p.D + dl];
        }
    };

    // tiles (and the groups inside them) from the last visited to the first
    const int ntiles = (ntok + kTile - 1) / kTile;
    // the wave's slot on its SIMD (HW_ID bits 3:0), for the priority turns below
    const int alt = static_cast<int>(__builtin_amdgcn_s_getreg((3 << 11) | 4) & 1);
    if (ntok > 0) {
        const int lb = (ntiles - 1) * kTile;
        stage_load(lb, ntok - lb);
        const int lg0 = (ntok - 1) / K * K;   // the last group
        load_group(lg0, ntok - lg0);
        stage_store((ntiles - 1) & 1);
    }
    __syncthreads();
    for (int ti = ntiles - 1; ti >= 0; --ti) {
        const int tbase = ti * kTile;
        const int tcnt = ntok - tbase < kTile ? ntok - tbase : kTile;
        const bool more = ti > 0;
        if (more) stage_load(tbase - kTile, kTile);   // every tile but the last is full
        const float *bc = lds_bc[ti & 1];

        for (int gi = (tcnt - 1) / K; gi >= 0; --gi) {
            const int gpos = tbase + gi * K;
            {   // groups left after this one: a wave with more left issues first, so
                // the waves sharing a SIMD stay abreast (as in the segment scan);
                // before the last four, the two waves of a SIMD take turns at the
                // higher of two levels (by the parity of their slot on the SIMD),
                // which keeps long sequences abreast too
                const int q = gpos / K;
                const int pr = q >= 4 ? 2 + ((alt + q) & 1) : q;
                if (pr >= 3) __builtin_amdgcn_s_setprio(3);
                else if (pr == 2) __builtin_amdgcn_s_setprio(2);
                else if (pr == 1) __builtin_amdgcn_s_setprio(1);
                else __builtin_amdgcn_s_setprio(0);
            }
            const int gcnt = ntok - gpos < K ? ntok - gpos : K;
            // this group's per-token inputs were requested during the previous
            // group; request the next group's (gpos - K) now
            R xr[K], dr[SP ? OWN : K], gr[K];
            float hck[NS];
#pragma unroll
            for (int j = 0; j < K; ++j) {
                xr[j] = nx[j];
                gr[j] = ng[j];
            }
#pragma unroll
            for (int j = 0; j < (SP ? OWN : K); ++j) dr[j] = nd[j];
            if (chunked) {   // the chunk's entry state decayed over the chunk so far
#pragma unroll
                for (int n = 0; n < NS; ++n)
                    hck[n] = fmaf(__builtin_amdgcn_exp2f(a2[n] * nS), nH[n], nck[n]);
            } else {
#pragma unroll
                for (int n = 0; n < NS; ++n) hck[n] = nck[n];
            }
            if (gpos > 0) load_group(gpos - K, K);
            float (*rd_)[K][NBC] = red[gi & 1];

            // the group's states and decays, recomputed forward from the checkpoint
            float hs[K][NS], ab[K][NS], delta[K], sgm[SP ? K : 1];
            if constexpr (SP) {
                float dlo[OWN], slo[OWN];
#pragma unroll
                for (int k = 0; k < OWN; ++k) {
                    const float dv = E::widen(dr[k]);
                    dlo[k] = softplus(dv);
                    slo[k] = sigmoid(dv);
                }
#pragma unroll
                for (int j = 0; j < K; ++j) {   // from lane j % G of the channel's quad
                    delta[j] = quad_bcast(dlo[j / G], j % G);
                    sgm[j] = quad_bcast(slo[j / G], j % G);
                }
            } else {
#pragma unroll
                for (int j = 0; j < K; ++j) delta[j] = E::widen(dr[j]);
            }
#pragma unroll
            for (int j = 0; j < K; ++j) {
                const float dx_ = delta[j] * E::widen(xr[j]);
                const float *brow = bc + (gi * K + j) * NBC + sub * NS;
#pragma unroll
                for (int n = 0; n < NS; ++n) {
                    const float hp = j > 0 ? hs[j - 1][n] : hck[n];
                    ab[j][n] = __builtin_amdgcn_exp2f(delta[j] * a2[n]);
                    hs[j][n] = fmaf(ab[j][n], hp, brow[n] * dx_);
                }
            }

            // the adjoint over the group, last visited position first
            R odx[K], oddt[K];
            auto ldrow = [&](const int j, float4 &rb, float4 &rc) {
                const float *row = bc + (gi * K + j) * NBC + sub * NS;   // Bm slice; Cm at + kN
                rb = *reinterpret_cast<const float4 *>(row);
                rc = *reinterpret_cast<const float4 *>(row + kN);
            };
            auto adjoint = [&](const int j, const float4 rb, const float4 rc) {
                static_assert(NS == 4, "one Bm and one Cm quad per lane");
                const float Bn[NS] = {rb.x, rb.y, rb.z, rb.w}, Cn[NS] = {rc.x, rc.y, rc.z, rc.w};
                const float xv = E::widen(xr[j]);
                const float gv = E::widen(gr[j]);
                const float dy = dys * gv;
                const float wy = DS ? act * gv : dy;   // weight of the dCm and dDskip partials
                dD = fmaf(wy, xv, dD);
                const float dlx = delta[j] * xv;
                float pb[NS], pc[NS];
                // dDelta = sum_n g_n (B_n x + A_n abar_n h_prev_n)
                //        = x * sum_n g_n B_n + sum_n (g_n abar_n h_prev_n) A_n
                float dd = 0.0f, dxs = 0.0f;
#pragma unroll
                for (int n = 0; n < NS; ++n) {
                    g[n] = fmaf(dy, Cn[n], g[n]);
                    pc[n] = wy * hs[j][n];
                    const float hp = j > 0 ? hs[j - 1][n] : hck[n];
                    dxs = fmaf(g[n], Bn[n], dxs);
                    pb[n] = g[n] * dlx;
                    g[n] *= ab[j][n];                    // carried to the earlier position
                    const float gah = g[n] * hp;         // g abar h_prev
                    dA[n] = fmaf(gah, delta[j], dA[n]);
                    dd = fmaf(gah, An[n], dd);
                }
                const float ddelta = group_sum<G>(fmaf(xv, dxs, dd));
                const float dxv = fmaf(delta[j], group_sum<G>(dxs), fmaf(dy, dsk, dxr * gv));
                float ddtv = ddelta;
                if constexpr (SP) ddtv *= sgm[j];
                odx[j] = E::pack(dxv);   // stored after the group: no branch per token
                oddt[j] = E::pack(ddtv);
                row_channel_sum<G>(pb);
                row_channel_sum<G>(pc);
                float *rw = rd_[wave * 4 + (lane >> 4)][j];
#pragma unroll
                for (int n = 0; n < NS; ++n) {   // equal values from every lane of an orbit
                    rw[sub * NS + n] = pb[n];
                    rw[kN + sub * NS + n] = pc[n];
                }
            };
            if (gcnt == K && DS) {
                // every group but a sequence's last: no branch per token; the
                // slices of the token before are requested before this token's
                // arithmetic, so their LDS round trip overlaps it (the compiler
                // otherwise waits on each token's read 4 instructions after
                // issuing it): the denoising hook's backward from saved
                // checkpoints 76.5 -> 73.3 us. Without ds the same order makes
                // the compiler spill 173 scalar registers into vector lanes
                // (prefill backward +16%), so that instance keeps the plain one.
                float4 rb[2], rc[2];   // token j's slices in [j & 1]
                ldrow(K - 1, rb[(K - 1) & 1], rc[(K - 1) & 1]);
#pragma unroll
                for (int j = K - 1; j >= 0; --j) {
                    if (j > 0) ldrow(j - 1, rb[(j - 1) & 1], rc[(j - 1) & 1]);
                    adjoint(j, rb[j & 1], rc[j & 1]);
                }
            } else if (gcnt == K) {
#pragma unroll
                for (int j = K - 1; j >= 0; --j) {
                    float4 rb, rc;
                    ldrow(j, rb, rc);
                    adjoint(j, rb, rc);
                }
            } else {
#pragma unroll
                for (int j = K - 1; j >= 0; --j)
                    if (j < gcnt) {
                        float4 rb, rc;
                        ldrow(j, rb, rc);
                        adjoint(j, rb, rc);
                    }
            }
            // the group's dx and ddt rows (lanes past the last channel store nothing)
            if (lg.active) {
#pragma unroll
                for (int j = 0; j < K; ++j) {
                    if (j >= gcnt) break;
                    const uint32_t orow = static_cast<uint32_t>(seg_row(sg, gpos + j));
                    if (p.dx) E::bstore(odx[j], rdx, doff, orow * dxrb);
                    if (p.ddt) E::bstore(oddt[j], rdd, doff, orow * ddrb);
                }
            }
            __syncthreads();
            {   // the block's sums over its channels: one thread per (token, column)
                const int j = threadIdx.x / NBC, col = threadIdx.x % NBC;
                float *dst = col < kN ? p.partB : p.partC;
                if (j < gcnt && (dst || (DS && col >= kN))) {
                    float v = 0.0f;
#pragma unroll
                    for (int w = 0; w < ROWS; ++w) v += rd_[w][j][col];
                    if constexpr (DS) {
                        if (col >= kN) {   // Cm * dCm, then dCm takes the factor s
                            dsum = fmaf(v, bc[(gi * K + j) * NBC + col], dsum);
                            v *= p.dyscale;
                        }
                    }
                    const int64_t t = sq.s0p + seg_row(sg, gpos + j);
                    if (dst) dst[(bg.tile * p.tokens + t) * kN + (col % kN)] = v;
                }
            }
            // no barrier here: the next group writes the other half of red, and
            // the one after it this half only past the next group's barrier
        }
        if (more) stage_store((ti - 1) & 1);
        __syncthreads();
    }

    if (lg.active) {
        const int64_t st = (b * p.D + dl) * kN + sub * NS;
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            if (p.dh_in) p.dh_in[st + n] = g[n];
            if (p.partA) p.partA[st + n] = dA[n];
        }
        if (DS && sub == 0) dsum = fmaf(dsk, dD, dsum);   // Dskip * dDskip
        if (p.partD && sub == 0) p.partD[b * p.D + dl] = DS ? p.dyscale * dD : dD;
    }
    if (p.partS) {   // uniform: every thread of the block reaches the barrier
        float v = dsum;
#pragma unroll
        for (int bit = 1; bit < 64; bit <<= 1) v += __shfl_xor(v, bit);
        if (lane == 0) red_s[wave] = v;
        __syncthreads();
        if (threadIdx.x == 0) {
            float t = 0.0f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) t += red_s[w];
            p.partS[b * p.tiles + bg.tile] = t;
        }
    }
}

constexpr int kSumThreads = 256;
constexpr int64_t kNarrowSum = 4096;

// A whole block per output: few outputs, each with at least a block's worth
// of partials (ds over every block of the call). Fewer partials go one per
// thread (dDskip of the denoising hook: 2048 outputs of 64 partials).
__host__ __device__ inline bool narrow_sum(const SumParams &p) {
    return p.n < kNarrowSum && p.P >= kSumThreads;
}

// The ordered sums of one backward call in one launch: segment k owns blocks
// [first[k], first[k + 1]). Narrow segments (narrow_sum) give each output a
// whole block (threads split the partials in order, then a fixed tree in
// LDS); the others give each thread one output, its partials added in order.
// A segment of few outputs (at most one block per CU) is latency-bound: its
// threads have sixteen loads in flight before they add them; a large one
// (the prefill's dBm, dCm: 0.5 M outputs) streams HBM and keeps four, which
// measured faster there.
constexpr int64_t kFewSumOutputs = 65536;
__global__ __launch_bounds__(kSumThreads) void sum_kernel(const SumBatch sb) {
    __shared__ float part[kSumThreads];
    int k = 0;
    while (k + 1 < sb.count && blockIdx.x >= sb.first[k + 1]) ++k;
    const SumParams &p = sb.seg[k];
    const int64_t blk = static_cast<int64_t>(blockIdx.x) - sb.first[k];
    constexpr int kInFlight = 16;
    if (narrow_sum(p)) {
        float acc = 0.0f;
        int64_t q = threadIdx.x;
        for (; q + (kInFlight - 1) * kSumThreads < p.P; q += kInFlight * kSumThreads) {
            float v[kInFlight];
#pragma unroll
            for (int j = 0; j < kInFlight; ++j) v[j] = p.src[(q + j * kSumThreads) * p.pstride + blk];
#pragma unroll
            for (int j = 0; j < kInFlight; ++j) acc += v[j];
        }
        for (; q < p.P; q += kSumThreads) acc += p.src[q * p.pstride + blk];
        part[threadIdx.x] = acc;
        __syncthreads();
#pragma unroll
        for (int w = kSumThreads / 2; w > 0; w >>= 1) {
            if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
            __syncthreads();
        }
        if (threadIdx.x == 0) p.dst[blk] = part[0];
        return;
    }
    const int64_t i = blk * kSumThreads + threadIdx.x;
    if (i >= p.n) return;
    float acc = 0.0f;
    int64_t q = 0;
    if (p.n <= kFewSumOutputs) {
        for (; q + kInFlight <= p.P; q += kInFlight) {
            float v[kInFlight];
#pragma unroll
            for (int j = 0; j < kInFlight; ++j) v[j] = p.src[(q + j) * p.pstride + i];
#pragma unroll
            for (int j = 0; j < kInFlight; ++j) acc += v[j];
        }
    }
    for (; q + 4 <= p.P; q += 4) {
        const float v0 = p.src[q * p.pstride + i], v1 = p.src[(q + 1) * p.pstride + i];
        const float v2 = p.src[(q + 2) * p.pstride + i], v3 = p.src[(q + 3) * p.pstride + i];
        acc = (((acc + v0) + v1) + v2) + v3;
    }
    for (; q < p.P; ++q) acc += p.src[q * p.pstride + i];
    p.dst[i] = acc;
}

// 4 lanes per channel (2 would need 341 VGPRs: one wave per SIMD)
template <bool REV, typename T, bool SP>
hipError_t launch_bwd_g(int G, const BwdParams &p, hipStream_t stream) {
    if (G != 4) return hipErrorInvalidValue;
    const int64_t grid = padded_grid(p.nblocks);
    if (p.want_ds)
        hipLaunchKernelGGL((bwd_kernel<REV, T, 4, SP, true>), dim3(grid), dim3(kWG), 0, stream, p);
    else
        hipLaunchKernelGGL((bwd_kernel<REV, T, 4, SP, false>), dim3(grid), dim3(kWG), 0, stream, p);
    return hipGetLastError();
}

template <bool REV, typename T>
hipError_t launch_bwd_s(int G, const BwdParams &p, hipStream_t stream) {
    return p.softplus ? launch_bwd_g<REV, T, true>(G, p, stream)
                      : launch_bwd_g<REV, T, false>(G, p, stream);
}

}  // namespace

hipError_t launch_backward(bool reverse, int dtype, int G, const BwdParams &p, hipStream_t stream) {
    if (reverse)
        return dtype == 1 ? launch_bwd_s<true, uint16_t>(G, p, stream)
                          : launch_bwd_s<true, float>(G, p, stream);
    return dtype == 1 ? launch_bwd_s<false, uint16_t>(G, p, stream)
                      : launch_bwd_s<false, float>(G, p, stream);
}

int64_t sum_blocks(const SumParams &p) {
    if (p.n <= 0) return 0;
    return narrow_sum(p) ? p.n : (p.n + kSumThreads - 1) / kSumThreads;
}

hipError_t launch_sums(const SumBatch &in, hipStream_t stream) {
    SumBatch sb = in;
    int64_t total = 0;
    for (int k = 0; k < sb.count; ++k) {
        sb.first[k] = total;
        total += sum_blocks(sb.seg[k]);
    }
    sb.first[sb.count] = total;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(sum_kernel, dim3(static_cast<uint32_t>(total)), dim3(kSumThreads), 0, stream, sb);
    return hipGetLastError();
}

}  // namespace r2l
