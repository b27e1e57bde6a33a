// bounds_check.cpp -- host-side replay of every memory access that the
// launches of one entry-point call would make, using the kernels' own index
// math (scan_geometry.h) and the same launch list (scan_plan.h). Nothing here
// touches a device: pointers are only compared as numbers.
//
// An access is in bounds when it lies inside the buffer its base pointer
// points into (a zero-size buffer admits no access). Per-token rows must also
// be rows of the segment's own sequence, and buffer-resource offsets must fit
// the resource (the hardware checks only the lane offset).
#include "bounds_check.h"

#include <cstdarg>
#include <cstdio>
#include <vector>

#include "scan_geometry.h"

namespace r2l {
namespace {

struct Region {
    const char *name;
    uintptr_t lo, hi;
};

class Checker {
  public:
    Checker(std::vector<Region> regions, r2l_access_report *rep) : regions_(std::move(regions)), rep_(rep) {}

    // The region that holds pointer p (nullptr if none).
    const Region *region_of(const void *p) const {
        const uintptr_t v = reinterpret_cast<uintptr_t>(p);
        const Region *best = nullptr;
        for (const Region &r : regions_)
            if (r.lo <= v && v < r.hi && (!best || r.hi - r.lo < best->hi - best->lo)) best = &r;
        return best;
    }

    bool ok() const { return !failed_; }

    // [addr, addr + bytes) inside the region of `base`.
    void access(const char *what, const Region *reg, uintptr_t addr, uint64_t bytes) {
        ++rep_->accesses;
        if (failed_) return;
        if (!reg) return fail("%s: base pointer is in no argument buffer (addr 0x%llx)", what,
                              (unsigned long long)addr);
        if (addr < reg->lo || addr + bytes > reg->hi)
            fail("%s: byte 0x%llx..+%llu outside %s [0x%llx, 0x%llx)", what,
                 (unsigned long long)addr, (unsigned long long)bytes, reg->name,
                 (unsigned long long)reg->lo, (unsigned long long)reg->hi);
    }

    // Words of the tracked buffers (the workspace; a saving forward's
    // checkpoints) written so far by the call's launches, in order: every read
    // of them must find its words written by an earlier launch.
    void set_workspace(const void *base, uint64_t bytes) { track(base, bytes); }
    void track(const void *base, uint64_t bytes) {
        if (base && bytes >= 4)
            tracked_.push_back({reinterpret_cast<uintptr_t>(base), std::vector<bool>(bytes / 4, false)});
    }
    void wrote(uintptr_t addr, uint64_t bytes) {
        Tracked *t = tracked_at(addr);
        if (!t) return;
        for (uint64_t w = (addr - t->lo) / 4; w < (addr - t->lo + bytes) / 4; ++w)
            if (w < t->written.size()) t->written[w] = true;
    }
    void read_written(const char *what, uintptr_t addr, uint64_t bytes) {
        Tracked *t = tracked_at(addr);
        if (!t || failed_) return;
        for (uint64_t w = (addr - t->lo) / 4; w < (addr - t->lo + bytes) / 4; ++w)
            if (w >= t->written.size() || !t->written[w])
                return fail("%s: reads byte 0x%llx that no earlier launch wrote", what,
                            (unsigned long long)(t->lo + 4 * w));
    }

    // The launch's grid covers its work exactly once: its valid blocks map one
    // to one onto the (sequence, chunk, tile) triples of `nblocks` =
    // sequences x chunks x tiles.
    void cover_blocks(const char *what, int64_t nblocks, int32_t tiles, int32_t nchunks) {
        if (failed_ || nblocks <= 0) return;
        std::vector<bool> seen(static_cast<size_t>(nblocks), false);
        for (int64_t bid = 0; bid < padded_grid(nblocks); ++bid) {
            const BlockGeom bg = block_geom(nblocks, tiles, nchunks, bid);
            if (!bg.valid) continue;
            const int64_t at = (bg.b * nchunks + bg.c) * tiles + bg.tile;
            if (bg.tile < 0 || bg.tile >= tiles || bg.c < 0 || bg.c >= nchunks || at < 0 ||
                at >= nblocks || seen[static_cast<size_t>(at)])
                return fail("%s: block %lld takes sequence %lld, chunk %d, tile %d: outside the "
                            "grid's work or taken twice", what, (long long)bid, (long long)bg.b,
                            bg.c, bg.tile);
            seen[static_cast<size_t>(at)] = true;
        }
        for (int64_t i = 0; i < nblocks; ++i)
            if (!seen[static_cast<size_t>(i)])
                return fail("%s: no block takes sequence %lld, chunk %lld, tile %lld", what,
                            (long long)(i / (int64_t(tiles) * nchunks)), (long long)((i / tiles) % nchunks),
                            (long long)(i % tiles));
    }

    void fail(const char *fmt, ...) __attribute__((format(printf, 2, 3))) {
        if (failed_) return;
        failed_ = true;
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(rep_->message, sizeof(rep_->message), fmt, ap);
        va_end(ap);
    }

  private:
    struct Tracked {
        uintptr_t lo;
        std::vector<bool> written;
    };
    Tracked *tracked_at(uintptr_t a) {
        for (Tracked &t : tracked_)
            if (a >= t.lo && a < t.lo + 4 * t.written.size()) return &t;
        return nullptr;
    }

    std::vector<Region> regions_;
    r2l_access_report *rep_;
    bool failed_ = false;
    std::vector<Tracked> tracked_;
};

uintptr_t U(const void *p) { return reinterpret_cast<uintptr_t>(p); }

void check_segment(Checker &ck, const Launch &l, const int32_t *cu_host) {
    const SegParams &p = l.seg;
    const bool launch_readout = (l.mode & kModeOutMask) != kModeState;
    const bool to_ws = (l.mode & kModeOutMask) == kModeWs;
    const int G = l.G, NS = kN / G;
    const int64_t es = l.dtype == R2L_DTYPE_BF16 ? 2 : 4;
    const Region *rA = ck.region_of(p.A), *rDs = p.Dskip ? ck.region_of(p.Dskip) : nullptr;
    const Region *rHin = p.hin ? ck.region_of(p.hin) : nullptr;
    const Region *rHfin = p.hfin ? ck.region_of(p.hfin) : nullptr;
    const Region *rSd = p.sdelta ? ck.region_of(p.sdelta) : nullptr;
    const Region *rX = ck.region_of(p.x), *rD = ck.region_of(p.dt), *rB = ck.region_of(p.Bm);
    const Region *rC = launch_readout ? ck.region_of(p.Cm) : nullptr;
    const bool reads_res = (l.mode & kModeOutMask) == kModeRes || (l.mode & kModeOutMask) == kModeGate;
    const Region *rR = reads_res ? ck.region_of(p.res) : nullptr;
    const Region *rBias = (l.mode & kModeBias) && p.dt_bias ? ck.region_of(p.dt_bias) : nullptr;
    const Region *rO = launch_readout && !to_ws ? ck.region_of(p.out) : nullptr;
    // kModeLds: the bidirectional rows live in LDS (row < kBidirLdsTokens), not the workspace
    const bool lrows = (l.mode & kModeLds) != 0;
    const Region *rW = to_ws && !lrows ? ck.region_of(p.yws) : nullptr;
    const Region *rAdd = (l.mode & kModeAdd) && !lrows ? ck.region_of(p.yadd) : nullptr;

    ck.cover_blocks("segment launch", p.nblocks, p.tiles, p.nchunks);
    for (int64_t bid = 0; bid < padded_grid(p.nblocks) && ck.ok(); ++bid) {
        const BlockGeom bg = block_geom(p.nblocks, p.tiles, p.nchunks, bid);
        if (!bg.valid) continue;
        const int64_t s0 = p.cu_seqlens ? cu_host[bg.b] : 0;
        const int64_t s1 = p.cu_seqlens ? cu_host[bg.b + 1] : 0;
        const SeqGeom sq = seq_geom(p, bg.b, s0, s1);
        const SegGeom sg = seg_geom(l.reverse, bg.c, p.chunk_len, sq.len);
        if (p.cu_seqlens) ck.access("cu_seqlens", ck.region_of(p.cu_seqlens),
                                    U(p.cu_seqlens) + bg.b * 4, 8);
        if (!segment_runs(p, sg, bg.c)) continue;
        // the body this block runs: a split chunk pass scans chunks > 0 state only
        const bool readout = launch_readout && !(p.split_c0 && bg.c > 0);
        const int mode = readout ? l.mode : kModeState;
        // checkpoints: kModeCkpt launches, except the state-only chunks of a split pass
        const bool ckpt_on = (l.mode & kModeCkpt) && !(p.split_c0 && bg.c > 0);
        const int NBC = readout ? 2 * kN : kN, STAGE = stage_cols(NBC);
        const float *hin = segment_hin(p, bg.b, bg.c);

        // per-lane loads and stores outside the token loop
        uint32_t dmin = UINT32_MAX, dmax = 0;
        for (int lane = 0; lane < kWG; ++lane) {
            const LaneGeom lg = lane_geom(bg.tile, lane, G, p.D);
            dmin = lg.d < dmin ? lg.d : dmin;
            dmax = lg.d > dmax ? lg.d : dmax;
            const int64_t st = static_cast<int64_t>(lg.d) * kN + lg.sub * NS;
            ck.access("A", rA, U(p.A) + st * 4, NS * 4);
            if (hin) {
                ck.access("h_in", rHin, U(hin) + st * 4, NS * 4);
                ck.read_written("h_in", U(hin) + st * 4, NS * 4);
            }
            if (readout && p.Dskip) ck.access("Dskip", rDs, U(p.Dskip) + lg.d * 4, 4);
            if (rBias) ck.access("dt_bias", rBias, U(p.dt_bias) + lg.d * 4, 4);
            if (p.hfin && lg.active) {
                const uintptr_t a = U(p.hfin) + (bg.b * p.hfin_b + bg.c * p.hfin_c + st) * 4;
                ck.access("h_final", rHfin, a, NS * 4);
                ck.wrote(a, NS * 4);
            }
            if (!readout && p.sdelta && lg.active && lg.sub == 0) {
                const uintptr_t a = U(p.sdelta) + (bg.b * p.sd_b + bg.c * p.sd_c + lg.d) * 4;
                ck.access("delta_sum", rSd, a, 4);
                ck.wrote(a, 4);
            }
        }
        if (!ck.ok()) return;

        // buffer-resource rows: row must be one of the sequence's rows; the
        // scalar offset row * row_bytes must fit 32 bits; the lane offset
        // must lie inside the resource; the address inside the tensor.
        auto row_access = [&](const char *what, const Region *reg, const void *base, int64_t elem_off,
                              int64_t row_elems, int k) {
            const int row = seg_row(sg, k);
            if (row < 0 || row >= sq.len)
                return ck.fail("%s: row %d outside the sequence of %lld rows (block %lld)", what, row,
                               (long long)sq.len, (long long)bid);
            const uint64_t soff = static_cast<uint64_t>(row) * static_cast<uint64_t>(row_elems * es);
            if (soff > UINT32_MAX) return ck.fail("%s: scalar offset %llu above 32 bits", what,
                                                  (unsigned long long)soff);
            const uint32_t nrec = seq_span_bytes(sq.len, row_elems, p.D, es);
            if (static_cast<uint64_t>(dmax) * es + es > nrec)
                return ck.fail("%s: lane offset beyond the buffer resource", what);
            const uintptr_t b0 = U(base) + elem_off * es + soff;
            ck.access(what, reg, b0 + static_cast<uint64_t>(dmin) * es, es);
            ck.access(what, reg, b0 + static_cast<uint64_t>(dmax) * es, es);
        };
        // fp32 [packed token, D] workspace rows (bidirectional scan): the
        // resource starts at the sequence's first packed row
        auto ws_row = [&](const char *what, const Region *reg, const float *base, int k, bool write) {
            const int row = seg_row(sg, k);
            if (lrows) {   // ylds[row * kWG + thread]
                if (row < 0 || row >= kBidirLdsTokens || row >= sq.len)
                    return ck.fail("%s: LDS row %d outside 0..%d (block %lld)", what, row,
                                   kBidirLdsTokens - 1, (long long)bid);
                return;
            }
            if (row < 0 || row >= sq.len)
                return ck.fail("%s: row %d outside the sequence of %lld rows (block %lld)", what, row,
                               (long long)sq.len, (long long)bid);
            const uint64_t soff = static_cast<uint64_t>(row) * static_cast<uint64_t>(p.D * 4);
            if (soff > UINT32_MAX) return ck.fail("%s: scalar offset %llu above 32 bits", what,
                                                  (unsigned long long)soff);
            if (static_cast<uint64_t>(dmax) * 4 + 4 > seq_span_bytes(sq.len, p.D, p.D, 4))
                return ck.fail("%s: lane offset beyond the buffer resource", what);
            const uintptr_t b0 = U(base) + static_cast<uint64_t>(sq.s0p * p.D) * 4 + soff;
            for (uint32_t d : {dmin, dmax}) {
                ck.access(what, reg, b0 + static_cast<uint64_t>(d) * 4, 4);
                if (write)
                    ck.wrote(b0 + static_cast<uint64_t>(d) * 4, 4);
                else
                    ck.read_written(what, b0 + static_cast<uint64_t>(d) * 4, 4);
            }
        };
        auto load_pos = [&](int k) {
            row_access("x", rX, p.x, sq.xo, p.xs, k);
            row_access("dt", rD, p.dt, sq.dto, p.dts, k);
            const int64_t rw = seg_row(sg, k);
            ck.read_written("x", U(p.x) + (sq.xo + rw * p.xs + dmin) * es, es);
            ck.read_written("dt", U(p.dt) + (sq.dto + rw * p.dts + dmin) * es, es);
            if ((mode & kModeOutMask) == kModeRes || (mode & kModeOutMask) == kModeGate) {
                row_access("res", rR, p.res, sq.ro, p.rs, k);
                ck.read_written("res", U(p.res) + (sq.ro + static_cast<int64_t>(seg_row(sg, k)) * p.rs) * es
                                       + static_cast<uint64_t>(dmin) * es, es);
            }
            if (mode & kModeAdd) ws_row("reverse readout rows", rAdd, p.yadd, k, false);
        };
        const int ntok = sg.ntok;
        // checkpoints: the state entering every group of kCkptTokens
        // positions, written by the active lanes
        if (p.ckpt && ckpt_on)
            for (int pos = 0; pos < ntok && ck.ok(); pos += kCkptTokens)
                for (int lane = 0; lane < kWG; ++lane) {
                    const LaneGeom lg = lane_geom(bg.tile, lane, G, p.D);
                    if (!lg.active) continue;
                    const int64_t row = ckpt_row(bg.b, sq.s0p, static_cast<int64_t>(bg.c) * p.chunk_len + pos);
                    for (int q = 0; q < NS / 4; ++q) {
                        const uintptr_t a = U(p.ckpt) + ckpt_quad(row, p.D, lg.d, lg.sub * (NS / 4) + q) * 4;
                        ck.access("checkpoint", ck.region_of(p.ckpt), a, 16);
                        ck.wrote(a, 16);
                    }
                    if (p.ckpt_s && !readout && lg.sub == 0) {
                        const uintptr_t as = U(p.ckpt_s) + (row * p.D + lg.d) * 4;
                        ck.access("checkpoint delta sum", ck.region_of(p.ckpt_s), as, 4);
                        ck.wrote(as, 4);
                    }
                }
        if (ntok > 0)
            for (int j = 0; j < kPrefetch; ++j) load_pos(prefetch_pos(j, ntok));
        for (int k = 0; k < ntok && ck.ok(); ++k) {
            load_pos(prefetch_pos(k + kPrefetch, ntok));
            if (readout && to_ws)
                ws_row("readout rows", rW, p.yws, k, true);
            else if (readout) {
                row_access("out", rO, p.out, sq.oo, p.os, k);
                const uint64_t o0 = U(p.out) + (sq.oo + static_cast<int64_t>(seg_row(sg, k)) * p.os) * es;
                ck.wrote(o0 + static_cast<uint64_t>(dmin) * es, (dmax - dmin + 1) * es);
            }
        }

        // Bm/Cm staging, tile by tile: per thread one run of STAGE elements
        // at lane offset row * row_bytes + col0 * es of its matrix's resource
        const int al = stage_align(NBC, static_cast<int>(es));
        for (int base = 0; base < ntok && ck.ok(); base += kTile) {
            const int cnt = ntok - base < kTile ? ntok - base : kTile;
            for (int lane = 0; lane < kWG && ck.ok(); ++lane) {
                const StageSlot ss = stage_slot(lane, NBC);
                if (ss.mat > (readout ? 1 : 0) || ss.k >= kTile || ss.col0 + STAGE > kN)
                    return ck.fail("staging slot of thread %d outside the tile", lane);
                if (ss.mat != stage_slot(lane & ~63, NBC).mat)
                    return ck.fail("staging matrix not uniform in the wave of thread %d", lane);
                const int64_t row = seg_row(sg, base + stage_pos(ss.k, cnt));
                if (row < 0 || row >= sq.len)
                    return ck.fail("staging row %lld outside the sequence", (long long)row);
                const bool isC = ss.mat != 0;
                const int64_t st = isC ? p.Cs : p.Bs;
                const uint64_t voff = static_cast<uint64_t>(row * st + ss.col0) * es;
                if (voff + STAGE * es > seq_span_bytes(sq.len, st, kN, es))
                    return ck.fail("staging run beyond the buffer resource (block %lld)", (long long)bid);
                const uintptr_t addr = U(isC ? p.Cm : p.Bm) + (isC ? sq.Co : sq.Bo) * es + voff;
                if (p.bc_vec && addr % al)
                    return ck.fail("staging vector load at 0x%llx not %d-byte aligned",
                                   (unsigned long long)addr, al);
                ck.access(isC ? "Cm" : "Bm", isC ? rC : rB, addr, STAGE * es);
            }
        }
    }
}

void check_carry(Checker &ck, const Launch &l, const int32_t *cu_host) {
    const CarryParams &p = l.carry;
    const Region *rA = ck.region_of(p.A), *rQ = ck.region_of(p.Q), *rS = ck.region_of(p.S);
    const Region *rH = p.Hc ? ck.region_of(p.Hc) : nullptr, *rin = p.hin ? ck.region_of(p.hin) : nullptr;
    const Region *rout = p.hout ? ck.region_of(p.hout) : nullptr;
    for (int64_t i = 0; i < p.batch * carry_tiles(p.D) * kCarryThreads && ck.ok(); ++i) {
        const int64_t bx = i / (carry_tiles(p.D) * kCarryThreads);
        const int64_t rem = i % (carry_tiles(p.D) * kCarryThreads);
        const CarryGeom g = carry_geom(p.D, bx, rem / kCarryThreads, static_cast<int>(rem % kCarryThreads));
        if (!g.valid) continue;
        const int64_t len = p.cu_seqlens ? static_cast<int64_t>(cu_host[g.b + 1]) - cu_host[g.b] : p.seqlen;
        const int nc = carry_chunks(len, p.chunk_len, p.nchunks);
        ck.access("A", rA, U(p.A) + (g.d * kN + g.n) * 4, 4);
        if (p.c0_seeded) {
            const uintptr_t q0 = U(p.Q) + ((g.b * p.nchunks * p.D + g.d) * kN + g.n) * 4;
            ck.access("Q", rQ, q0, 4);
            ck.read_written("Q of chunk 0", q0, 4);
        } else if (p.hin) {
            ck.access("h_in", rin, U(p.hin) + ((g.b * p.D + g.d) * kN + g.n) * 4, 4);
        }
        for (int c = p.c0_seeded ? 1 : 0; c < nc && ck.ok(); ++c) {
            const int64_t sc = (g.b * p.nchunks + c) * p.D + g.d;
            if (p.Hc) {
                ck.access("H", rH, U(p.Hc) + (sc * kN + g.n) * 4, 4);
                ck.wrote(U(p.Hc) + (sc * kN + g.n) * 4, 4);
            }
            if (c == nc - 1 && !p.hout) break;
            ck.access("S", rS, U(p.S) + sc * 4, 4);
            ck.read_written("S", U(p.S) + sc * 4, 4);
            ck.access("Q", rQ, U(p.Q) + (sc * kN + g.n) * 4, 4);
            ck.read_written("Q", U(p.Q) + (sc * kN + g.n) * 4, 4);
        }
        if (p.hout) ck.access("h_out", rout, U(p.hout) + ((g.b * p.D + g.d) * kN + g.n) * 4, 4);
    }
}

void check_copy(Checker &ck, const Launch &l) {
    const CopyParams &p = l.copy;
    const int64_t es = l.dtype == R2L_DTYPE_BF16 ? 2 : 4;
    const Region *rs = ck.region_of(p.src), *rd = ck.region_of(p.dst);
    for (int64_t r = 0; r < p.rows && ck.ok(); ++r) {
        const CopyRow cr = copy_row(p, r);
        // columns 0 .. D-1 of the row (one thread per column)
        ck.access("res (copied)", rs, U(p.src) + cr.src * es, p.D * es);
        ck.access("out (copy)", rd, U(p.dst) + cr.dst * es, p.D * es);
    }
}

void check_backward(Checker &ck, const Launch &l, const int32_t *cu_host) {
    const BwdParams &p = l.bwd;
    const int G = l.G, NS = kN / G, K = kCkptTokens, NBC = 2 * kN, STAGE = stage_cols(NBC);
    const int64_t es = l.dtype == R2L_DTYPE_BF16 ? 2 : 4;
    const Region *rA = ck.region_of(p.A), *rDs = p.Dskip ? ck.region_of(p.Dskip) : nullptr;
    const Region *rX = ck.region_of(p.x), *rD = ck.region_of(p.dt), *rG = ck.region_of(p.dout);
    const Region *rB = ck.region_of(p.Bm), *rC = ck.region_of(p.Cm);
    const Region *rdx = p.dx ? ck.region_of(p.dx) : nullptr, *rdd = p.ddt ? ck.region_of(p.ddt) : nullptr;
    const Region *rCk = p.ckpt ? ck.region_of(p.ckpt) : nullptr;
    const Region *rHo = p.dh_out ? ck.region_of(p.dh_out) : nullptr;
    const Region *rHi = p.dh_in ? ck.region_of(p.dh_in) : nullptr;
    ck.cover_blocks("backward launch", p.nblocks, p.tiles, 1);
    for (int64_t bid = 0; bid < padded_grid(p.nblocks) && ck.ok(); ++bid) {
        const BlockGeom bg = block_geom(p.nblocks, p.tiles, 1, bid);
        if (!bg.valid) continue;
        const int64_t s0 = p.cu_seqlens ? cu_host[bg.b] : 0;
        const int64_t s1 = p.cu_seqlens ? cu_host[bg.b + 1] : 0;
        if (p.cu_seqlens) ck.access("cu_seqlens", ck.region_of(p.cu_seqlens), U(p.cu_seqlens) + bg.b * 4, 8);
        const BwdSeqGeom sq = bwd_seq_geom(p, bg.b, s0, s1);
        const SegGeom sg = seg_geom(l.reverse, 0, sq.len > 0 ? sq.len : 1, sq.len);
        const int ntok = sg.ntok;

        uint32_t dmin = UINT32_MAX, dmax = 0;
        for (int lane = 0; lane < kWG; ++lane) {
            const LaneGeom lg = lane_geom(bg.tile, lane, G, p.D);
            dmin = lg.d < dmin ? lg.d : dmin;
            dmax = lg.d > dmax ? lg.d : dmax;
            const int64_t st = static_cast<int64_t>(lg.d) * kN + lg.sub * NS;
            ck.access("A", rA, U(p.A) + st * 4, NS * 4);
            if (p.Dskip) ck.access("Dskip", rDs, U(p.Dskip) + lg.d * 4, 4);
            if (!lg.active) continue;
            const int64_t bs = bg.b * p.D * kN + st;
            if (p.dh_out) ck.access("dh_out", rHo, U(p.dh_out) + bs * 4, NS * 4);
            if (p.dh_in) ck.access("dh_in", rHi, U(p.dh_in) + bs * 4, NS * 4);
            if (p.partA) {
                ck.access("partial dA", ck.region_of(p.partA), U(p.partA) + bs * 4, NS * 4);
                ck.wrote(U(p.partA) + bs * 4, NS * 4);
            }
            if (p.partD && lg.sub == 0) {
                const uintptr_t a = U(p.partD) + (bg.b * p.D + lg.d) * 4;
                ck.access("partial dDskip", ck.region_of(p.partD), a, 4);
                ck.wrote(a, 4);
            }
        }
        if (p.partS) {
            const uintptr_t a = U(p.partS) + (bg.b * p.tiles + bg.tile) * 4;
            ck.access("partial ds", ck.region_of(p.partS), a, 4);
            ck.wrote(a, 4);
        }
        // per-token rows through buffer resources (see check_segment)
        auto row_access = [&](const char *what, const Region *reg, const void *base, int64_t elem_off,
                              int64_t row_elems, int pos) {
            const int row = seg_row(sg, pos);
            if (row < 0 || row >= sq.len)
                return ck.fail("%s: row %d outside the sequence of %lld rows", what, row, (long long)sq.len);
            const uint64_t soff = static_cast<uint64_t>(row) * static_cast<uint64_t>(row_elems * es);
            if (soff > UINT32_MAX) return ck.fail("%s: scalar offset above 32 bits", what);
            if (static_cast<uint64_t>(dmax) * es + es > seq_span_bytes(sq.len, row_elems, p.D, es))
                return ck.fail("%s: lane offset beyond the buffer resource", what);
            const uintptr_t b0 = U(base) + elem_off * es + soff;
            ck.access(what, reg, b0 + static_cast<uint64_t>(dmin) * es, es);
            ck.access(what, reg, b0 + static_cast<uint64_t>(dmax) * es, es);
        };
        for (int gpos = 0; gpos < ntok && ck.ok(); gpos += K) {
            const int gcnt = ntok - gpos < K ? ntok - gpos : K;
            for (int j = 0; j < K; ++j) {
                const int pos = gpos + (j < gcnt ? j : gcnt - 1);
                row_access("x", rX, p.x, sq.xo, p.xs, pos);
                row_access("dt", rD, p.dt, sq.dto, p.dts, pos);
                row_access("dout", rG, p.dout, sq.go, p.gs, pos);
            }
            for (int j = 0; j < gcnt; ++j) {
                if (p.dx) row_access("dx", rdx, p.dx, sq.dxo, p.dxs, gpos + j);
                if (p.ddt) row_access("ddt", rdd, p.ddt, sq.ddo, p.dds, gpos + j);
                const int64_t t = sq.s0p + seg_row(sg, gpos + j);
                if (t < 0 || t >= p.tokens) return ck.fail("partial row %lld outside the tokens", (long long)t);
                for (float *part : {p.partB, p.partC}) {
                    if (!part) continue;
                    const uintptr_t a = U(part) + ((bg.tile * p.tokens + t) * kN) * 4;
                    ck.access("partial dBm/dCm", ck.region_of(part), a, kN * 4);
                    ck.wrote(a, kN * 4);
                }
            }
            for (int lane = 0; lane < kWG; ++lane) {
                const LaneGeom lg = lane_geom(bg.tile, lane, G, p.D);
                const int64_t row = ckpt_row(bg.b, sq.s0p, gpos);
                if (NS != 4) return ck.fail("the backward reads one checkpoint quad per lane");
                const uintptr_t a = U(p.ckpt) + ckpt_quad(row, p.D, lg.d, lg.sub) * 4;
                ck.access("checkpoint", rCk, a, 16);
                ck.read_written("checkpoint", a, 16);
                if (p.Hc) {   // chunked phase 1: the chunk's entry state and the delta sum
                    if (p.chunk_len <= 0 || p.chunk_len % K)
                        return ck.fail("chunk length %d is not a multiple of the group", p.chunk_len);
                    const int64_t c = gpos / p.chunk_len;
                    if (c >= p.nchunks) return ck.fail("group %d past the last chunk", gpos);
                    const uintptr_t ah = U(p.Hc) + (((bg.b * p.nchunks + c) * p.D + lg.d) * kN + lg.sub * NS) * 4;
                    ck.access("chunk entry state", ck.region_of(p.Hc), ah, NS * 4);
                    ck.read_written("chunk entry state", ah, NS * 4);
                    const uintptr_t as = U(p.ckpt_s) + (row * p.D + lg.d) * 4;
                    ck.access("checkpoint delta sum", ck.region_of(p.ckpt_s), as, 4);
                    ck.read_written("checkpoint delta sum", as, 4);
                }
            }
        }
        // Bm / Cm staging: the last tile first, then each earlier (full) tile
        const int ntiles = (ntok + kTile - 1) / kTile;
        for (int ti = ntiles - 1; ti >= 0 && ck.ok(); --ti) {
            const int base = ti * kTile, cnt = ntok - base < kTile ? ntok - base : kTile;
            if (ti < ntiles - 1 && cnt != kTile) return ck.fail("an earlier tile is not full");
            for (int lane = 0; lane < kWG; ++lane) {
                const StageSlot ss = stage_slot(lane, NBC);
                const int64_t row = seg_row(sg, base + stage_pos(ss.k, cnt));
                if (row < 0 || row >= sq.len) return ck.fail("staging row outside the sequence");
                const bool isC = ss.mat != 0;
                const int64_t st = isC ? p.Cs : p.Bs;
                const uint64_t voff = static_cast<uint64_t>(row * st + ss.col0) * es;
                if (voff + STAGE * es > seq_span_bytes(sq.len, st, kN, es))
                    return ck.fail("staging run beyond the buffer resource");
                const uintptr_t addr = U(isC ? p.Cm : p.Bm) + (isC ? sq.Co : sq.Bo) * es + voff;
                if (p.bc_vec && addr % stage_align(NBC, static_cast<int>(es)))
                    return ck.fail("staging vector load not aligned");
                ck.access(isC ? "Cm" : "Bm", isC ? rC : rB, addr, STAGE * es);
            }
        }
    }
}

void check_sum(Checker &ck, const Launch &l) {
    for (int k = 0; k < l.sums.count && ck.ok(); ++k) {
        const SumParams &p = l.sums.seg[k];
        const Region *rs = p.P > 0 ? ck.region_of(p.src) : nullptr, *rd = ck.region_of(p.dst);
        ck.access("gradient (sum)", rd, U(p.dst), p.n * 4);
        for (int64_t q = 0; q < p.P && ck.ok(); ++q) {
            ck.access("partial (sum)", rs, U(p.src) + q * p.pstride * 4, p.n * 4);
            ck.read_written("partial (sum)", U(p.src) + q * p.pstride * 4, p.n * 4);
        }
    }
}

}  // namespace

r2l_status check_backward_accesses(bool reverse, const r2l_scan_args *a, const r2l_grad_args *g,
                                   const BwdPlan &pl, const int32_t *cu_host, r2l_access_report *rep,
                                   const float *saved, size_t saved_bytes) {
    const int64_t es = elem_size(a->dtype), D = a->dim, N = kN;
    const int64_t tok = tokens_of(a);
    std::vector<Region> regs;
    auto add = [&](const char *name, const void *p, uint64_t bytes) {
        if (p && bytes) regs.push_back({name, U(p), U(p) + bytes});
    };
    auto tspan = [&](const void *p, int64_t stride, int64_t bstride, int64_t cols) -> uint64_t {
        if (!p || tok <= 0) return 0;
        const int64_t ext = is_ragged(a)
            ? (tok - 1) * stride + cols
            : (a->batch - 1) * eff_bstride(a, bstride, stride) + (a->seqlen - 1) * stride + cols;
        return static_cast<uint64_t>(ext * es);
    };
    add("x", a->x, tspan(a->x, a->x_stride, a->x_batch_stride, D));
    add("dt", a->dt, tspan(a->dt, a->dt_stride, a->dt_batch_stride, D));
    add("Bm", a->Bm, tspan(a->Bm, a->Bm_stride, a->Bm_batch_stride, N));
    add("Cm", a->Cm, tspan(a->Cm, a->Cm_stride, a->Cm_batch_stride, N));
    add("dout", g->dout, tspan(g->dout, g->dout_stride, g->dout_batch_stride, D));
    add("dx", g->dx, tspan(g->dx, g->dx_stride, g->dx_batch_stride, D));
    add("ddt", g->ddt, tspan(g->ddt, g->ddt_stride, g->ddt_batch_stride, D));
    add("A", a->A, static_cast<uint64_t>(D * N * 4));
    add("Dskip", a->Dskip, static_cast<uint64_t>(D * 4));
    add("h_in", a->h_in, static_cast<uint64_t>(a->batch * D * N * 4));
    add("dh_out", g->dh_out, static_cast<uint64_t>(a->batch * D * N * 4));
    add("dh_in", g->dh_in, static_cast<uint64_t>(a->batch * D * N * 4));
    add("dBm", g->dBm, static_cast<uint64_t>(tok * N * 4));
    add("dCm", g->dCm, static_cast<uint64_t>(tok * N * 4));
    add("dA", g->dA, static_cast<uint64_t>(D * N * 4));
    add("dDskip", g->dDskip, static_cast<uint64_t>(D * 4));
    add("ds", g->ds, 4);
    add("cu_seqlens", a->cu_seqlens, static_cast<uint64_t>((a->batch + 1) * 4));
    const char *ws = static_cast<const char *>(g->workspace);
    const size_t end_S = pl.chunked ? pl.off_Q : pl.ws_bytes;
    const size_t offs[] = {pl.off_ck, pl.off_B, pl.off_C, pl.off_A, pl.off_D, pl.off_S, end_S};
    const char *names[] = {"workspace checkpoints", "workspace dBm partials", "workspace dCm partials",
                           "workspace dA partials", "workspace dDskip partials", "workspace ds partials"};
    for (int i = 0; i < 6; ++i)
        if (ws) add(names[i], ws + offs[i], offs[i + 1] - offs[i]);
    if (ws && pl.chunked) {
        const size_t co[] = {pl.off_Q, pl.off_Sc, pl.off_H, pl.off_cks, pl.ws_bytes};
        const char *cn[] = {"workspace chunk states", "workspace chunk delta sums",
                            "workspace chunk entry states", "workspace checkpoint delta sums"};
        for (int i = 0; i < 4; ++i) add(cn[i], ws + co[i], co[i + 1] - co[i]);
    }
    if (saved) add("saved checkpoints", saved, saved_bytes);   // an input: written by the forward
    Checker ck(std::move(regs), rep);
    ck.set_workspace(g->workspace, pl.ws_bytes);
    Launch ls[kMaxBwdLaunches];
    const int n = build_bwd_launches(reverse, a, g, pl, ls, saved);
    for (int i = 0; i < n && ck.ok(); ++i) {
        ++rep->launches;
        switch (ls[i].kind) {
            case Launch::Segment:
                if (ls[i].seg.bc_vec) ++rep->vector_staging;
                check_segment(ck, ls[i], cu_host);
                break;
            case Launch::Backward:
                if (ls[i].bwd.bc_vec) ++rep->vector_staging;
                check_backward(ck, ls[i], cu_host);
                break;
            case Launch::Carry:
                check_carry(ck, ls[i], cu_host);
                break;
            case Launch::Sum:
                check_sum(ck, ls[i]);
                break;
            default:
                ck.fail("unexpected launch kind in a backward plan");
        }
    }
    return ck.ok() ? R2L_OK : R2L_ERR_INVALID_ARG;
}

r2l_status check_bidir_accesses(const r2l_scan_args *a, const r2l_dir_args *rev, const BidirPlan &bp,
                                const int32_t *cu_host, r2l_access_report *rep) {
    const int64_t es = elem_size(a->dtype), D = a->dim, N = kN;
    const int64_t tok = tokens_of(a);
    const r2l_scan_args r = reverse_view(a, rev);
    std::vector<Region> regs;
    auto add = [&](const char *name, const void *p, uint64_t bytes) {
        if (p && bytes) regs.push_back({name, U(p), U(p) + bytes});
    };
    auto tspan = [&](const void *p, int64_t stride, int64_t bstride, int64_t cols) -> uint64_t {
        if (!p || tok <= 0) return 0;
        const int64_t ext = is_ragged(a)
            ? (tok - 1) * stride + cols
            : (a->batch - 1) * eff_bstride(a, bstride, stride) + (a->seqlen - 1) * stride + cols;
        return static_cast<uint64_t>(ext * es);
    };
    add("x", a->x, tspan(a->x, a->x_stride, a->x_batch_stride, D));
    add("dt", a->dt, tspan(a->dt, a->dt_stride, a->dt_batch_stride, D));
    add("Bm", a->Bm, tspan(a->Bm, a->Bm_stride, a->Bm_batch_stride, N));
    add("Cm", a->Cm, tspan(a->Cm, a->Cm_stride, a->Cm_batch_stride, N));
    add("reverse dt", r.dt, tspan(r.dt, r.dt_stride, r.dt_batch_stride, D));
    add("reverse Bm", r.Bm, tspan(r.Bm, r.Bm_stride, r.Bm_batch_stride, N));
    add("reverse Cm", r.Cm, tspan(r.Cm, r.Cm_stride, r.Cm_batch_stride, N));
    add("res", a->res, tspan(a->res, a->res_stride, a->res_batch_stride, D));
    add("out", a->out, tspan(a->out, a->out_stride, a->out_batch_stride, D));
    add("A", a->A, static_cast<uint64_t>(D * N * 4));
    add("reverse A", r.A, static_cast<uint64_t>(D * N * 4));
    add("Dskip", a->Dskip, static_cast<uint64_t>(D * 4));
    add("reverse Dskip", r.Dskip, static_cast<uint64_t>(D * 4));
    add("h_in", a->h_in, static_cast<uint64_t>(a->batch * D * N * 4));
    add("h_out", a->h_out, static_cast<uint64_t>(a->batch * D * N * 4));
    add("cu_seqlens", a->cu_seqlens, static_cast<uint64_t>((a->batch + 1) * 4));
    const char *ws = static_cast<const char *>(a->workspace);
    const Plan &pl = bp.pl;
    const size_t c0 = bp.off_chunk;
    if (ws && bp.readout) add("workspace readout rows", ws, c0);
    if (ws && pl.chunked) {
        add("workspace Q", ws + c0, pl.off_S);
        add("workspace S", ws + c0 + pl.off_S, (bp.readout ? pl.off_H : pl.ws_bytes) - pl.off_S);
        if (bp.readout) add("workspace H", ws + c0 + pl.off_H, pl.ws_bytes - pl.off_H);
    }
    Checker ck(std::move(regs), rep);
    ck.set_workspace(a->workspace, bp.ws_bytes);
    Launch ls[kMaxBidirLaunches];
    const int n = build_bidir_launches(a, rev, bp, ls);
    for (int i = 0; i < n && ck.ok(); ++i) {
        ++rep->launches;
        const Launch &l = ls[i];
        if (l.kind == Launch::Bidir) {
            // the fused launch: the reverse pass, then the forward pass
            Launch pass = l;
            pass.kind = Launch::Segment;
            pass.reverse = true;
            pass.mode = kModeWs | (l.mode & kModeLds);
            pass.seg = l.seg;
            if (pass.seg.bc_vec) ++rep->vector_staging;
            check_segment(ck, pass, cu_host);
            pass.reverse = false;
            pass.mode = l.mode;
            pass.seg = l.seg2;
            if (pass.seg.bc_vec) ++rep->vector_staging;
            if (ck.ok()) check_segment(ck, pass, cu_host);
        } else if (l.kind == Launch::Segment) {
            if (l.seg.bc_vec) ++rep->vector_staging;
            check_segment(ck, l, cu_host);
        } else if (l.kind == Launch::Copy) {
            check_copy(ck, l);
        } else if (l.kind == Launch::Carry) {
            check_carry(ck, l, cu_host);
        } else {
            ck.fail("unexpected launch kind in a bidirectional plan");
        }
    }
    return ck.ok() ? R2L_OK : R2L_ERR_INVALID_ARG;
}

namespace {

void check_conv(Checker &ck, const Launch &l, const int32_t *cu_host) {
    const ConvParams &p = l.conv;
    const int64_t es = l.dtype == R2L_DTYPE_BF16 ? 2 : 4;
    const Region *rx = ck.region_of(p.x), *ru = ck.region_of(p.u), *rw = ck.region_of(p.w);
    const Region *rb = p.b ? ck.region_of(p.b) : nullptr;
    if (p.K < 1 || p.K > kConvMaxTaps) return ck.fail("conv: %d taps", p.K);
    ck.cover_blocks("conv launch", p.nblocks, p.tiles, p.nchunks);
    for (int64_t bid = 0; bid < padded_grid(p.nblocks) && ck.ok(); ++bid) {
        const BlockGeom bg = block_geom(p.nblocks, p.tiles, p.nchunks, bid);
        if (!bg.valid) continue;
        const int64_t s0 = p.cu_seqlens ? cu_host[bg.b] : bg.b * p.seqlen;
        const int64_t len = p.cu_seqlens ? cu_host[bg.b + 1] - cu_host[bg.b] : p.seqlen;
        if (p.cu_seqlens) ck.access("cu_seqlens", ck.region_of(p.cu_seqlens), U(p.cu_seqlens) + bg.b * 4, 8);
        const int64_t lo = static_cast<int64_t>(bg.c) * kConvTokens;
        if (lo >= len) continue;
        const int64_t hi = lo + kConvTokens < len ? lo + kConvTokens : len;
        const int64_t V = conv_lane_channels(static_cast<int>(es));   // channels per lane
        if (p.D % V) return ck.fail("conv: %lld channels, not a multiple of %lld per lane",
                                    (long long)p.D, (long long)V);
        const int64_t d0 = static_cast<int64_t>(bg.tile) * kWG * V;
        const int64_t d1 = (d0 + kWG * V < p.D ? d0 + kWG * V : p.D) - 1;   // last active channel
        if (d0 > d1) continue;
        // 8-byte accesses: every lane's run starts 8-byte aligned
        if ((U(p.x) + ((s0 + lo) * p.xs + d0) * es) % 8 || (U(p.u) + ((s0 + lo) * p.us + d0) * es) % 8 ||
            (p.xs * es) % 8 || (p.us * es) % 8)
            return ck.fail("conv: an 8-byte access is not 8-byte aligned");
        for (int64_t d : {d0, d1}) {
            ck.access("conv_w", rw, U(p.w) + d * p.K * 4, p.K * 4);
            if (rb) ck.access("conv_b", rb, U(p.b) + d * 4, 4);
        }
        // loads: the chunk and a halo of kConvMaxTaps - 1 rows, cut at the sequence's end
        const int64_t halo_end = lo + kConvTokens + kConvMaxTaps - 1;
        const int64_t last = (halo_end < len ? halo_end : len) - 1;
        for (int64_t t = lo; t <= last && ck.ok(); ++t)
            for (int64_t d : {d0, d1}) {
                const uintptr_t addr = U(p.x) + ((s0 + t) * p.xs + d) * es;
                ck.access("conv x", rx, addr, es);
                ck.read_written("conv x", addr, es);
            }
        for (int64_t t = lo; t < hi && ck.ok(); ++t) {
            const uintptr_t a0 = U(p.u) + ((s0 + t) * p.us + d0) * es;
            ck.access("conv u", ru, a0, es);
            ck.access("conv u", ru, a0 + (d1 - d0) * es, es);
            ck.wrote(a0, (d1 - d0 + 1) * es);
        }
    }
}

// A library GEMM: every matrix it is given lies inside its buffer, and its
// inputs that live in the workspace were written before.
void check_gemm(Checker &ck, const Launch &l) {
    const GemmParams &g = l.gemm;
    const int64_t es = l.dtype == R2L_DTYPE_BF16 ? 2 : 4;
    auto mat = [&](const char *what, const void *p, int64_t rows, int64_t cols, int64_t ld, bool write) {
        if (ld < cols) return ck.fail("%s: leading dimension %lld < %lld", what, (long long)ld, (long long)cols);
        const uint64_t bytes = static_cast<uint64_t>((rows - 1) * ld + cols) * es;
        ck.access(what, ck.region_of(p), U(p), bytes);
        for (int64_t r = 0; r < rows && ck.ok(); ++r) {
            const uintptr_t a0 = U(p) + static_cast<uint64_t>(r * ld) * es;
            if (write)
                ck.wrote(a0, cols * es);
            else
                ck.read_written(what, a0, cols * es);
        }
    };
    if (g.M <= 0 || g.N <= 0 || g.K <= 0) return ck.fail("gemm: empty shape");
    mat("gemm X", g.X, g.M, g.K, g.ldx, false);
    mat("gemm W", g.W, g.N, g.K, g.ldw, false);
    if (g.beta != 0.0f) mat("gemm C", g.C, g.M, g.N, g.ldc, false);
    mat("gemm Y", g.Y, g.M, g.N, g.ldy, true);
    if (g.ws) ck.access("gemm scratch", ck.region_of(g.ws), U(g.ws), g.ws_bytes);
}

}  // namespace

r2l_status check_sidecar_accesses(const r2l_sidecar_args *a, const SidecarPlan &sp,
                                  const int32_t *cu_host, r2l_access_report *rep) {
    const int64_t es = a->dtype == R2L_DTYPE_BF16 ? 2 : 4, di = a->d_inner, dm = a->d_model;
    const int64_t T = sp.tokens, N = kN, R = a->dt_rank;
    std::vector<Region> regs;
    auto add = [&](const char *name, const void *p, uint64_t bytes) {
        if (p && bytes) regs.push_back({name, U(p), U(p) + bytes});
    };
    auto rows = [&](int64_t n, int64_t ld, int64_t cols) -> uint64_t {
        return n > 0 ? static_cast<uint64_t>(((n - 1) * ld + cols) * es) : 0;
    };
    add("hidden", a->hidden, rows(T, a->hidden_stride, dm));
    add("out", a->out, rows(T, a->out_stride, dm));
    add("W_in", a->W_in, rows(2 * di, dm, dm));
    add("W_x", a->W_x, rows(R + 2 * N, di, di));
    add("W_dt", a->W_dt, rows(di, R, R));
    add("W_out", a->W_out, rows(dm, di, di));
    add("conv_w", a->conv_w, static_cast<uint64_t>(di * a->d_conv * 4));
    add("conv_b", a->conv_b, static_cast<uint64_t>(di * 4));
    add("dt_bias", a->dt_bias, static_cast<uint64_t>(di * 4));
    add("A", a->A, static_cast<uint64_t>(di * N * 4));
    add("Dskip", a->Dskip, static_cast<uint64_t>(di * 4));
    add("cu_seqlens", a->cu_seqlens, static_cast<uint64_t>((a->batch + 1) * 4));
    const char *ws = static_cast<const char *>(a->workspace);
    if (ws && sp.runs) {
        add("workspace x|z", ws + sp.off_xz, sp.off_u - sp.off_xz);
        add("workspace u", ws + sp.off_u, sp.off_xdbl - sp.off_u);
        add("workspace r|B|C", ws + sp.off_xdbl, sp.off_dt - sp.off_xdbl);
        add("workspace dt", ws + sp.off_dt, sp.off_g - sp.off_dt);
        add("workspace gated y", ws + sp.off_g, sp.off_chunk - sp.off_g);
        if (sp.pl.chunked) {
            const char *c = ws + sp.off_chunk;
            add("workspace Q", c, sp.pl.off_S);
            add("workspace S", c + sp.pl.off_S, sp.pl.off_H - sp.pl.off_S);
            add("workspace H", c + sp.pl.off_H, sp.pl.ws_bytes - sp.pl.off_H);
        }
        add("workspace gemm scratch", ws + sp.off_gemm, sp.ws_bytes - sp.off_gemm);
    }
    Checker ck(std::move(regs), rep);
    ck.set_workspace(sp.runs ? a->workspace : nullptr, sp.runs ? sp.ws_bytes : 0);
    Launch ls[kMaxSidecarLaunches];
    const int n = build_sidecar_launches(a, sp, ls);
    for (int i = 0; i < n && ck.ok(); ++i) {
        ++rep->launches;
        const Launch &l = ls[i];
        switch (l.kind) {
            case Launch::Segment:
                if (l.seg.bc_vec) ++rep->vector_staging;
                check_segment(ck, l, cu_host);
                break;
            case Launch::Carry: check_carry(ck, l, cu_host); break;
            case Launch::Copy: check_copy(ck, l); break;
            case Launch::Conv: check_conv(ck, l, cu_host); break;
            case Launch::Gemm: check_gemm(ck, l); break;
            default: ck.fail("unexpected launch kind in a sidecar plan");
        }
    }
    return ck.ok() ? R2L_OK : R2L_ERR_INVALID_ARG;
}

r2l_status check_accesses(Op op, const r2l_scan_args *a, const Plan &pl, const int32_t *cu_host,
                          r2l_access_report *rep, float *ckpt, size_t ckpt_bytes) {
    const int64_t es = elem_size(a->dtype), D = a->dim, N = kN;
    const int64_t tok = tokens_of(a);
    std::vector<Region> regs;
    auto add = [&](const char *name, const void *p, uint64_t bytes) {
        if (p && bytes) regs.push_back({name, U(p), U(p) + bytes});
    };
    auto tspan = [&](const void *p, int64_t stride, int64_t bstride, int64_t cols) -> uint64_t {
        if (!p || tok <= 0) return 0;
        const int64_t ext = is_ragged(a)
            ? (tok - 1) * stride + cols
            : (a->batch - 1) * eff_bstride(a, bstride, stride) + (a->seqlen - 1) * stride + cols;
        return static_cast<uint64_t>(ext * es);
    };
    add("x", a->x, tspan(a->x, a->x_stride, a->x_batch_stride, D));
    add("dt", a->dt, tspan(a->dt, a->dt_stride, a->dt_batch_stride, D));
    add("Bm", a->Bm, tspan(a->Bm, a->Bm_stride, a->Bm_batch_stride, N));
    add("Cm", a->Cm, tspan(a->Cm, a->Cm_stride, a->Cm_batch_stride, N));
    add("res", a->res, tspan(a->res, a->res_stride, a->res_batch_stride, D));
    add("out", a->out, tspan(a->out, a->out_stride, a->out_batch_stride, D));
    add("A", a->A, static_cast<uint64_t>(D * N * 4));
    add("Dskip", a->Dskip, static_cast<uint64_t>(D * 4));
    add("h_in", a->h_in, static_cast<uint64_t>(a->batch * D * N * 4));
    add("h_out", a->h_out, static_cast<uint64_t>(a->batch * D * N * 4));
    add("cu_seqlens", a->cu_seqlens, static_cast<uint64_t>((a->batch + 1) * 4));
    if (pl.chunked) {
        const char *ws = static_cast<const char *>(a->workspace);
        add("workspace Q", ws, pl.off_S);
        add("workspace S", ws + pl.off_S, (runs_readout(op, a) ? pl.off_H : pl.ws_bytes) - pl.off_S);
        if (runs_readout(op, a)) add("workspace H", ws + pl.off_H, pl.ws_bytes - pl.off_H);
    }
    const bool saving = ckpt != nullptr;
    if (saving) add("checkpoints", ckpt, ckpt_bytes);
    Checker ck(std::move(regs), rep);
    if (pl.chunked) ck.set_workspace(a->workspace, pl.ws_bytes);
    if (saving) ck.track(ckpt, checkpoint_bytes(a));
    Launch ls[kMaxSaveLaunches];
    const int n = saving ? build_save_launches(op, a, pl, ckpt, ls) : build_launches(op, a, pl, ls);
    // launch order: no scan may read an input after the residual copy of the
    // same call has overwritten it (out aliasing x, dt, Bm or Cm)
    for (int i = 0; i < n && ck.ok(); ++i) {
        if (ls[i].kind != Launch::Copy) continue;
        const Region *dst = ck.region_of(ls[i].copy.dst);
        for (int j = i + 1; j < n && ck.ok(); ++j) {
            if (ls[j].kind != Launch::Segment) continue;
            const SegParams &p = ls[j].seg;
            const void *ins[] = {p.x, p.dt, p.Bm, p.Cm, p.res};
            const char *names[] = {"x", "dt", "Bm", "Cm", "res"};
            for (int k = 0; k < 5; ++k)
                if (ins[k] && ck.region_of(ins[k]) == dst)
                    ck.fail("launch %d reads %s after launch %d (the residual copy) overwrote it",
                            j, names[k], i);
        }
    }
    for (int i = 0; i < n && ck.ok(); ++i) {
        ++rep->launches;
        if (ls[i].kind == Launch::Segment) {
            if (ls[i].seg.bc_vec) ++rep->vector_staging;
            check_segment(ck, ls[i], cu_host);
        } else if (ls[i].kind == Launch::Copy) {
            check_copy(ck, ls[i]);
        } else {
            check_carry(ck, ls[i], cu_host);
        }
    }
    // a saving forward leaves every checkpoint row the backward reads written
    for (int64_t b = 0; saving && b < a->batch && ck.ok(); ++b) {
        const int64_t s0 = is_ragged(a) ? cu_host[b] : b * a->seqlen;
        const int64_t len = is_ragged(a) ? cu_host[b + 1] - cu_host[b] : a->seqlen;
        for (int64_t pos = 0; pos < len && ck.ok(); pos += kCkptTokens)
            ck.read_written("checkpoint row (for the backward)",
                            U(ckpt) + static_cast<uint64_t>(ckpt_row(b, s0, pos) * D * N) * 4, D * N * 4);
    }
    return ck.ok() ? R2L_OK : R2L_ERR_INVALID_ARG;
}

}  // namespace r2l
