// scan_geometry.h -- the index math of the segment-scan and carry kernels,
// shared by the kernels (device) and by the host-side access checker
// (bounds_check.cpp), so that the checker sees exactly the addresses the
// kernels form.
#pragma once

#include <stdint.h>

#include "scan_internal.h"

#if defined(__HIPCC__)
#define R2L_HD __host__ __device__ __forceinline__
#else
#define R2L_HD inline
#endif

namespace r2l {

constexpr int kPrefetch = 8;   // tokens of x/dt/res loaded ahead of use
static_assert(kN == 16, "carry_geom splits (channel, state) with a 4-bit shift");

// Block -> (sequence b, chunk c, channel tile). Launches pad the grid to a
// multiple of 8 and remap ids so that consecutive logical blocks (the tiles of
// one segment) land on one XCD: hardware block i goes to XCD i % 8.
struct BlockGeom {
    bool valid;
    int tile;
    int c;
    int64_t b;
};

R2L_HD int64_t padded_grid(int64_t nblocks) { return ((nblocks + 7) / 8) * 8; }

// 32-bit arithmetic: the host keeps the padded grid below 2^31 blocks.
R2L_HD BlockGeom block_geom(int64_t nblocks, int32_t tiles, int32_t nchunks, int64_t bid) {
    BlockGeom g{false, 0, 0, 0};
    const uint32_t nb = static_cast<uint32_t>(nblocks);
    const uint32_t id = static_cast<uint32_t>(bid);
    const uint32_t per = (nb + 7) >> 3;
    const uint32_t logical = (id & 7) * per + (id >> 3);
    if (logical >= nb) return g;
    g.valid = true;
    const uint32_t t = static_cast<uint32_t>(tiles), nc = static_cast<uint32_t>(nchunks);
    // An integer division by a runtime value is ~20 scalar instructions at
    // every wave's start; the common shapes take the short ways (a power-of-two
    // tile count, one chunk).
    uint32_t seg;
    if ((t & (t - 1)) == 0) {
        g.tile = static_cast<int>(logical & (t - 1));
        seg = logical >> __builtin_ctz(t);
    } else {
        g.tile = static_cast<int>(logical % t);
        seg = logical / t;
    }
    if (nc == 1) {
        g.c = 0;
        g.b = static_cast<int64_t>(seg);
    } else {
        g.c = static_cast<int>(seg % nc);
        g.b = static_cast<int64_t>(seg / nc);
    }
    return g;
}

// Packed token index of sequence b's first row (the row space of the
// workspace's per-token arrays): the ragged offset, or b * seqlen.
R2L_HD int64_t packed_start(const int32_t *cu_seqlens, int64_t seqlen, int64_t b, int64_t s0) {
    return cu_seqlens ? s0 : b * seqlen;
}

// Sequence b: its length, its packed start and the element offset of its
// first row in each token-major tensor. s0, s1 are cu_seqlens[b],
// cu_seqlens[b+1] (ragged).
struct SeqGeom {
    int64_t len, s0p, xo, dto, Bo, Co, ro, oo;
};

R2L_HD SeqGeom seq_geom(const SegParams &p, int64_t b, int64_t s0, int64_t s1) {
    SeqGeom q;
    q.s0p = packed_start(p.cu_seqlens, p.seqlen, b, s0);
    if (p.cu_seqlens) {
        q.len = s1 - s0;
        q.xo = s0 * p.xs; q.dto = s0 * p.dts; q.Bo = s0 * p.Bs; q.Co = s0 * p.Cs;
        q.ro = s0 * p.rs; q.oo = s0 * p.os;
    } else {
        q.len = p.seqlen;
        q.xo = b * p.xbs; q.dto = b * p.dtbs; q.Bo = b * p.Bbs; q.Co = b * p.Cbs;
        q.ro = b * p.rbs; q.oo = b * p.obs;
    }
    return q;
}

// Chunk c of a sequence of len tokens, in visiting order. `run` is false for
// a chunk past the end (the block exits); chunk 0 always runs, possibly with
// no token, because it writes the final state. The k-th visited token of the
// segment is sequence row t_first + step * k, for 0 <= k < ntok.
struct SegGeom {
    bool run;
    bool last;    // the sequence's last chunk
    int ntok;
    int t_first;
    int step;
};

R2L_HD SegGeom seg_geom(bool rev, int c, int64_t chunk_len, int64_t len) {
    SegGeom g{false, false, 0, 0, rev ? -1 : 1};
    const int64_t v0 = static_cast<int64_t>(c) * chunk_len;
    if (c > 0 && v0 >= len) return g;
    const int64_t v1 = v0 + chunk_len < len ? v0 + chunk_len : len;
    g.run = true;
    g.last = v1 >= len;
    g.ntok = v1 > v0 ? static_cast<int>(v1 - v0) : 0;
    g.t_first = static_cast<int>(rev ? len - 1 - v0 : v0);
    return g;
}

// Whether a launch scans chunk c at all: the readout pass of a plan whose
// chunk pass already wrote chunk 0 skips it, and a chunk pass whose caller
// wants no final state skips each sequence's last chunk (c > 0), whose local
// results nothing reads.
R2L_HD bool segment_runs(const SegParams &p, const SegGeom &sg, int c) {
    if (!sg.run) return false;
    if (p.skip_c0 && c == 0) return false;
    if (p.skip_last && c > 0 && sg.last) return false;
    return true;
}

// State a segment starts from: its slot of hin, except in a split chunk pass,
// where only chunk 0 starts from the call's initial state (hin) and the others
// from zero.
R2L_HD const float *segment_hin(const SegParams &p, int64_t b, int c) {
    if (!p.hin || (p.split_c0 && c > 0)) return nullptr;
    return p.hin + b * p.hin_b + c * p.hin_c;
}

R2L_HD int seg_row(const SegGeom &g, int k) { return g.t_first + g.step * k; }

// The visited position whose inputs are loaded into the register ring when
// position k is wanted: k itself while it exists, else the last one (a
// harmless reload). Only meaningful when ntok > 0.
R2L_HD int prefetch_pos(int k, int ntok) { return k < ntok ? k : ntok - 1; }

// Lane -> channel: G adjacent lanes share channel d and hold states
// sub*NS .. sub*NS+NS-1. Lanes past the last channel shadow it (same inputs,
// bit-identical results) so that every lane can run the same code.
struct LaneGeom {
    bool active;
    int sub;
    uint32_t d;
};

R2L_HD LaneGeom lane_geom(int tile, int lane, int G, int64_t D) {
    LaneGeom g;
    const int64_t gl = static_cast<int64_t>(tile) * kWG + lane;
    const int64_t own = gl / G;
    g.sub = static_cast<int>(gl % G);
    g.active = own < D;
    g.d = static_cast<uint32_t>(g.active ? own : D - 1);
    return g;
}

// Bm/Cm staging of one tile of kTile tokens, nbc staged columns per token (kN
// of Bm, then kN of Cm when the readout needs them). Thread tid fills
// stage_cols(nbc) consecutive columns, from col0 on, of matrix `mat` (0: Bm,
// 1: Cm) for tile token k: LDS floats k*nbc + mat*kN + col0 ... Threads
// 0..127 take Bm and 128..255 Cm (readout), so the matrix is uniform per wave.
struct StageSlot {
    int mat, k, col0;
};

R2L_HD constexpr int stage_cols(int nbc) { return kTile * nbc / kWG; }

R2L_HD StageSlot stage_slot(int tid, int nbc) {
    const int cols = stage_cols(nbc);
    const int per_row = kN / cols;             // threads per matrix row
    const int per_mat = kTile * per_row;
    const int r = tid % per_mat;
    return StageSlot{tid / per_mat, r / per_row, (r % per_row) * cols};
}

// Byte alignment that lets a thread fetch its columns with one or two
// vector loads (8 or 16 bytes each).
R2L_HD constexpr int stage_align(int nbc, int es) {
    return stage_cols(nbc) * es < 16 ? stage_cols(nbc) * es : 16;
}

// The tile token whose row a thread loads for slot token k: slots past the
// tile's last token (a short last tile) repeat that token's row, so every
// thread loads and stores without a branch; those slots are never read.
R2L_HD int stage_pos(int k, int tcnt) { return k < tcnt ? k : tcnt - 1; }

// Bytes a raw buffer resource over one sequence of a tensor covers.
R2L_HD uint32_t seq_span_bytes(int64_t len, int64_t row_elems, int64_t D, int64_t es) {
    const int64_t rows = len > 0 ? len - 1 : 0;
    return static_cast<uint32_t>((rows * row_elems + D) * es);
}

// Carry kernel: a 2-D grid, x = sequence b, y = tile of kCarryThreads
// (channel, state) pairs; thread t of tile y covers channel (y*kCarryThreads +
// t) / kN and state t % kN. No division.
constexpr int kCarryThreads = 256;
struct CarryGeom {
    bool valid;
    int n;
    int64_t d, b;
};

R2L_HD int64_t carry_tiles(int64_t D) { return (D * kN + kCarryThreads - 1) / kCarryThreads; }

R2L_HD CarryGeom carry_geom(int64_t D, int64_t bx, int64_t by, int tid) {
    CarryGeom g{false, 0, 0, 0};
    const int64_t i = by * kCarryThreads + tid;
    if (i >= D * kN) return g;
    g.valid = true;
    g.n = static_cast<int>(i & (kN - 1));
    g.d = i >> 4;
    g.b = bx;
    return g;
}

// ---- backward ---------------------------------------------------------------
// Checkpoint row of the group starting at visited position pos (a multiple
// of kCkptTokens) of the sequence starting at packed token s0p: distinct for
// every (sequence, group), below ckpt_rows().
R2L_HD int64_t ckpt_row(int64_t b, int64_t s0p, int64_t pos) { return (s0p + pos) / kCkptTokens + b; }
R2L_HD int64_t ckpt_rows(int64_t tokens, int64_t batch) { return tokens / kCkptTokens + batch + 1; }
// Float offset of states [4q, 4q + 4) of channel d in checkpoint row `row`.
// A row holds kN/4 planes of [D][4]: a wave whose lanes (consecutive
// channels) store or load one quad each touches one contiguous run.
R2L_HD int64_t ckpt_quad(int64_t row, int64_t D, int64_t d, int q) {
    return ((row * (kN / 4) + q) * D + d) * 4;
}

// Sequence b in the backward's tensors (element offsets of its first row).
struct BwdSeqGeom {
    int64_t len, s0p, xo, dto, Bo, Co, go, dxo, ddo;
};

R2L_HD BwdSeqGeom bwd_seq_geom(const BwdParams &p, int64_t b, int64_t s0, int64_t s1) {
    BwdSeqGeom q;
    q.s0p = packed_start(p.cu_seqlens, p.seqlen, b, s0);
    if (p.cu_seqlens) {
        q.len = s1 - s0;
        q.xo = s0 * p.xs; q.dto = s0 * p.dts; q.Bo = s0 * p.Bs; q.Co = s0 * p.Cs;
        q.go = s0 * p.gs; q.dxo = s0 * p.dxs; q.ddo = s0 * p.dds;
    } else {
        q.len = p.seqlen;
        q.xo = b * p.xbs; q.dto = b * p.dtbs; q.Bo = b * p.Bbs; q.Co = b * p.Cbs;
        q.go = b * p.gbs; q.dxo = b * p.dxbs; q.ddo = b * p.ddbs;
    }
    return q;
}

// Row copy: kCopyThreads columns per block along x, rows along y (looping
// when there are more rows than kCopyMaxRowBlocks).
constexpr int kCopyThreads = 256;
constexpr int64_t kCopyMaxRowBlocks = 65535;
struct CopyRow {
    int64_t src, dst;   // element offsets of the row's first column
};

R2L_HD CopyRow copy_row(const CopyParams &p, int64_t r) {
    if (p.seqlen > 0) {
        const int64_t b = r / p.seqlen, l = r % p.seqlen;
        return CopyRow{b * p.sbs + l * p.ss, b * p.dbs + l * p.ds};
    }
    return CopyRow{r * p.ss, r * p.ds};
}

R2L_HD int carry_chunks(int64_t len, int32_t chunk_len, int32_t nchunks) {
    const int64_t nc = (len + chunk_len - 1) / chunk_len;
    return static_cast<int>(nc < nchunks ? nc : nchunks);
}

}  // namespace r2l
