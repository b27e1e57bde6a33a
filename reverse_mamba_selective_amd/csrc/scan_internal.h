// scan_internal.h -- parameters shared by the host dispatcher (r2l_api.cpp) and
// the gfx950 kernels (scan_kernels.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "r2l_scan.h"

namespace r2l {

constexpr int kN = 16;      // state size the kernels are built for
constexpr int kWG = 256;    // threads per workgroup (4 wave64s)
constexpr int kTile = 64;   // tokens of Bm/Cm rows staged in LDS at a time

// What a segment scan writes per token: nothing (state only), y, or the gated
// residual with x itself or a separate tensor as the residual.
constexpr int kModeState = 0;
constexpr int kModeY = 1;
constexpr int kModeResX = 2;
constexpr int kModeRes = 3;
// The bidirectional scan's two passes: the first writes its y as fp32 rows to
// the workspace (kModeWs), the second adds them to its own y before its
// output rule (kModeAdd combined with kModeY, kModeResX or kModeRes).
constexpr int kModeWs = 4;
constexpr int kModeOutMask = 7;
constexpr int kModeAdd = 8;
// The sidecar block's scan: out = y * SiLU(z), z read through the residual
// slot (kModeGate); Delta = softplus(dt + dt_bias[d]) (kModeBias, also in the
// state-only chunks of its plans).
constexpr int kModeGate = 5;
constexpr int kModeBias = 16;
// The fused bidirectional launch over sequences of at most kBidirLdsTokens
// tokens keeps the first pass's fp32 rows in LDS instead of the workspace
// (each lane reads back only its own channel's rows).
constexpr int kModeLds = 32;
constexpr int kBidirLdsTokens = 32;
// The scan stores the state entering every kCkptTokens-th visited position
// at SegParams::ckpt: the backward's phase 1 (state only), or a forward scan
// with readout that saves them for the backward (chunks scanned state-only
// from zero inside a readout plan never store).
constexpr int kModeCkpt = 64;

// One launch of the segment kernel scans "segments": chunk c (in visiting
// order) of sequence b, for a tile of kWG lanes. With G lanes per channel a
// tile covers kWG / G channels.
struct SegParams {
    int64_t seqlen;              // dense tokens per sequence (when cu_seqlens == nullptr)
    const int32_t *cu_seqlens;   // ragged offsets [batch+1] or nullptr
    int64_t D;
    int32_t chunk_len;           // tokens per chunk, visiting order
    int32_t nchunks;             // chunks per sequence in the grid
    int32_t tiles;               // channel tiles per segment
    int64_t nblocks;             // batch * nchunks * tiles (logical blocks)

    // token strides (xs, ...) and, dense layout only, batch strides (xbs, ...), in elements
    const void *x;  int64_t xs, xbs;
    const void *dt; int64_t dts, dtbs;
    const void *Bm; int64_t Bs, Bbs;
    const void *Cm; int64_t Cs, Cbs;
    // every Bm/Cm row start is aligned for the staging's vector loads
    int32_t bc_vec;
    const float *A;
    const float *Dskip;
    int32_t softplus;

    // state before the segment's first visited token: hin + b*hin_b + c*hin_c + d*kN
    const float *hin; int64_t hin_b, hin_c;
    // state after its last visited token
    float *hfin; int64_t hfin_b, hfin_c;
    // sum of Delta over the segment per channel: sdelta + b*sd_b + c*sd_c + d
    float *sdelta; int64_t sd_b, sd_c;

    const void *res; int64_t rs, rbs;
    float s;
    void *out; int64_t os, obs;

    // chunked readout plans:
    int32_t split_c0;   // chunk pass: chunk 0 reads out from hin, chunks > 0 are state only from 0
    int32_t skip_c0;    // readout pass: chunk 0 was written by the chunk pass
    int32_t skip_last;  // chunk pass: skip each sequence's last chunk (c > 0)

    // backward, phase 1 (state only): the state before every kCkptTokens-th
    // visited position of the sequence, at ckpt + (ckpt_row * D + d) * kN.
    // A chunked phase 1 scans each chunk from zero: its checkpoints are
    // chunk-local, and ckpt_s (when set) receives, at ckpt_row * D + d, the
    // sum of Delta from the chunk's start to the checkpoint.
    float *ckpt;
    float *ckpt_s;

    // bidirectional scan: fp32 [packed tokens, D] rows of y written by the
    // first pass (kModeWs) and added by the second (kModeAdd)
    float *yws;
    const float *yadd;

    // sidecar block (kModeBias): added to dt before softplus, [D]
    const float *dt_bias;
};

// The sidecar's depthwise conv + SiLU over the x half of the in-projection:
// u[t,d] = SiLU(b[d] + sum_{j<K} w[d, K-1-j] * x[t+j, d]) within each
// sequence. One workgroup per (sequence, chunk of kConvTokens, tile of kWG
// channels).
constexpr int kConvTokens = 32;
constexpr int kConvMaxTaps = 4;
// channels one conv lane covers: one 8-byte access (4 bf16 or 2 fp32)
__host__ __device__ constexpr int conv_lane_channels(int elem_bytes) { return 8 / elem_bytes; }
struct ConvParams {
    int64_t seqlen;              // dense tokens per sequence (cu_seqlens == nullptr)
    const int32_t *cu_seqlens;
    int64_t D;
    int32_t K;
    int32_t nchunks;             // ceil(longest sequence / kConvTokens)
    int32_t tiles;
    int64_t nblocks;             // batch * nchunks * tiles
    const void *x; int64_t xs;   // token rows (packed tokens)
    const float *w;              // [D, K]
    const float *b;              // [D] or nullptr
    void *u; int64_t us;
};

// One library GEMM of the sidecar, row-major: Y[M, N] = alpha * X[M, K] W[N, K]^T
// + beta * C[M, N] (C read only when beta != 0), in the storage type (fp32
// accumulation).
struct GemmParams {
    r2l_gemm_context ctx;        // the caller's hipBLASLt handle and algorithm choices
    int64_t M, N, K;
    const void *X; int64_t ldx;
    const void *W; int64_t ldw;
    const void *C; int64_t ldc;
    void *Y; int64_t ldy;
    float alpha, beta;
    void *ws; size_t ws_bytes;   // the library's scratch, inside the caller's workspace
};

// ---- backward (gradients of a scan with readout) ----------------------------
// Visited positions are taken in groups of kCkptTokens; phase 1 stores the
// state entering each group, phase 2 recomputes a group's states from it and
// runs the adjoint over the group backwards.
constexpr int kCkptTokens = 8;

struct BwdParams {
    int64_t seqlen;              // dense tokens per sequence (when cu_seqlens == nullptr)
    const int32_t *cu_seqlens;
    int64_t D;
    int32_t tiles;               // channel tiles per sequence (kWG / G channels each)
    int64_t nblocks;             // batch * tiles
    int64_t tokens;              // packed token count (row space of the partial sums)

    const void *x;  int64_t xs, xbs;
    const void *dt; int64_t dts, dtbs;
    const void *Bm; int64_t Bs, Bbs;
    const void *Cm; int64_t Cs, Cbs;
    int32_t bc_vec;
    const float *A;
    const float *Dskip;
    int32_t softplus;

    float dyscale;               // dL/dy = dyscale * dout (s with a residual, else 1)
    float dxres;                 // 1 when the residual is x itself (dx += dout), else 0
    int32_t want_ds;             // accumulate dout * y for ds

    const float *ckpt;           // phase 1's checkpoints
    // chunked phase 1 (Hc != nullptr): the true state entering a group of
    // chunk c = pos / chunk_len is ckpt + exp(A * ckpt_s) * Hc[b][c], Hc the
    // state entering the chunk ([batch][nchunks][D][kN], from the carry)
    int32_t chunk_len, nchunks;
    const float *Hc;
    const float *ckpt_s;
    const void *dout; int64_t gs, gbs;
    const float *dh_out;         // [batch, D, kN] or nullptr
    void *dx;  int64_t dxs, dxbs;     // or nullptr
    void *ddt; int64_t dds, ddbs;     // or nullptr
    float *dh_in;                // [batch, D, kN] or nullptr

    // partial sums, reduced by sum launches in a fixed order
    float *partB, *partC;        // [tiles][tokens][kN]: over the block's channels
    float *partA;                // [batch][D][kN]: over the sequence's tokens
    float *partD;                // [batch][D]
    float *partS;                // [nblocks]
};

// dst[i] = sum over p < P of src[p * pstride + i], for i < n (in order of p).
struct SumParams {
    const float *src;
    int64_t P, pstride, n;
    float *dst;
};
// Up to five such sums in one launch (first[] is filled at launch).
constexpr int kMaxSums = 5;
struct SumBatch {
    SumParams seg[kMaxSums];
    int32_t count;
    int64_t first[kMaxSums + 1];
};

// Joins chunk results (local final state Q from a zero start and the Delta sum
// S of each chunk) into the state entering every chunk and the final state.
struct CarryParams {
    int64_t batch;
    int64_t seqlen;
    const int32_t *cu_seqlens;
    int64_t D;
    int32_t chunk_len;
    int32_t nchunks;
    const float *A;
    const float *hin;            // [batch, D, N] or nullptr (zero)
    const float *Q;              // [batch, nchunks, D, N]
    const float *S;              // [batch, nchunks, D]
    float *Hc;                   // [batch, nchunks, D, N] state entering each chunk, or nullptr
    float *hout;                 // [batch, D, N] or nullptr
    int32_t c0_seeded;           // Q of chunk 0 is the true state after it (hin is not read)
};

// Copies D elements of each token row from src to dst (a call with s == 0
// writes the residual itself). Dense layout (seqlen > 0): row r is token
// r % seqlen of sequence r / seqlen, at b * batch stride + l * stride;
// packed layout (seqlen == 0): row r at r * stride. Strides in elements.
struct CopyParams {
    int64_t rows;
    int64_t seqlen;
    int64_t D;
    const void *src; int64_t ss, sbs;
    void *dst; int64_t ds, dbs;
};

// dtype: 0 fp32, 1 bf16. G in {1, 2, 4}. mode: kMode*.
hipError_t launch_segment_scan(bool reverse, int dtype, int G, int mode,
                               const SegParams &p, hipStream_t stream);
hipError_t launch_carry(const CarryParams &p, hipStream_t stream);
// bidirectional scan: one launch running both passes (unchunked plans), or a
// segment launch of one direction's chunked plan (modes kModeWs, kModeAdd | m)
hipError_t launch_bidir_fused(int dtype, int out_mode, bool lds_rows, const SegParams &pr,
                              const SegParams &pf, hipStream_t stream);
hipError_t launch_bidir_segment(bool reverse, int dtype, int mode, const SegParams &p,
                                hipStream_t stream);
hipError_t launch_copy(int dtype, const CopyParams &p, hipStream_t stream);
// sidecar: the conv + SiLU, and a segment launch of its scan (modes
// kModeGate | kModeBias, or kModeState | kModeBias)
hipError_t launch_conv(int dtype, const ConvParams &p, hipStream_t stream);
hipError_t launch_sidecar_segment(int dtype, int mode, const SegParams &p, hipStream_t stream);
// The caller-owned GEMM context (include/r2l_scan.h): create on the current
// device, check that a handle is a live context of the current device,
// destroy. Each returns a description of a failure, or nullptr.
const char *gemm_context_create(r2l_gemm_context *out);
const char *gemm_context_check(r2l_gemm_context ctx);
const char *gemm_context_destroy(r2l_gemm_context ctx);
// a GEMM through hipBLASLt with the context's handle and its algorithm for the
// shape (chosen on first use); returns a description of a failure, or nullptr
const char *run_gemm(r2l_gemm_context ctx, int dtype, const GemmParams &p, hipStream_t stream);
// times the library's candidates for this GEMM on `stream` (writing Y, or
// y_scratch when given, with the same leading dimension) and keeps the fastest
// in the context for later calls of the same shape; synchronizes the stream
const char *tune_gemm(r2l_gemm_context ctx, int dtype, const GemmParams &p, void *y_scratch,
                      hipStream_t stream);
// r2l_scan_noalloc: the device address of the library's scratch array on the
// current device (looked up once per device), kNoallocScratchBytes long
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(void **ptr);
// G in {2, 4}
hipError_t launch_backward(bool reverse, int dtype, int G, const BwdParams &p, hipStream_t stream);
hipError_t launch_sums(const SumBatch &p, hipStream_t stream);

}  // namespace r2l
