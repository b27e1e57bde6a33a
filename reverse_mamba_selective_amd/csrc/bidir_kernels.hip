// bidir_kernels.hip -- gfx950 kernels of the bidirectional full-window scan:
// the forward scan of x with one parameter set plus the reverse scan of the
// same x with another, readouts added, then the gated residual. This is the
// full-window bidirectional Mamba scan of the earlier block-diffusion hybrids
// that "Training Hybrid Block Diffusion Language Models with Partial
// Bidirectionality" (problem statement) contrasts with its reverse scan
// restricted to the active block; "Bifocal Diffusion Language Models"
// (section 4) compares the directions in its ablations.
//
// Mapping onto CDNA4 (one lane per channel, as the single-direction scans):
//  * Unchunked plans run one launch: each workgroup owns (sequence, tile of
//    kWG channels), scans its tile right to left writing y_reverse as fp32 rows
//    of the workspace (or of LDS, when every sequence has at most
//    kBidirLdsTokens tokens), then left to right, adding those rows to its own
//    y before the output rule. Every lane reads back only what it wrote itself
//    (its channel's rows), so no synchronisation beyond program order is
//    needed, and the second pass finds x and dt in L2: x is fetched from HBM
//    once per call.
//  * Chunked plans (long windows with few channels) run the reverse
//    direction's chunked plan writing the fp32 rows, then the forward
//    direction's chunked plan adding them (the readout passes of both carry
//    the mode; chunks scanned state-only are untouched).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scan_device.h"
#include "scan_geometry.h"
#include "scan_internal.h"
#include "scan_segment.h"

namespace r2l {
namespace {

// One workgroup per (sequence, channel tile); pr and pf describe the reverse
// and forward passes over the same grid (unchunked, one lane per channel).
// LR: every sequence has at most kBidirLdsTokens tokens and the rows stay in
// LDS (kBidirLdsTokens x kWG fp32, 32 KB).
template <typename T, int OUT, bool SP, bool LR>
__global__ __launch_bounds__(kWG) void bidir_kernel(const SegParams pr, const SegParams pf) {
    __shared__ __align__(16) float lds[2 * kTile * 2 * kN];
    __shared__ float ylds[LR ? kBidirLdsTokens * kWG : 1];
    constexpr int L = LR ? kModeLds : 0;
    const BlockGeom bg = block_geom(pf.nblocks, pf.tiles, 1, blockIdx.x);
    if (!bg.valid) return;
    const int64_t b = bg.b;
    const int64_t s0 = pf.cu_seqlens ? pf.cu_seqlens[b] : 0;
    const int64_t s1 = pf.cu_seqlens ? pf.cu_seqlens[b + 1] : 0;

    const SeqGeom sqr = seq_geom(pr, b, s0, s1);
    const SegGeom sgr = seg_geom(true, 0, pr.chunk_len, sqr.len);
    scan_segment<true, T, 1, kModeWs | L, SP>(pr, lds, bg, sqr, sgr, nullptr, ylds);
    __syncthreads();   // the staging area changes hands

    const SeqGeom sqf = seq_geom(pf, b, s0, s1);
    const SegGeom sgf = seg_geom(false, 0, pf.chunk_len, sqf.len);
    scan_segment<false, T, 1, kModeAdd | OUT | L, SP>(pf, lds, bg, sqf, sgf, segment_hin(pf, b, 0),
                                                      ylds);
}

template <typename T, int OUT, bool SP>
hipError_t fused(bool lr, const SegParams &pr, const SegParams &pf, hipStream_t stream) {
    if (lr)
        hipLaunchKernelGGL((bidir_kernel<T, OUT, SP, true>), dim3(padded_grid(pf.nblocks)), dim3(kWG),
                           0, stream, pr, pf);
    else
        hipLaunchKernelGGL((bidir_kernel<T, OUT, SP, false>), dim3(padded_grid(pf.nblocks)), dim3(kWG),
                           0, stream, pr, pf);
    return hipGetLastError();
}

template <typename T, bool SP>
hipError_t fused_o(int out, bool lr, const SegParams &pr, const SegParams &pf, hipStream_t stream) {
    switch (out) {
        case kModeY: return fused<T, kModeY, SP>(lr, pr, pf, stream);
        case kModeResX: return fused<T, kModeResX, SP>(lr, pr, pf, stream);
        case kModeRes: return fused<T, kModeRes, SP>(lr, pr, pf, stream);
        default: return hipErrorInvalidValue;
    }
}

template <bool REV, typename T, int MODE, bool SP>
hipError_t seg(const SegParams &p, hipStream_t stream) {
    hipLaunchKernelGGL((segment_scan_kernel<REV, T, 1, MODE, SP>), dim3(padded_grid(p.nblocks)),
                       dim3(kWG), 0, stream, p);
    return hipGetLastError();
}

template <typename T, bool SP>
hipError_t seg_m(bool reverse, int mode, const SegParams &p, hipStream_t stream) {
    if (reverse) return mode == kModeWs ? seg<true, T, kModeWs, SP>(p, stream) : hipErrorInvalidValue;
    switch (mode) {
        case kModeAdd | kModeY: return seg<false, T, kModeAdd | kModeY, SP>(p, stream);
        case kModeAdd | kModeResX: return seg<false, T, kModeAdd | kModeResX, SP>(p, stream);
        case kModeAdd | kModeRes: return seg<false, T, kModeAdd | kModeRes, SP>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_bidir_fused(int dtype, int out_mode, bool lds_rows, const SegParams &pr,
                              const SegParams &pf, hipStream_t stream) {
    const bool sp = pf.softplus != 0;
    if (dtype == 1)
        return sp ? fused_o<uint16_t, true>(out_mode, lds_rows, pr, pf, stream)
                  : fused_o<uint16_t, false>(out_mode, lds_rows, pr, pf, stream);
    return sp ? fused_o<float, true>(out_mode, lds_rows, pr, pf, stream)
              : fused_o<float, false>(out_mode, lds_rows, pr, pf, stream);
}

hipError_t launch_bidir_segment(bool reverse, int dtype, int mode, const SegParams &p,
                                hipStream_t stream) {
    const bool sp = p.softplus != 0;
    if (dtype == 1)
        return sp ? seg_m<uint16_t, true>(reverse, mode, p, stream)
                  : seg_m<uint16_t, false>(reverse, mode, p, stream);
    return sp ? seg_m<float, true>(reverse, mode, p, stream)
              : seg_m<float, false>(reverse, mode, p, stream);
}

}  // namespace r2l
