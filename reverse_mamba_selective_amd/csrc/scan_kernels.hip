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
#include "scan_segment.h"

namespace r2l {
namespace {

using namespace dev;

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

// Checkpointing scans run one lane per channel.
template <bool REV, typename T, int MODE, bool SP>
hipError_t launch_ck(int G, const SegParams &p, hipStream_t stream) {
    if (G != 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL((segment_scan_kernel<REV, T, 1, MODE | kModeCkpt, SP>),
                       dim3(padded_grid(p.nblocks)), dim3(kWG), 0, stream, p);
    return hipGetLastError();
}

template <bool REV, typename T, bool SP>
hipError_t launch_m(int mode, int G, const SegParams &p, hipStream_t stream) {
    switch (mode) {
        case kModeState | kModeCkpt: return launch_ck<REV, T, kModeState, SP>(G, p, stream);
        case kModeY | kModeCkpt: return launch_ck<REV, T, kModeY, SP>(G, p, stream);
        case kModeResX | kModeCkpt: return launch_ck<REV, T, kModeResX, SP>(G, p, stream);
        case kModeRes | kModeCkpt: return launch_ck<REV, T, kModeRes, SP>(G, p, stream);
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
