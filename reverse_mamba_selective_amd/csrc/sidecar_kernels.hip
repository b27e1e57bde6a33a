// sidecar_kernels.hip -- gfx950 kernels of the sidecar block around the R2L
// scan ("Bifocal Diffusion Language Models", section 2, names a Mamba SSM
// sidecar run over the reversed sequence and gives none of its internals;
// this is the plain Mamba block): the depthwise conv + SiLU, and the scan
// instantiations with the dt bias and the SiLU(z) gate. The four projections
// are library GEMMs (gemm.cpp).
//
// The conv of the reversed sequence is, in the original order, an
// anti-causal conv: tap K-1-j weighs the token j positions to the right. A
// lane owns 8 bytes of channels (4 bf16 or 2 fp32) of a chunk of
// kConvTokens tokens: it issues the loads of the chunk and its halo together
// (the conv is bound by memory latency otherwise), then computes the chunk;
// a wave moves 512 consecutive bytes of a token row per access.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scan_device.h"
#include "scan_geometry.h"
#include "scan_internal.h"
#include "scan_segment.h"

namespace r2l {
namespace {

template <typename T>
__global__ __launch_bounds__(kWG) void conv_silu_kernel(const ConvParams p) {
    using E = Elem<T>;
    constexpr int CT = kConvTokens, W = kConvTokens + kConvMaxTaps - 1;
    constexpr int V = conv_lane_channels(sizeof(T));      // channels per lane, one 8-byte access
    const BlockGeom bg = block_geom(p.nblocks, p.tiles, p.nchunks, blockIdx.x);
    if (!bg.valid) return;
    const int64_t b = bg.b;
    int64_t s0, len;
    if (p.cu_seqlens) {
        s0 = p.cu_seqlens[b];
        len = p.cu_seqlens[b + 1] - s0;
    } else {
        s0 = b * p.seqlen;
        len = p.seqlen;
    }
    const int64_t lo = static_cast<int64_t>(bg.c) * CT;
    if (lo >= len) return;
    const int64_t d0 = (static_cast<int64_t>(bg.tile) * kWG + threadIdx.x) * V;
    if (d0 >= p.D) return;                  // D is a multiple of V

    // w[c][j] weighs x[t + j] of channel d0 + c; taps past K are zero
    float w[V][kConvMaxTaps], bias[V];
#pragma unroll
    for (int c = 0; c < V; ++c) {
#pragma unroll
        for (int j = 0; j < kConvMaxTaps; ++j)
            w[c][j] = j < p.K ? p.w[(d0 + c) * p.K + (p.K - 1 - j)] : 0.0f;
        bias[c] = p.b ? p.b[d0 + c] : 0.0f;
    }
    const T *x = static_cast<const T *>(p.x) + (s0 + lo) * p.xs + d0;
    T *u = static_cast<T *>(p.u) + (s0 + lo) * p.us + d0;
    const int64_t n = len - lo;   // tokens of the sequence from lo on (>= 1)

    // every input of the chunk and its halo first (independent 8-byte loads
    // in flight together), zero past the sequence
    uint2 v[W];
#pragma unroll
    for (int i = 0; i < W; ++i)
        v[i] = i < n ? *reinterpret_cast<const uint2 *>(x + i * p.xs) : make_uint2(0u, 0u);
    auto elem = [&](const uint2 &q, int c) {   // channel c of a loaded run
        const uint32_t word = c * static_cast<int>(sizeof(T)) < 4 ? q.x : q.y;
        if constexpr (sizeof(T) == 2)
            return __uint_as_float((c & 1) ? (word & 0xFFFF0000u) : (word << 16));
        else
            return __uint_as_float(word);
    };
#pragma unroll
    for (int i = 0; i < CT; ++i) {
        if (i >= n) break;
        float o[V];
#pragma unroll
        for (int c = 0; c < V; ++c) {
            float acc = bias[c];
#pragma unroll
            for (int j = 0; j < kConvMaxTaps; ++j) acc = fmaf(w[c][j], elem(v[i + j], c), acc);
            // SiLU(v) = v / (1 + e^-v)
            o[c] = acc * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-acc * kLog2e));
        }
        uint2 q;
        if constexpr (sizeof(T) == 2) {
            q.x = static_cast<uint32_t>(E::pack(o[0])) | (static_cast<uint32_t>(E::pack(o[1])) << 16);
            q.y = static_cast<uint32_t>(E::pack(o[2])) | (static_cast<uint32_t>(E::pack(o[3])) << 16);
        } else {
            q.x = __float_as_uint(o[0]);
            q.y = __float_as_uint(o[1]);
        }
        *reinterpret_cast<uint2 *>(u + i * p.us) = q;
    }
}

template <typename T, int MODE>
hipError_t seg(const SegParams &p, hipStream_t stream) {
    hipLaunchKernelGGL((segment_scan_kernel<true, T, 1, MODE, true>), dim3(padded_grid(p.nblocks)),
                       dim3(kWG), 0, stream, p);
    return hipGetLastError();
}

template <typename T>
hipError_t seg_m(int mode, const SegParams &p, hipStream_t stream) {
    switch (mode) {
        case kModeGate | kModeBias: return seg<T, kModeGate | kModeBias>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_conv(int dtype, const ConvParams &p, hipStream_t stream) {
    if (p.nblocks <= 0) return hipSuccess;
    const dim3 grid(static_cast<uint32_t>(padded_grid(p.nblocks)));
    if (dtype == 1)
        hipLaunchKernelGGL(conv_silu_kernel<uint16_t>, grid, dim3(kWG), 0, stream, p);
    else
        hipLaunchKernelGGL(conv_silu_kernel<float>, grid, dim3(kWG), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_sidecar_segment(int dtype, int mode, const SegParams &p, hipStream_t stream) {
    return dtype == 1 ? seg_m<uint16_t>(mode, p, stream) : seg_m<float>(mode, p, stream);
}

}  // namespace r2l
