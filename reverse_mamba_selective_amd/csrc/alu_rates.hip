// alu_rates.hip -- issue-rate micro-benchmark of the gfx950 vector ALU, the
// measurement behind the scan's ALU roofline (libr2l_alu_rates.so, loaded by
// bench.py --alu-rates only; not part of the scan library).
//
// The selective scan needs one exponential per (token, channel, state) beside
// four fp32 VALU operations, so what an exponential costs in VALU issue slots,
// alone and mixed with FMAs, sets the ALU ceiling. Each kernel runs NC
// independent dependency chains per lane (enough independent work that issue,
// not latency, bounds it at the chosen occupancy) for `iters` iterations:
//   kind 0: v_fma_f32 only      a = a * c + d           (NC fmas / iteration)
//   kind 1: v_exp_f32 only      a = exp2(-a)            (NC exps / iteration)
//   kind 2: v_exp_f32 + 4 fmas  a = exp2(-a); b0..b3 = b * c + d
//                                                       (NC exps + 4 NC fmas)
//   kind 3: v_log_f32 only      a = log2(|a|)           (the abs is a source
//                               modifier; the chain settles at +inf, and the
//                               unit's issue rate does not depend on the value)
// The time of kind 1 or 2 over kind 0, per instruction, gives the issue slots
// one transcendental takes. Thread 0 of every block also records the shader
// clock counter (clock64, s_memtime) and the constant-rate wall clock
// (wall_clock64, s_memrealtime) around its loop, so that the cycles a SIMD
// spends per wave instruction, and the shader clock the device actually ran
// at, come out of the same run.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

constexpr int kNC = 16;   // independent chains per lane

template <int KIND>
__global__ __launch_bounds__(256) void alu_rate_kernel(float *out, unsigned long long *clk,
                                                       int iters, float c, float d) {
    const int tid = blockIdx.x * blockDim.x + threadIdx.x;
    const unsigned long long c0 = clock64(), w0 = wall_clock64();
    float a[kNC], b[4 * kNC];
#pragma unroll
    for (int i = 0; i < kNC; ++i) a[i] = KIND == 3 ? 3.0e38f : 0.5f + 0.01f * (tid & 7) + 0.001f * i;
#pragma unroll
    for (int i = 0; i < 4 * kNC; ++i) b[i] = 0.25f + 0.001f * i;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < kNC; ++i) {
            if constexpr (KIND == 0) {
                a[i] = fmaf(a[i], c, d);
            } else if constexpr (KIND == 1) {
                a[i] = __builtin_amdgcn_exp2f(-a[i]);
            } else if constexpr (KIND == 2) {
                a[i] = __builtin_amdgcn_exp2f(-a[i]);
#pragma unroll
                for (int j = 0; j < 4; ++j) b[4 * i + j] = fmaf(b[4 * i + j], c, d);
            } else {
                a[i] = __builtin_amdgcn_logf(fabsf(a[i]));
            }
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kNC; ++i) s += a[i];
    if constexpr (KIND == 2) {
#pragma unroll
        for (int i = 0; i < 4 * kNC; ++i) s += b[i];
    }
    const unsigned long long c1 = clock64(), w1 = wall_clock64();
    out[tid] = s;
    if (threadIdx.x == 0 && clk) {
        clk[4 * blockIdx.x] = c0;
        clk[4 * blockIdx.x + 1] = c1;
        clk[4 * blockIdx.x + 2] = w0;
        clk[4 * blockIdx.x + 3] = w1;
    }
}

}  // namespace

extern "C" {

// Launches kind `kind` (0..3) over blocks x 256 threads on `stream`; out holds
// blocks * 256 floats, clk (or NULL) blocks * 4 counters: shader clock at the
// start and end of block's loop, wall clock at the start and end. Returns a
// hipError_t. Per lane and iteration the kernel issues 16 instructions of the
// measured kind (kind 2: 16 exps and 64 fmas).
__attribute__((visibility("default"))) int r2l_alu_rate_launch(int kind, int blocks, int iters,
                                                               float *out,
                                                               unsigned long long *clk,
                                                               void *stream) {
    if (blocks <= 0 || iters <= 0 || !out) return hipErrorInvalidValue;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid(static_cast<uint32_t>(blocks)), block(256);
    switch (kind) {
        case 0: hipLaunchKernelGGL(alu_rate_kernel<0>, grid, block, 0, s, out, clk, iters, 0.999f, 0.001f); break;
        case 1: hipLaunchKernelGGL(alu_rate_kernel<1>, grid, block, 0, s, out, clk, iters, 0.999f, 0.001f); break;
        case 2: hipLaunchKernelGGL(alu_rate_kernel<2>, grid, block, 0, s, out, clk, iters, 0.999f, 0.001f); break;
        case 3: hipLaunchKernelGGL(alu_rate_kernel<3>, grid, block, 0, s, out, clk, iters, 0.999f, 0.001f); break;
        default: return hipErrorInvalidValue;
    }
    return static_cast<int>(hipGetLastError());
}

// Rate of wall_clock64() in kHz on the current device.
__attribute__((visibility("default"))) int r2l_alu_wall_clock_khz(int *khz) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev);
    return static_cast<int>(e);
}

}  // extern "C"
