// scan_device.h -- device helpers shared by the gfx950 kernels (forward
// segment scan, carry, copy, backward): element access, raw buffer resources,
// softplus with hardware base-2 ops, sums across the lanes of a channel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace r2l {
namespace dev {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- element access -------------------------------------------------------
template <typename T>
struct Elem;

template <>
struct Elem<float> {
    using raw_t = uint32_t;
    static __device__ __forceinline__ float ld(const float *p) { return *p; }
    static __device__ __forceinline__ void st(float *p, float v) { *p = v; }
    static __device__ __forceinline__ raw_t ld_raw(const float *p) {
        return *reinterpret_cast<const uint32_t *>(p);
    }
    static __device__ __forceinline__ void st_raw(float *p, raw_t v) {
        *reinterpret_cast<uint32_t *>(p) = v;
    }
    static __device__ __forceinline__ float widen(raw_t v) { return __uint_as_float(v); }
    static __device__ __forceinline__ raw_t pack(float v) { return __float_as_uint(v); }
    static __device__ __forceinline__ raw_t bload(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                  uint32_t soff) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
    }
    static __device__ __forceinline__ void bstore(raw_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                  uint32_t soff) {
        __builtin_amdgcn_raw_buffer_store_b32(v, r, voff, soff, 0);
    }
    // element j of a run of staged elements held as 32-bit words
    static __device__ __forceinline__ float word_elem(const uint32_t *w, int j) {
        return __uint_as_float(w[j]);
    }
    // the run of NE elements at voff, one buffer load per element
    template <int NE>
    static __device__ __forceinline__ void bload_elems(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                       uint32_t *w) {
#pragma unroll
        for (int j = 0; j < NE; ++j) w[j] = __builtin_amdgcn_raw_buffer_load_b32(r, voff + 4 * j, 0, 0);
    }
};

// bf16 is carried as its 16 raw bits.
template <>
struct Elem<uint16_t> {
    using raw_t = uint16_t;
    static __device__ __forceinline__ float ld(const uint16_t *p) {
        return __uint_as_float(static_cast<uint32_t>(*p) << 16);
    }
    static __device__ __forceinline__ void st(uint16_t *p, float v) {
        *p = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));  // v_cvt_pk_bf16_f32, RNE
    }
    static __device__ __forceinline__ raw_t ld_raw(const uint16_t *p) { return *p; }
    static __device__ __forceinline__ void st_raw(uint16_t *p, raw_t v) { *p = v; }
    static __device__ __forceinline__ float widen(raw_t v) {
        return __uint_as_float(static_cast<uint32_t>(v) << 16);
    }
    static __device__ __forceinline__ raw_t pack(float v) {
        return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));  // v_cvt_pk_bf16_f32, RNE
    }
    static __device__ __forceinline__ raw_t bload(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                  uint32_t soff) {
        return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
    }
    static __device__ __forceinline__ void bstore(raw_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                  uint32_t soff) {
        __builtin_amdgcn_raw_buffer_store_b16(v, r, voff, soff, 0);
    }
    // element j of a run held as words: two bf16 per word, the first in the
    // low half (little-endian)
    static __device__ __forceinline__ float word_elem(const uint32_t *w, int j) {
        return __uint_as_float((j & 1) ? (w[j >> 1] & 0xFFFF0000u) : (w[j >> 1] << 16));
    }
    template <int NE>
    static __device__ __forceinline__ void bload_elems(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                       uint32_t *w) {
#pragma unroll
        for (int j = 0; j < NE; j += 2) {
            const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(r, voff + 2 * j, 0, 0);
            const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(r, voff + 2 * j + 2, 0, 0);
            w[j >> 1] = lo | (hi << 16);
        }
    }
};

// NW words at voff with 8- or 16-byte loads (voff and the resource base
// aligned to the load width).
template <int NW>
__device__ __forceinline__ void bload_words(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t *w) {
    static_assert(NW == 2 || NW % 4 == 0, "staging run width");
    if constexpr (NW == 2) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0);
        w[0] = v[0];
        w[1] = v[1];
    } else {
#pragma unroll
        for (int q = 0; q < NW / 4; ++q) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16 * q, 0, 0);
            w[4 * q] = v[0];
            w[4 * q + 1] = v[1];
            w[4 * q + 2] = v[2];
            w[4 * q + 3] = v[3];
        }
    }
}

// Raw buffer resource over [base, base + bytes) (word 3: the gfx9 raw-buffer
// format). Its bound applies to the per-lane offset only; the scalar offset
// added to it is not checked by the hardware.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0,
                                             static_cast<int>(bytes), 0x00020000);
}

// log(1 + e^v) = max(v, 0) + log(1 + e^-|v|), with base-2 hardware ops.
// max(v, 0) is taken as a signed-integer max of the bit patterns (one
// instruction; a float max would add a canonicalising one): positive floats
// order like their bits, every negative one has a negative pattern.
__device__ __forceinline__ float softplus(float v) {
    const float e = __builtin_amdgcn_exp2f(-fabsf(v) * kLog2e);
    const float l = __builtin_amdgcn_logf(1.0f + e);
    return fmaf(l, kLn2, __int_as_float(max(__float_as_int(v), 0)));
}

// Sum of y over the G lanes (adjacent, same quad) that share a channel.
template <int G>
__device__ __forceinline__ float group_sum(float y) {
    if constexpr (G >= 2) {
        const int o = __builtin_amdgcn_mov_dpp(__float_as_int(y), 0xB1, 0xF, 0xF, true);  // quad_perm 1,0,3,2
        y += __int_as_float(o);
    }
    if constexpr (G >= 4) {
        const int o = __builtin_amdgcn_mov_dpp(__float_as_int(y), 0x4E, 0xF, 0xF, true);  // quad_perm 2,3,0,1
        y += __int_as_float(o);
    }
    return y;
}

}  // namespace dev
}  // namespace r2l
