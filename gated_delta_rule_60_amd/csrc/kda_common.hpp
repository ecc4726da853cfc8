// kda_common.hpp -- device helpers shared by the libkda kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kda.h"

namespace kda {

// ---------------------------------------------------------------- forget gate
// g = g_min * sigmoid(exp(A) * z) = g_min / (1 + 2^(-rate * z)) with rate = exp(A) * log2(e),
// one per (head, key channel).  Hardware exp2 and reciprocal (about 1 ulp each) keep g within
// 1e-6 of the exact value over g in [-5, 0]; saturation gives g_min and -0.  The separate gate
// kernel and the chunk kernel's fused gate both call these, with contraction off, so the two
// paths produce the same bits of g.
__device__ __forceinline__ float gate_rate(float A) {
#pragma clang fp contract(off)
    return expf(A) * 1.4426950408889634f;
}
__device__ __forceinline__ float gate_log_decay(float rate, float z, float g_min) {
#pragma clang fp contract(off)
    const float e = __builtin_amdgcn_exp2f(-(rate * z));
    return g_min * __builtin_amdgcn_rcpf(1.0f + e);
}

// ---------------------------------------------------------------- bf16 <-> fp32 (bit level)
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return static_cast<uint16_t>((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Element i of a buffer stored as KDA_F32 or KDA_BF16, as fp32.
template <int DT>
__device__ __forceinline__ float load_as_f32(const void* p, int64_t i) {
    if constexpr (DT == KDA_F32) return static_cast<const float*>(p)[i];
    else return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
}

template <int DT>
__device__ __forceinline__ void store_from_f32(void* p, int64_t i, float x) {
    if constexpr (DT == KDA_F32) static_cast<float*>(p)[i] = x;
    else static_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(x);
}

// Four consecutive elements starting at i (i % 4 == 0, buffer 8/16-byte aligned).
template <int DT>
__device__ __forceinline__ float4 load4_as_f32(const void* p, int64_t i) {
    if constexpr (DT == KDA_F32) {
        return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    } else {
        uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
        return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                           __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
    }
}

template <int DT>
__device__ __forceinline__ void store4_from_f32(void* p, int64_t i, float4 x) {
    if constexpr (DT == KDA_F32) {
        *reinterpret_cast<float4*>(static_cast<float*>(p) + i) = x;
    } else {
        uint2 w;
        w.x = static_cast<uint32_t>(f32_to_bf16_bits(x.x)) | (static_cast<uint32_t>(f32_to_bf16_bits(x.y)) << 16);
        w.y = static_cast<uint32_t>(f32_to_bf16_bits(x.z)) | (static_cast<uint32_t>(f32_to_bf16_bits(x.w)) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + i) = w;
    }
}

}  // namespace kda
