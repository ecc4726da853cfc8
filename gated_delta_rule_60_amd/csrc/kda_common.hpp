// kda_common.hpp -- device helpers shared by the libkda kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kda.h"

namespace kda {

// ---------------------------------------------------------------- forget gate
// g = g_min * sigmoid(exp(A) * z) = g_min / (1 + 2^(-rate * z)) with rate = exp(A) * log2(e),
// one per (head, key channel), held as an unevaluated pair hi + lo of floats formed from its fp64
// value.  The argument rate * z is carried the same way: the rounded product p, and the rest (the
// product's rounding error and lo * z, at most 2^-23 |p|) by fma.  e = 2^-p comes from the hardware
// exp2 (exact argument, 1 ulp), and 1 + 2^-(p + rest) = d + de exactly up to second order in rest:
// d = 1 + e rounded, de its rounding error (Fast2Sum) less e * rest * ln 2.  g_min / (d + de) is
// the rounded quotient corrected once by its residual.  Error budget: e 1 ulp, the quotient 0.5
// ulp, so g lands within 1.5 ulp of the exact value while |rate * z| <= 126; beyond that p is
// clamped and g is g_min on one side and below 2^-123 in magnitude on the other.  The separate
// gate kernel and the prefill kernels' fused gate call these alike, so the two paths produce the
// same bits.
struct GateRate {
    float hi, lo;
};
__device__ __forceinline__ GateRate gate_rate(float A) {
    const double r = exp(static_cast<double>(A)) * 1.4426950408889634074;
    const float hi = static_cast<float>(r);
    return {hi, static_cast<float>(r - static_cast<double>(hi))};
}
__device__ __forceinline__ float gate_log_decay(float rate_hi, float rate_lo, float z, float g_min) {
#pragma clang fp contract(off)
    const float p = rate_hi * z;
    const float rest = __builtin_fmaf(rate_lo, z, __builtin_fmaf(rate_hi, z, -p));   // rate * z - p
    const float e = __builtin_amdgcn_exp2f(-__builtin_amdgcn_fmed3f(p, -126.0f, 126.0f));
    const float d = 1.0f + e;
    const float big = __builtin_fmaxf(e, 1.0f), small = __builtin_fminf(e, 1.0f);
    const float de = __builtin_fmaf(-e, rest * 0.69314718055994531f, (big - d) + small);
    const float r0 = __builtin_amdgcn_rcpf(d);
    const float q0 = g_min * r0;
    const float res = __builtin_fmaf(-q0, de, __builtin_fmaf(-q0, d, g_min));
    return __builtin_fmaf(res, r0, q0);
}
__device__ __forceinline__ float gate_log_decay(GateRate rate, float z, float g_min) {
    return gate_log_decay(rate.hi, rate.lo, z, g_min);
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
