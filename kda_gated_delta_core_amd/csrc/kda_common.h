// Shared device-side helpers of the KDA HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kD = 128;  // head_dim, fixed by the method's geometry check

typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }

// BF16 is the top half of an IEEE binary32: widening is exact
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// binary32 -> BF16, round to nearest even; a NaN stays a (quiet) NaN of the same sign
__device__ __forceinline__ uint32_t f32_to_bf16(float x)
{
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// kda_gate and the beta sigmoid inside a core kernel's loads (workspace page, fields gate and g_raw:
// the gate is the bounded log-decay kda_gate makes from g_raw; field beta: a sigmoid of its logit;
// config page, dt_bias per (head, channel), a_log per head, gate_lower_bound).  The pages print no
// gate formula; the reading implemented is
//     gate = lower * sigmoid(exp(a_log[h]) * (g_raw + dt_bias[h][i])),   beta = sigmoid(beta logit)
// evaluated in FP32 with the hardware exp2 and reciprocal (each within about one unit in the last
// place): a few units of 2^-24 on the gate, far inside the core's tolerance.
struct GateParams {
    const unsigned short* g_raw;  // [rows][heads][128] BF16, in the gate's own layout
    const float* dt_bias;         // [heads][128]
    const float* a_log;           // [heads]
    float lower;                  // gate_lower_bound, <= 0
};
__device__ __forceinline__ float sigmoid_f32(float z)
{
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}
// 1 / sqrt(x) for x > 0 in FP64: the hardware estimate and one Newton step
__device__ __forceinline__ double norm_rsqrt(double x)
{
    const double r = __builtin_amdgcn_rsq(x);
    return r * (1.5 - 0.5 * (x * r) * r);
}
__device__ __forceinline__ float kda_gate_f32(float g_raw, float dt_bias, float rate, float lower)
{
    return lower * sigmoid_f32(rate * (g_raw + dt_bias));
}

// Raw buffer access: a descriptor (base address, size in bytes) held in scalar
// registers plus a 32-bit per-lane byte offset and a wave-uniform byte offset.
// Lane offsets computed once outside a loop then need no per-iteration vector
// address registers.  Offsets at or past the size read zeros and drop stores.
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr int kRawBufferWord3 = 0x00020000;  // gfx9 raw (untyped) buffer, 32-bit elements
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawBufferWord3);
}
__device__ __forceinline__ float4 buf_ld4(rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ float buf_ld1(rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ void buf_st4(rsrc_t r, int voff, int soff, float4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v), r, voff,
                                           soff, 0);
}
__device__ __forceinline__ void buf_st1(rsrc_t r, int voff, int soff, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, voff, soff, 0);
}

// One 16x16x4 FP32 MFMA step:  acc[16x16] += A[16x4] * B[4x16].
// Lane l supplies A[l % 16][l / 16] in `a` and B[l / 16][l % 16] in `b`;
// acc element r of lane l is C[4 * (l / 16) + r][l % 16].
__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 acc)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

}  // namespace kda
