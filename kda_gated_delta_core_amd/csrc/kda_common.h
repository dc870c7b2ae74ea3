// Shared device-side helpers of the KDA HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kD = 128;  // head_dim, fixed by the method's geometry check

typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }

// One 16x16x4 FP32 MFMA step:  acc[16x16] += A[16x4] * B[4x16].
// Lane l supplies A[l % 16][l / 16] in `a` and B[l / 16][l % 16] in `b`;
// acc element r of lane l is C[4 * (l / 16) + r][l % 16].
__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 acc)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

}  // namespace kda
