// Sigmoid-gated RMSNorm of the core's output, gfx950: the step that follows
// the KDA core in the block (module page, pipeline line: the core's output
// goes through a sigmoid-gated RMSNorm with the o_norm weight and the output
// gate g_b(g_a(h)), then to o_proj; the gate passes through a logistic sigmoid, not a SiLU).
// Per (token, head), over the 128 value channels j:
//
//     y_j = core_j / sqrt(mean_i core_i^2 + eps) * w_j * sigmoid(g_j)
//
// core FP32 (the core's own output), g and y BF16 [T, heads * 128] (workspace
// page, fields out_gate and o_norm_out), w BF16 [128] shared by the heads
// (config page, Glm5NextKdaWeights::o_norm), eps = rms_norm_eps (config page).
//
// HBM-bound: 512 + 256 + 256 bytes per (token, head) and a handful of flops.
// 16 lanes own a (token, head) vector, 8 channels each, so every access is a
// full 16-byte one (two for the FP32 core) and coalesced; each 16-lane group
// takes two vectors and issues all their loads before any arithmetic.  The
// sum of squares and the scale 1 / sqrt(mean + eps) are formed in FP64 (each
// FP32 square is exact there, the 128-term sum cannot overflow or flush), so
// every finite core gives an accurate scale; the rest is FP32 and the result
// is rounded to BF16 to nearest even.  The scale is the hardware FP64
// reciprocal square root refined by one Newton step, the sigmoid the hardware
// exp2 and reciprocal (within a few units of 2^-24): with the IEEE divisions
// and the accurate expf of each element the kernel spent as long in its
// arithmetic as in its memory traffic.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kNormThreads = 256;
constexpr int kLanes = 16;                               // lanes per (token, head) vector
constexpr int kGroups = kNormThreads / kLanes;           // vector groups per block
constexpr int kGroupVecs = 2;                            // vectors per group
constexpr int kVecPerBlock = kGroups * kGroupVecs;


typedef unsigned u32x4 __attribute__((ext_vector_type(4)));  // 8 BF16 values

// core as float4s (two per lane and vector), gate / weight / out as 8 BF16 per 16 bytes
__global__ __launch_bounds__(kNormThreads) void gated_rmsnorm_kernel(const floatx4* __restrict__ core,
                                                                     const u32x4* __restrict__ gate,
                                                                     const u32x4* __restrict__ weight,
                                                                     u32x4* __restrict__ out, long long n_vec,
                                                                     double eps)
{
    // group q of the block takes vectors v0 and v0 + kGroups, so each load
    // instruction of the block covers kGroups consecutive vectors
    const long long v0 = (long long)blockIdx.x * kVecPerBlock + threadIdx.x / kLanes;
    const int j8 = threadIdx.x % kLanes;  // channels 8 j8 .. 8 j8 + 7
    const u32x4 w = weight[j8];
    floatx4 c[kGroupVecs][2];
    u32x4 g[kGroupVecs];
#pragma unroll
    for (int i = 0; i < kGroupVecs; ++i) {
        const long long vec = v0 + kGroups * i;
        const size_t e = (size_t)(vec < n_vec ? vec : 0) * kLanes + j8;  // 8-channel unit
        c[i][0] = __builtin_nontemporal_load(core + 2 * e);
        c[i][1] = __builtin_nontemporal_load(core + 2 * e + 1);
        g[i] = __builtin_nontemporal_load(gate + e);
    }
    float w8[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        w8[2 * k] = bf16_to_f32(w[k] & 0xffffu);
        w8[2 * k + 1] = bf16_to_f32(w[k] >> 16);
    }
#pragma unroll
    for (int i = 0; i < kGroupVecs; ++i) {
        float x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = c[i][k / 4][k % 4];
        double ss = 0.0;
#pragma unroll
        for (int k = 0; k < 8; ++k) ss += (double)x[k] * x[k];
#pragma unroll
        for (int off = 1; off < kLanes; off <<= 1) ss += __shfl_xor(ss, off, kLanes);
        const double r = norm_rsqrt(ss * (1.0 / kD) + eps);
        u32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float ya = (float)(x[2 * k] * r) * w8[2 * k] * sigmoid_f32(bf16_to_f32(g[i][k] & 0xffffu));
            const float yb = (float)(x[2 * k + 1] * r) * w8[2 * k + 1] * sigmoid_f32(bf16_to_f32(g[i][k] >> 16));
            o[k] = f32_to_bf16(ya) | (f32_to_bf16(yb) << 16);
        }
        const long long vec = v0 + kGroups * i;
        if (vec < n_vec) __builtin_nontemporal_store(o, out + (size_t)vec * kLanes + j8);
    }
}

}  // namespace

int launch_gated_rmsnorm(const float* core, const uint16_t* gate, const uint16_t* weight, uint16_t* out,
                         long long n_vec, float eps, hipStream_t stream)
{
    const long long grid = (n_vec + kVecPerBlock - 1) / kVecPerBlock;
    hipLaunchKernelGGL(gated_rmsnorm_kernel, dim3((unsigned)grid), dim3(kNormThreads), 0, stream,
                       reinterpret_cast<const floatx4*>(core), reinterpret_cast<const u32x4*>(gate),
                       reinterpret_cast<const u32x4*>(weight), reinterpret_cast<u32x4*>(out), n_vec, (double)eps);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kda
