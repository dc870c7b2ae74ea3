// Per-lane pieces of the decode front end (depthwise causal conv1d update,
// SiLU, L2 on q and k), kept apart from the kernel so that any kernel that
// runs the front end computes the same bits.  A wave owns one 128-channel head
// vector of q, k or v; lane l owns channels l and l + 64.
#pragma once

#include "kda_common.h"

namespace kda {

// the K slots (conv state) and K weights of one lane's two channels
template <int K>
struct FeLane {
    float w[2][K], s[2][K];
};

// cv: first channel of the vector; st: conv state of that channel ([channel][K] floats)
template <int K>
__device__ __forceinline__ void fe_load(FeLane<K>& f, const unsigned short* __restrict__ conv_w, const float* st,
                                        size_t cv, int lane)
{
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < K; ++i) f.w[m][i] = bf16_to_f32(conv_w[(cv + lane + 64 * m) * K + i]);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const float* const p = st + (size_t)(lane + 64 * m) * K;
        if constexpr (K == 4) {
            const float4 a = *reinterpret_cast<const float4*>(p);
            f.s[m][0] = a.x; f.s[m][1] = a.y; f.s[m][2] = a.z; f.s[m][3] = a.w;
        } else {
#pragma unroll
            for (int i = 0; i < K; ++i) f.s[m][i] = p[i];
        }
    }
}

// the lane's slots to [channel][K] state or snapshot memory of the vector
template <int K>
__device__ __forceinline__ void fe_store(const FeLane<K>& f, float* st, int lane)
{
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        float* const p = st + (size_t)(lane + 64 * m) * K;
        if constexpr (K == 4) *reinterpret_cast<float4*>(p) = make_float4(f.s[m][0], f.s[m][1], f.s[m][2], f.s[m][3]);
        else
#pragma unroll
            for (int i = 0; i < K; ++i) p[i] = f.s[m][i];
    }
}

// One DPP lane move of a double (both 32-bit halves with the same control);
// lanes outside ROW_MASK get 0.  With every row enabled (the quad permutes and
// mirrors, which have a source for every lane) no old value is needed.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ double dpp_f64(double x)
{
    const unsigned long long u = (unsigned long long)__double_as_longlong(x);
    unsigned lo, hi;
    if constexpr (ROW_MASK == 0xf) {
        lo = (unsigned)__builtin_amdgcn_mov_dpp((int)(unsigned)u, CTRL, 0xf, 0xf, false);
        hi = (unsigned)__builtin_amdgcn_mov_dpp((int)(unsigned)(u >> 32), CTRL, 0xf, 0xf, false);
    } else {
        lo = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)u, CTRL, ROW_MASK, 0xf, false);
        hi = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)(u >> 32), CTRL, ROW_MASK, 0xf, false);
    }
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Sum of x over the 64 lanes of a wave, returned to every lane, in a fixed
// order: quads, eights, rows of 16 (DPP quad permutes and row mirrors), then
// the rows through the row broadcasts, the total landing in lane 63.
__device__ __forceinline__ double wave_sum_f64(double x)
{
    x += dpp_f64<0xB1>(x);        // quad_perm [1, 0, 3, 2]
    x += dpp_f64<0x4E>(x);        // quad_perm [2, 3, 0, 1]
    x += dpp_f64<0x141>(x);       // row_half_mirror
    x += dpp_f64<0x140>(x);       // row_mirror
    x += dpp_f64<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
    x += dpp_f64<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
    const unsigned long long u = (unsigned long long)__double_as_longlong(x);
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)u, 63);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(u >> 32), 63);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// One token: the new inputs x0, x1 (BF16) enter the newest slot, y = sum_k w[k] slot[k],
// y = y sigmoid(y); with l2 (a q or k wave, wave-uniform) the vector is scaled by
// 1 / sqrt(sum y^2 + eps), the sum formed in FP64 over the whole wave.  The
// sigmoid is 1 / (1 + 2^(-y log2 e)) from the hardware exp2 and reciprocal
// (within a few units of 2^-24 of the exact value), and the scale is the
// hardware FP64 reciprocal square root refined by one Newton step (far below
// FP32 resolution), which keeps the row short: the prefill form runs this body
// for every token of a prefill.
template <int K>
__device__ __forceinline__ void fe_row(FeLane<K>& f, unsigned short x0, unsigned short x1, bool l2, double eps,
                                       float (&y)[2])
{
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int i = 0; i + 1 < K; ++i) f.s[m][i] = f.s[m][i + 1];
        f.s[m][K - 1] = bf16_to_f32(m == 0 ? x0 : x1);
        float a = f.w[m][0] * f.s[m][0];
#pragma unroll
        for (int i = 1; i < K; ++i) a = fmaf(f.w[m][i], f.s[m][i], a);
        y[m] = a * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504f * a));
    }
    if (l2) {
        const double x = wave_sum_f64((double)y[0] * y[0] + (double)y[1] * y[1]) + eps;
        double r = __builtin_amdgcn_rsq(x);
        r = r * (1.5 - 0.5 * (x * r) * r);  // one Newton step
        y[0] = (float)(y[0] * r);
        y[1] = (float)(y[1] * r);
    }
}

}  // namespace kda
