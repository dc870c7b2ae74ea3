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

// One token: the new inputs x0, x1 (BF16) enter the newest slot, y = sum_k w[k] slot[k],
// y = y sigmoid(y); with l2 (a q or k wave, wave-uniform) the vector is scaled by
// 1 / sqrt(sum y^2 + eps), the sum formed in FP64 with shuffles over the whole wave.
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
        y[m] = a / (1.0f + expf(-a));
    }
    if (l2) {
        double ss = (double)y[0] * y[0] + (double)y[1] * y[1];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) ss += __shfl_xor(ss, off);
        const double r = 1.0 / sqrt(ss + eps);
        y[0] = (float)(y[0] * r);
        y[1] = (float)(y[1] * r);
    }
}

}  // namespace kda
