// Decode front end of the KDA block, gfx950: the depthwise causal conv1d
// update, SiLU, and L2 on q and k, fused into one kernel whose output is the
// q, k, v the recurrent core consumes (module page, pipeline line: conv1d +
// SiLU, then L2 on q and k only; decode fuses conv, SiLU and L2 in one kernel;
// the conv state keeps conv_kernel slots and is shifted left before
// convolving).  Per sequence, token and channel c of the conv_dim = 3 H 128
// channels (q | k | v):
//
//     slots <- (slots[1], ..., slots[K-1], x_c)        K = conv_kernel <= 4
//     y_c    = sum_k w[c][k] slots[k]                  slot K-1 the newest input
//     y_c    = y_c * sigmoid(y_c)
//     q, k  : y / sqrt(sum over the head's 128 channels of y^2 + l2_eps)
//
// qkv BF16 [B][T][conv_dim] (workspace page, qkv_proj), w BF16 [conv_dim][K]
// (config page, Glm5NextKdaWeights::conv), conv state FP32 [B][conv_dim][K]
// (config page, conv_state_elems), l2_eps applied inside the square root
// (config page, l2_eps).  Outputs q, k, v FP32 [B][T][H][128], the layout of
// kda_recurrent_step / kda_recurrent_k.
//
// One wave per (sequence, part, head) vector; lane l owns channels l and
// l + 64 and keeps their K slots and K weights in registers for all T rows, so
// the state is read and written once per call.  With that ownership every
// memory instruction of a wave covers one contiguous range (128 B of input,
// 256 B of output, 1 KiB of state or snapshot at K = 4); pairs of adjacent
// channels per lane, which leave every other 16 bytes of a range to a second
// instruction, were 13% slower on the 4-row walk with snapshots.  The next
// row's inputs are loaded while the current row is computed.  A q or k wave
// reduces sum y^2 in FP64 with shuffles alone (no barrier), which makes the
// scale exact for any finite input.  The arithmetic does not depend on T, so
// T rows in one call equal T one-row calls bit for bit.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kFeThreads = 256;             // four head vectors per workgroup, one per wave
constexpr int kFeVecs = kFeThreads / 64;

__device__ __forceinline__ float fe_bf16(uint32_t bits) { return __uint_as_float(bits << 16); }

// one wave per (sequence, part, head) vector; lane l owns channels l and l + 64
template <int K>
__global__ __launch_bounds__(kFeThreads) void front_end_kernel(const unsigned short* __restrict__ qkv,
                                                               const unsigned short* __restrict__ conv_w,
                                                               float* __restrict__ conv_state,
                                                               float* __restrict__ q_out, float* __restrict__ k_out,
                                                               float* __restrict__ v_out,
                                                               float* __restrict__ snaps, int n_snap, int batch,
                                                               int heads, int T, double eps)
{
    const int lane = threadIdx.x % 64;
    const long long gv = (long long)blockIdx.x * kFeVecs + threadIdx.x / 64;
    if (gv >= (long long)batch * 3 * heads) return;  // whole waves leave; no workgroup barrier below
    const int vec = (int)(gv % (3 * heads));
    const int b = (int)(gv / (3 * heads));
    const int part = vec / heads, h = vec % heads;
    const int C = 3 * heads * kD;
    const size_t cv = (size_t)vec * kD;  // first channel of the vector

    float w[2][K], s[2][K];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < K; ++i) w[m][i] = fe_bf16(conv_w[(cv + lane + 64 * m) * K + i]);
    float* const st = conv_state + ((size_t)b * C + cv) * K;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        float* const p = st + (size_t)(lane + 64 * m) * K;
        if constexpr (K == 4) {
            const float4 a = *reinterpret_cast<const float4*>(p);
            s[m][0] = a.x; s[m][1] = a.y; s[m][2] = a.z; s[m][3] = a.w;
        } else {
#pragma unroll
            for (int i = 0; i < K; ++i) s[m][i] = p[i];
        }
    }
    float* const out = part == 0 ? q_out : (part == 1 ? k_out : v_out);
    const unsigned short* const xp = qkv + (size_t)b * T * C + cv + lane;  // row 0, channel l
    unsigned short xn0 = xp[0], xn1 = xp[64];
    for (int t = 0; t < T; ++t) {
        const size_t row = (size_t)b * T + t;
        const unsigned short x0 = xn0, x1 = xn1;
        if (t + 1 < T) {
            xn0 = xp[(size_t)(t + 1) * C];
            xn1 = xp[(size_t)(t + 1) * C + 64];
        }
        float y[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
            for (int i = 0; i + 1 < K; ++i) s[m][i] = s[m][i + 1];
            s[m][K - 1] = fe_bf16(m == 0 ? x0 : x1);
            float a = w[m][0] * s[m][0];
#pragma unroll
            for (int i = 1; i < K; ++i) a = fmaf(w[m][i], s[m][i], a);
            y[m] = a / (1.0f + expf(-a));
        }
        if (part < 2) {
            double ss = (double)y[0] * y[0] + (double)y[1] * y[1];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) ss += __shfl_xor(ss, off);
            const double r = 1.0 / sqrt(ss + eps);
            y[0] = (float)(y[0] * r);
            y[1] = (float)(y[1] * r);
        }
        float* const o = out + (row * heads + h) * kD + lane;
        o[0] = y[0];
        o[64] = y[1];
        if (t < n_snap) {
            float* const sn = snaps + (((size_t)t * batch + b) * C + cv) * K;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                float* const p = sn + (size_t)(lane + 64 * m) * K;
                if constexpr (K == 4) *reinterpret_cast<float4*>(p) = make_float4(s[m][0], s[m][1], s[m][2], s[m][3]);
                else
#pragma unroll
                    for (int i = 0; i < K; ++i) p[i] = s[m][i];
            }
        }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        float* const p = st + (size_t)(lane + 64 * m) * K;
        if constexpr (K == 4) *reinterpret_cast<float4*>(p) = make_float4(s[m][0], s[m][1], s[m][2], s[m][3]);
        else
#pragma unroll
            for (int i = 0; i < K; ++i) p[i] = s[m][i];
    }
}

}  // namespace

int launch_front_end(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state, float* q, float* k, float* v,
                     float* snaps, int n_snap, int batch, int heads, int T, int conv_kernel, float l2_eps,
                     hipStream_t stream)
{
    const long long n_vec = (long long)batch * 3 * heads;
    const dim3 grid((unsigned)((n_vec + kFeVecs - 1) / kFeVecs)), block(kFeThreads);
    const auto* x = reinterpret_cast<const unsigned short*>(qkv);
    const auto* w = reinterpret_cast<const unsigned short*>(conv_w);
    const double eps = l2_eps;
    switch (conv_kernel) {
    case 1: hipLaunchKernelGGL(front_end_kernel<1>, grid, block, 0, stream, x, w, conv_state, q, k, v, snaps, n_snap, batch, heads, T, eps); break;
    case 2: hipLaunchKernelGGL(front_end_kernel<2>, grid, block, 0, stream, x, w, conv_state, q, k, v, snaps, n_snap, batch, heads, T, eps); break;
    case 3: hipLaunchKernelGGL(front_end_kernel<3>, grid, block, 0, stream, x, w, conv_state, q, k, v, snaps, n_snap, batch, heads, T, eps); break;
    case 4: hipLaunchKernelGGL(front_end_kernel<4>, grid, block, 0, stream, x, w, conv_state, q, k, v, snaps, n_snap, batch, heads, T, eps); break;
    default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kda
