// Decode front end of the KDA block, gfx950: the depthwise causal conv1d
// update, SiLU, and L2 on q and k, fused into one kernel whose output is the
// q, k, v the recurrent core consumes (module page, pipeline line: conv1d and
// SiLU on q, k, v, then L2 on q and k alone; on that page the decode form does
// all three steps in a single kernel, and the conv state holds conv_kernel
// slots that shift by one before each convolution).  Per sequence, token and channel c of the conv_dim = 3 H 128
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
// (config page, l2_eps).  Outputs either q, k, v FP32 [B][T][H][128], the
// layout of kda_recurrent_step / kda_recurrent_k, or BF16 conv_out in the
// input's own [B][T][conv_dim] layout (workspace page, conv_out: BF16, L2
// already applied on the decode path), rounded to nearest even from the same
// FP32 values, which kda_recurrent_step_bf16 / kda_recurrent_k_bf16 read.
//
// One wave per (sequence, part, head) vector; lane l owns channels l and
// l + 64 and keeps their K slots and K weights in registers for all T rows, so
// the state is read and written once per call.  With that ownership every
// memory instruction of a wave covers one contiguous range (128 B of input,
// 256 B of output, 1 KiB of state or snapshot at K = 4); pairs of adjacent
// channels per lane, which leave every other 16 bytes of a range to a second
// instruction, were 13% slower on the 4-row walk with snapshots.  The next
// row's inputs are loaded while the current row is computed.  A q or k wave
// reduces sum y^2 in FP64 with DPP lane moves alone (no barrier), so the sum
// neither overflows nor flushes for any finite input.  The arithmetic does not
// depend on T, so T rows in one call equal T one-row calls bit for bit.
#include "kda_front_end.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kFeThreads = 256;             // four head vectors per workgroup, one per wave
constexpr int kFeVecs = kFeThreads / 64;

// one wave per (sequence, part, head) vector; lane l owns channels l and l + 64
template <int K, bool kBf16Out>
__global__ __launch_bounds__(kFeThreads) void front_end_kernel(const unsigned short* __restrict__ qkv,
                                                               const unsigned short* __restrict__ conv_w,
                                                               float* __restrict__ conv_state,
                                                               float* __restrict__ q_out, float* __restrict__ k_out,
                                                               float* __restrict__ v_out,
                                                               unsigned short* __restrict__ conv_out,
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

    FeLane<K> f;
    float* const st = conv_state + ((size_t)b * C + cv) * K;
    fe_load(f, conv_w, st, cv, lane);
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
        fe_row(f, x0, x1, part < 2, eps, y);
        if constexpr (kBf16Out) {
            unsigned short* const o = conv_out + (row * 3 * heads + vec) * kD + lane;  // [b][t][part][h][.]
            o[0] = (unsigned short)f32_to_bf16(y[0]);
            o[64] = (unsigned short)f32_to_bf16(y[1]);
        } else {
            float* const o = out + (row * heads + h) * kD + lane;
            o[0] = y[0];
            o[64] = y[1];
        }
        if (t < n_snap) fe_store(f, snaps + (((size_t)t * batch + b) * C + cv) * K, lane);
    }
    fe_store(f, st, lane);
}

template <int K>
void launch_fe(dim3 grid, const unsigned short* x, const unsigned short* w, float* conv_state, float* q, float* k,
               float* v, unsigned short* conv_out, float* snaps, int n_snap, int batch, int heads, int T, double eps,
               hipStream_t stream)
{
    if (conv_out)
        hipLaunchKernelGGL((front_end_kernel<K, true>), grid, dim3(kFeThreads), 0, stream, x, w, conv_state, nullptr,
                           nullptr, nullptr, conv_out, snaps, n_snap, batch, heads, T, eps);
    else
        hipLaunchKernelGGL((front_end_kernel<K, false>), grid, dim3(kFeThreads), 0, stream, x, w, conv_state, q, k, v,
                           nullptr, snaps, n_snap, batch, heads, T, eps);
}

// Prefill form: the same computation over a whole prefill, parallel over
// tokens.  One wave per (sequence, strip of kFeStrip tokens, part, head)
// vector: its K slots start as the inputs of the K times before the strip (the
// conv state's slot K + time for times before the call), then it walks the
// strip's rows with the decode form's per-row body, so every row gets the bits
// the decode form walking all T rows gives it.  Outputs go to the chunk-padded
// [B][t_pad][H][128] rows of kda_chunk_prefill; rows >= T are not written.  The
// conv state is left alone here (earlier strips read it) and advanced by
// prefill_conv_state_kernel afterwards.
constexpr int kFeStrip = 32;

template <int K>
__global__ __launch_bounds__(kFeThreads) void prefill_front_end_kernel(const unsigned short* __restrict__ qkv,
                                                                       const unsigned short* __restrict__ conv_w,
                                                                       const float* __restrict__ conv_state,
                                                                       float* __restrict__ q_out,
                                                                       float* __restrict__ k_out,
                                                                       float* __restrict__ v_out, int batch,
                                                                       int heads, int T, int t_pad, int n_strips,
                                                                       double eps)
{
    const int lane = threadIdx.x % 64;
    const long long gv = (long long)blockIdx.x * kFeVecs + threadIdx.x / 64;
    const int n_part = 3 * heads;
    if (gv >= (long long)batch * n_strips * n_part) return;  // whole waves leave; no workgroup barrier below
    const int vec = (int)(gv % n_part);
    const long long bs = gv / n_part;
    const int strip = (int)(bs % n_strips), b = (int)(bs / n_strips);
    const int part = vec / heads, h = vec % heads;
    const int C = 3 * heads * kD;
    const size_t cv = (size_t)vec * kD;  // first channel of the vector
    const int t0 = strip * kFeStrip, t1 = min(T, t0 + kFeStrip);

    FeLane<K> f;
    const unsigned short* const xp = qkv + (size_t)b * T * C + cv + lane;  // row 0, channel l
    const float* const st = conv_state + ((size_t)b * C + cv) * K;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int i = 0; i < K; ++i) {
            f.w[m][i] = bf16_to_f32(conv_w[(cv + lane + 64 * m) * K + i]);
            const int tau = t0 - K + i;  // the time slot i holds before row t0
            f.s[m][i] = tau >= 0 ? bf16_to_f32(xp[(size_t)tau * C + 64 * m]) : st[(size_t)(lane + 64 * m) * K + K + tau];
        }
    }
    float* const out = part == 0 ? q_out : (part == 1 ? k_out : v_out);
    unsigned short xn0 = xp[(size_t)t0 * C], xn1 = xp[(size_t)t0 * C + 64];
    for (int t = t0; t < t1; ++t) {
        const unsigned short x0 = xn0, x1 = xn1;
        if (t + 1 < t1) {
            xn0 = xp[(size_t)(t + 1) * C];
            xn1 = xp[(size_t)(t + 1) * C + 64];
        }
        float y[2];
        fe_row(f, x0, x1, part < 2, eps, y);
        float* const o = out + (((size_t)b * t_pad + t) * heads + h) * kD + lane;
        o[0] = y[0];
        o[64] = y[1];
    }
}

// After the prefill: the conv state of every (sequence, channel) becomes the
// inputs of the last K times (from the old state for times before the call).
// One thread per (sequence, channel); it reads its old slots before writing.
template <int K>
__global__ __launch_bounds__(256) void prefill_conv_state_kernel(const unsigned short* __restrict__ qkv,
                                                                 float* __restrict__ conv_state, int batch, int C,
                                                                 int T)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;  // b * C + channel
    if (i >= (long long)batch * C) return;
    const long long b = i / C, c = i % C;
    float* const st = conv_state + (size_t)i * K;
    float old[K];
#pragma unroll
    for (int j = 0; j < K; ++j) old[j] = st[j];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int tau = T - K + j;  // before the call when < 0: old slot K + tau
        float keep = old[0];
#pragma unroll
        for (int u = 1; u < K; ++u) keep = (u == K + tau) ? old[u] : keep;
        st[j] = tau >= 0 ? bf16_to_f32(qkv[((size_t)b * T + tau) * C + c]) : keep;
    }
}

// Varlen form: sequences packed back to back (tokens cu[s] .. cu[s + 1] - 1 of
// qkv [total][conv_dim]), each with its own conv state [n][conv_dim][K];
// outputs [total][H][128], the inputs of kda_chunk_prefill_varlen.  Waves take
// fixed strips of kFeStrip packed tokens; a strip may cross sequences, and at
// the first row of a sequence the slots are re-seeded from that sequence's
// conv state, so no window reaches across a boundary.  The offsets are read
// clamped to [0, total], which keeps every access inside the buffers whatever
// they hold (offsets that are not non-decreasing give unspecified values).
__device__ __forceinline__ int fe_cu(const int* cu, int s, int total)
{
    const int c = cu[s];
    return c < 0 ? 0 : (c > total ? total : c);
}

template <int K>
__global__ __launch_bounds__(kFeThreads) void prefill_front_end_varlen_kernel(
    const unsigned short* __restrict__ qkv, const unsigned short* __restrict__ conv_w,
    const float* __restrict__ conv_state, float* __restrict__ q_out, float* __restrict__ k_out,
    float* __restrict__ v_out, const int* __restrict__ cu, int n_seqs, int heads, int total, int n_strips, double eps)
{
    const int lane = threadIdx.x % 64;
    const long long gv = (long long)blockIdx.x * kFeVecs + threadIdx.x / 64;
    const int n_part = 3 * heads;
    if (gv >= (long long)n_strips * n_part) return;  // whole waves leave; no workgroup barrier below
    const int vec = (int)(gv % n_part), strip = (int)(gv / n_part);
    const int part = vec / heads, h = vec % heads;
    const int C = 3 * heads * kD;
    const size_t cv = (size_t)vec * kD;
    // rows past the last sequence (cu[n] .. total - 1) belong to none and are not written
    const int t0 = strip * kFeStrip, t1 = min(min(total, t0 + kFeStrip), fe_cu(cu, n_seqs, total));
    if (t0 >= t1) return;
    // the sequence of row t0: the last s with cu[s] <= t0 (wave-uniform, scalar loads)
    int lo = 0, hi = n_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (fe_cu(cu, mid, total) <= t0) lo = mid;
        else hi = mid - 1;
    }
    int sq = lo, nxt = fe_cu(cu, sq + 1, total);  // the row where the sequence after sq begins
    FeLane<K> f;
    const unsigned short* const xp = qkv + cv + lane;  // row 0, channel l
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < K; ++i) f.w[m][i] = bf16_to_f32(conv_w[(cv + lane + 64 * m) * K + i]);
    auto seed = [&](int s, int t) {  // slots before row t of sequence s
        // its first row; at most t, so the state slot below stays in [0, K) whatever the offsets hold
        const int start = min(fe_cu(cu, s, total), t);
        const float* const st = conv_state + ((size_t)s * C + cv) * K;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int i = 0; i < K; ++i) {
                const int tau = t - K + i;  // packed row slot i holds; before the sequence: state slot
                f.s[m][i] = tau >= start ? bf16_to_f32(xp[(size_t)tau * C + 64 * m])
                                         : st[(size_t)(lane + 64 * m) * K + K + (tau - start)];
            }
    };
    seed(sq, t0);
    float* const out = part == 0 ? q_out : (part == 1 ? k_out : v_out);
    unsigned short xn0 = xp[(size_t)t0 * C], xn1 = xp[(size_t)t0 * C + 64];
    for (int t = t0; t < t1; ++t) {
        const unsigned short x0 = xn0, x1 = xn1;
        if (t + 1 < t1) {
            xn0 = xp[(size_t)(t + 1) * C];
            xn1 = xp[(size_t)(t + 1) * C + 64];
        }
        if (t >= nxt) {  // row t opens a later sequence (skipping empty ones): fresh slots from its state
            while (sq + 1 < n_seqs && fe_cu(cu, sq + 1, total) <= t) ++sq;
            nxt = sq + 1 < n_seqs ? fe_cu(cu, sq + 1, total) : total;
            seed(sq, t);
        }
        float y[2];
        fe_row(f, x0, x1, part < 2, eps, y);
        float* const o = out + ((size_t)t * heads + h) * kD + lane;
        o[0] = y[0];
        o[64] = y[1];
    }
}

// After a varlen prefill: each sequence's conv state becomes the inputs of its
// last K tokens (old slots for times before its start).  One thread per
// (sequence, channel); an empty sequence keeps its state.
template <int K>
__global__ __launch_bounds__(256) void prefill_conv_state_varlen_kernel(const unsigned short* __restrict__ qkv,
                                                                        float* __restrict__ conv_state,
                                                                        const int* __restrict__ cu, int n_seqs,
                                                                        int C, int total)
{
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;  // s * C + channel
    if (i >= (long long)n_seqs * C) return;
    const int s = (int)(i / C), c = (int)(i % C);
    const int a = fe_cu(cu, s, total), e = max(a, fe_cu(cu, s + 1, total));
    const int len = e - a;
    float* const st = conv_state + (size_t)i * K;
    float old[K];
#pragma unroll
    for (int j = 0; j < K; ++j) old[j] = st[j];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int tau = len - K + j;  // local time; before the sequence when < 0: old slot K + tau
        float keep = old[0];
#pragma unroll
        for (int u = 1; u < K; ++u) keep = (u == K + tau) ? old[u] : keep;
        st[j] = tau >= 0 ? bf16_to_f32(qkv[(size_t)(a + tau) * C + c]) : keep;
    }
}

template <int K>
void launch_prefill_fe_varlen(const unsigned short* x, const unsigned short* w, float* conv_state, float* q, float* k,
                              float* v, const int* cu, int n_seqs, int heads, int total, double eps,
                              hipStream_t stream)
{
    const int n_strips = (total + kFeStrip - 1) / kFeStrip;
    const long long n_vec = (long long)n_strips * 3 * heads;
    hipLaunchKernelGGL(prefill_front_end_varlen_kernel<K>, dim3((unsigned)((n_vec + kFeVecs - 1) / kFeVecs)),
                       dim3(kFeThreads), 0, stream, x, w, conv_state, q, k, v, cu, n_seqs, heads, total, n_strips,
                       eps);
    const int C = 3 * heads * kD;
    const long long n_ch = (long long)n_seqs * C;
    hipLaunchKernelGGL(prefill_conv_state_varlen_kernel<K>, dim3((unsigned)((n_ch + 255) / 256)), dim3(256), 0,
                       stream, x, conv_state, cu, n_seqs, C, total);
}

template <int K>
void launch_prefill_fe(const unsigned short* x, const unsigned short* w, float* conv_state, float* q, float* k,
                       float* v, int batch, int heads, int T, int t_pad, double eps, hipStream_t stream)
{
    const int n_strips = (T + kFeStrip - 1) / kFeStrip;
    const long long n_vec = (long long)batch * n_strips * 3 * heads;
    hipLaunchKernelGGL(prefill_front_end_kernel<K>, dim3((unsigned)((n_vec + kFeVecs - 1) / kFeVecs)),
                       dim3(kFeThreads), 0, stream, x, w, conv_state, q, k, v, batch, heads, T, t_pad, n_strips, eps);
    const int C = 3 * heads * kD;
    const long long n_ch = (long long)batch * C;
    hipLaunchKernelGGL(prefill_conv_state_kernel<K>, dim3((unsigned)((n_ch + 255) / 256)), dim3(256), 0, stream, x,
                       conv_state, batch, C, T);
}

}  // namespace

int launch_prefill_front_end(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state, float* q, float* k,
                             float* v, int batch, int heads, int T, int t_pad, int conv_kernel, float l2_eps,
                             hipStream_t stream)
{
    const auto* x = reinterpret_cast<const unsigned short*>(qkv);
    const auto* w = reinterpret_cast<const unsigned short*>(conv_w);
    const double eps = l2_eps;
    switch (conv_kernel) {
    case 1: launch_prefill_fe<1>(x, w, conv_state, q, k, v, batch, heads, T, t_pad, eps, stream); break;
    case 2: launch_prefill_fe<2>(x, w, conv_state, q, k, v, batch, heads, T, t_pad, eps, stream); break;
    case 3: launch_prefill_fe<3>(x, w, conv_state, q, k, v, batch, heads, T, t_pad, eps, stream); break;
    case 4: launch_prefill_fe<4>(x, w, conv_state, q, k, v, batch, heads, T, t_pad, eps, stream); break;
    default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_conv_state_advance(const uint16_t* qkv, float* conv_state, int batch, int heads, int T, int conv_kernel,
                              hipStream_t stream)
{
    const auto* x = reinterpret_cast<const unsigned short*>(qkv);
    const int C = 3 * heads * kD;
    const dim3 grid((unsigned)(((long long)batch * C + 255) / 256));
    switch (conv_kernel) {
    case 1: hipLaunchKernelGGL(prefill_conv_state_kernel<1>, grid, dim3(256), 0, stream, x, conv_state, batch, C, T); break;
    case 2: hipLaunchKernelGGL(prefill_conv_state_kernel<2>, grid, dim3(256), 0, stream, x, conv_state, batch, C, T); break;
    case 3: hipLaunchKernelGGL(prefill_conv_state_kernel<3>, grid, dim3(256), 0, stream, x, conv_state, batch, C, T); break;
    case 4: hipLaunchKernelGGL(prefill_conv_state_kernel<4>, grid, dim3(256), 0, stream, x, conv_state, batch, C, T); break;
    default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_conv_state_advance_varlen(const uint16_t* qkv, float* conv_state, const int* cu_seqlens, int n_seqs,
                                     int heads, int total, int conv_kernel, hipStream_t stream)
{
    const auto* x = reinterpret_cast<const unsigned short*>(qkv);
    const int C = 3 * heads * kD;
    const dim3 grid((unsigned)(((long long)n_seqs * C + 255) / 256));
    switch (conv_kernel) {
    case 1: hipLaunchKernelGGL(prefill_conv_state_varlen_kernel<1>, grid, dim3(256), 0, stream, x, conv_state, cu_seqlens, n_seqs, C, total); break;
    case 2: hipLaunchKernelGGL(prefill_conv_state_varlen_kernel<2>, grid, dim3(256), 0, stream, x, conv_state, cu_seqlens, n_seqs, C, total); break;
    case 3: hipLaunchKernelGGL(prefill_conv_state_varlen_kernel<3>, grid, dim3(256), 0, stream, x, conv_state, cu_seqlens, n_seqs, C, total); break;
    case 4: hipLaunchKernelGGL(prefill_conv_state_varlen_kernel<4>, grid, dim3(256), 0, stream, x, conv_state, cu_seqlens, n_seqs, C, total); break;
    default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_prefill_front_end_varlen(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state, float* q,
                                    float* k, float* v, const int* cu_seqlens, int n_seqs, int heads, int total,
                                    int conv_kernel, float l2_eps, hipStream_t stream)
{
    const auto* x = reinterpret_cast<const unsigned short*>(qkv);
    const auto* w = reinterpret_cast<const unsigned short*>(conv_w);
    const double eps = l2_eps;
    switch (conv_kernel) {
    case 1: launch_prefill_fe_varlen<1>(x, w, conv_state, q, k, v, cu_seqlens, n_seqs, heads, total, eps, stream); break;
    case 2: launch_prefill_fe_varlen<2>(x, w, conv_state, q, k, v, cu_seqlens, n_seqs, heads, total, eps, stream); break;
    case 3: launch_prefill_fe_varlen<3>(x, w, conv_state, q, k, v, cu_seqlens, n_seqs, heads, total, eps, stream); break;
    case 4: launch_prefill_fe_varlen<4>(x, w, conv_state, q, k, v, cu_seqlens, n_seqs, heads, total, eps, stream); break;
    default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_front_end(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state, float* q, float* k, float* v,
                     uint16_t* conv_out, float* snaps, int n_snap, int batch, int heads, int T, int conv_kernel,
                     float l2_eps, hipStream_t stream)
{
    const long long n_vec = (long long)batch * 3 * heads;
    const dim3 grid((unsigned)((n_vec + kFeVecs - 1) / kFeVecs));
    const auto* x = reinterpret_cast<const unsigned short*>(qkv);
    const auto* w = reinterpret_cast<const unsigned short*>(conv_w);
    auto* co = reinterpret_cast<unsigned short*>(conv_out);
    const double eps = l2_eps;
    switch (conv_kernel) {
    case 1: launch_fe<1>(grid, x, w, conv_state, q, k, v, co, snaps, n_snap, batch, heads, T, eps, stream); break;
    case 2: launch_fe<2>(grid, x, w, conv_state, q, k, v, co, snaps, n_snap, batch, heads, T, eps, stream); break;
    case 3: launch_fe<3>(grid, x, w, conv_state, q, k, v, co, snaps, n_snap, batch, heads, T, eps, stream); break;
    case 4: launch_fe<4>(grid, x, w, conv_state, q, k, v, co, snaps, n_snap, batch, heads, T, eps, stream); break;
    default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace kda
