// Recurrent (decode) form of the KDA gated delta-rule core, gfx950.
//
// One kernel serves both decode entry points: a single token per sequence is
// the T = 1 case of the row-serial walk, so kda_recurrent_step and
// kda_recurrent_k execute the same instructions and agree bit for bit
// (layer page, Glm5NextKdaLayer::decode_k: the row path must match k serial
// decodes exactly).
//
// Memory plan (kernel-table page, recurrent_smem: one state read and one
// state write per step, the decayed state kept on chip between the two
// passes).  A workgroup owns one (sequence, head, 32-column value slice); its
// 512 threads load the slice of the 64 KiB head state straight into VGPRs
// with 16-byte loads (thread = 4 adjacent value columns x 2 key rows, a wave
// covers 8 rows of 128-byte segments), keep it there for all rows of the
// walk, and write it back once.  The slices of one head go to blocks 8 apart,
// which the dispatcher places on the same XCD, so each 512-byte state row is
// read and written through one L2.  Per row the only cross-thread traffic is
// the reduction of the read-outs over the key index: a xor-shuffle across the
// row groups inside the wave, then the eight waves' partial sums through LDS,
// summed once per (value, column group) in wave order and read back.  No
// atomics: every thread sums in the same fixed order, so results are
// deterministic.
//
// Geometry (measured, interleaved in one process, B=128 H=32 k=4 with 4
// snapshots / B=64 H=32 step): 512 threads x 4 slices 294 / 45.9 us; 256 x 4
// 317 / 46.1; 1024 x 2 298 / 47.2; 512 x 2 339 / 46.9; 1024 x 1 306 / 46.6;
// capping the workgroups per compute unit (LDS padding) was slower in every
// case (512 x 4 at 3 per CU 312, at 2 per CU 381).
//
// Inputs come in two forms: FP32 q, k, v as three [B][T][H][128] arrays, or
// BF16 q, k and v packed in one row a token as [B][T][3][H][128], the layout
// the decode front end writes (workspace page, conv_out: the BF16 output of the
// convolution and SiLU, with the L2 of q and k already applied when decoding).  BF16 widens to FP32 exactly and the row
// body is shared, so the BF16 form on BF16 data gives the bits of the FP32
// form on the widened values.
//
// Further forms of the same kernel (template switches): the gate and beta
// formed from their raw projections (kGated); the sigmoid-gated RMSNorm of
// every output row (kNorm, whole-head workgroups, the row then meeting in one
// wave); and, with the norm, the decode front end run by three of the
// workgroup's waves on the raw projections (FE_K = conv_kernel), so the
// whole step of the block between its projections is one kernel.
#include "kda_common.h"
#include "kda_front_end.h"
#include "kda_internal.h"

namespace kda {

template <int NSLICE, int THREADS = 256>
struct RecGeom {
    static constexpr int kThreads = THREADS;
    static constexpr int kCols = kD / NSLICE;           // value columns per workgroup
    static constexpr int kColGroups = kCols / 4;        // float4 column groups
    static constexpr int kRowGroups = kThreads / kColGroups;
    static constexpr int kRows = kD / kRowGroups;       // key rows per thread
    static constexpr int kWaves = kThreads / 64;
    static_assert(kColGroups <= 64 && 64 % kColGroups == 0, "a wave must hold whole row groups");
    // more than four waves: the waves' partial sums are reduced once per
    // (value, column group) by one thread each, then read back, instead of
    // every thread summing every wave
    static constexpr bool kTwoStage = kWaves > 4;
};

// Value slices per head.  Part of the arithmetic contract: the reduction tree
// depends on it, and both decode entry points use this one instance.
#ifndef KDA_REC_SLICES
#define KDA_REC_SLICES 4
#endif
#ifndef KDA_REC_THREADS
#define KDA_REC_THREADS 512
#endif
constexpr int kRecSlices = KDA_REC_SLICES;
constexpr int kRecThreads = KDA_REC_THREADS;
using RecG = RecGeom<kRecSlices, kRecThreads>;

// The carried state is streamed once per call: non-temporal hints keep it from
// displacing other data in the caches.
#ifndef KDA_REC_NONTEMPORAL
#define KDA_REC_NONTEMPORAL 1
#endif
__device__ __forceinline__ float4 state_ld(const float* p)
{
#if KDA_REC_NONTEMPORAL
    const float4* q = reinterpret_cast<const float4*>(p);
    return make_float4(__builtin_nontemporal_load(&q->x), __builtin_nontemporal_load(&q->y),
                       __builtin_nontemporal_load(&q->z), __builtin_nontemporal_load(&q->w));
#else
    return ld4(p);
#endif
}
__device__ __forceinline__ void state_st(float* p, float4 v)
{
#if KDA_REC_NONTEMPORAL
    float4* q = reinterpret_cast<float4*>(p);
    __builtin_nontemporal_store(v.x, &q->x);
    __builtin_nontemporal_store(v.y, &q->y);
    __builtin_nontemporal_store(v.z, &q->z);
    __builtin_nontemporal_store(v.w, &q->w);
#else
    st4(p, v);
#endif
}

// One row of the walk for one thread of a slice: decay of its state rows,
// partial read-outs, the reduction over key rows (xor shuffles inside the
// wave, then the slice's waves in order through s_red), delta, the rank-1
// update.  Returns the thread's four outputs (stored by row group 0).  The
// caller has staged the key, query and decay of the row in LDS and passes the
// thread's four values of v and the row's beta.
template <class G>
__device__ __forceinline__ float4 rec_row(float4 (&s)[G::kRows], const float* s_k, const float* s_q,
                                          const float* s_a, float (*s_red)[9][G::kColGroups],
                                          float (*s_tot)[G::kColGroups], float4 vv, float bt, int cg, int rg,
                                          int wave, int lane)
{
    // decay in place, then partial read-outs with the key and the query
    float red[9];
#pragma unroll
    for (int x = 0; x < 9; ++x) red[x] = 0.f;
    float kr[G::kRows];
#pragma unroll
    for (int m = 0; m < G::kRows; ++m) {
        const int i = rg + G::kRowGroups * m;
        const float a = s_a[i], kk = s_k[i], qq = s_q[i];
        kr[m] = kk;
        s[m].x *= a;
        s[m].y *= a;
        s[m].z *= a;
        s[m].w *= a;
        red[0] = fmaf(kk, s[m].x, red[0]);
        red[1] = fmaf(kk, s[m].y, red[1]);
        red[2] = fmaf(kk, s[m].z, red[2]);
        red[3] = fmaf(kk, s[m].w, red[3]);
        red[4] = fmaf(qq, s[m].x, red[4]);
        red[5] = fmaf(qq, s[m].y, red[5]);
        red[6] = fmaf(qq, s[m].z, red[6]);
        red[7] = fmaf(qq, s[m].w, red[7]);
        red[8] = fmaf(qq, kk, red[8]);
    }
    // reduce over the row groups of this wave ...
#pragma unroll
    for (int off = G::kColGroups; off < 64; off <<= 1) {
#pragma unroll
        for (int x = 0; x < 9; ++x) red[x] += __shfl_xor(red[x], off);
    }
    // ... then over the waves, in wave order
    if (lane < G::kColGroups) {
#pragma unroll
        for (int x = 0; x < 9; ++x) s_red[wave][x][lane] = red[x];
    }
    __syncthreads();
    float tot[9];
    if constexpr (G::kTwoStage) {
        const int tid = wave * 64 + lane;
        if (tid < 9 * G::kColGroups) {
            const int x = tid / G::kColGroups, c = tid % G::kColGroups;
            float acc = s_red[0][x][c];
#pragma unroll
            for (int w = 1; w < G::kWaves; ++w) acc += s_red[w][x][c];
            s_tot[x][c] = acc;
        }
        __syncthreads();
#pragma unroll
        for (int x = 0; x < 9; ++x) tot[x] = s_tot[x][cg];
    } else {
#pragma unroll
        for (int x = 0; x < 9; ++x) {
            float acc = s_red[0][x][cg];
#pragma unroll
            for (int w = 1; w < G::kWaves; ++w) acc += s_red[w][x][cg];
            tot[x] = acc;
        }
    }
    // delta = beta (v - S^T k);  out = S_dec^T q + (q.k) delta  (= S_new^T q)
    float4 d, o;
    d.x = bt * (vv.x - tot[0]);
    d.y = bt * (vv.y - tot[1]);
    d.z = bt * (vv.z - tot[2]);
    d.w = bt * (vv.w - tot[3]);
    o.x = fmaf(tot[8], d.x, tot[4]);
    o.y = fmaf(tot[8], d.y, tot[5]);
    o.z = fmaf(tot[8], d.z, tot[6]);
    o.w = fmaf(tot[8], d.w, tot[7]);
#pragma unroll
    for (int m = 0; m < G::kRows; ++m) {
        s[m].x = fmaf(kr[m], d.x, s[m].x);
        s[m].y = fmaf(kr[m], d.y, s[m].y);
        s[m].z = fmaf(kr[m], d.z, s[m].z);
        s[m].w = fmaf(kr[m], d.w, s[m].w);
    }
    return o;
}

// The sigmoid-gated RMSNorm of each output row (module page, pipeline line: the core's output goes
// through an RMSNorm with weight o_norm, gated by a sigmoid of g_b(g_a(h))), done where a whole-head
// workgroup has the row: y = x / sqrt(mean(x^2) + eps) * o_norm * sigmoid(out_gate), the sum of
// squares and the scale in FP64, the products in FP32, y rounded to BF16 (the arithmetic of
// gated_rmsnorm_kernel, with the 128 squares summed in another order).
struct NormParams {
    const unsigned short* out_gate;  // [B][T][H][128] BF16
    const unsigned short* o_norm;    // [128] BF16
    unsigned short* y;               // [B][T][H][128] BF16
    double eps;
};


// The decode front end inside the kernel (FE_K = conv_kernel > 0): `qkv` then holds the raw BF16
// projections ([B][T][3 H 128], a token's q, k, v channels in one row), and waves 0, 1, 2 of the whole-head
// workgroup run the front end of the head's q, k and v vectors with the code of
// kda_decode_front_end (fe_load, fe_row, fe_store: the same bits), keeping their conv slots in
// registers for all T rows.
struct FeParams {
    const unsigned short* conv_w;  // [3 H 128][K] BF16
    float* conv_state;             // [B][3 H 128][K] FP32, updated in place
    float* conv_snaps;             // [n_snap][B][3 H 128][K] FP32 or null
    double l2_eps;
};

// kGated: the gate comes from kda_gate of gp.g_raw (gate not read) and beta holds the logits,
// passed through the sigmoid here (see GateParams).
// kNorm (whole-head workgroups only): each output row also goes through the gated RMSNorm into
// np.y; out may then be null (the FP32 row is not stored).
// FE_K > 0 (whole-head workgroups with kNorm): the front end runs first (see FeParams).
template <int NSLICE, bool kPackedBf16, int THREADS = 256, bool kGated = false, bool kNorm = false, int FE_K = 0>
__global__ __launch_bounds__(THREADS) void recurrent_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                        const float* __restrict__ v,
                                                        const unsigned short* __restrict__ qkv,
                                                        const float* __restrict__ gate,
                                                        const float* __restrict__ beta, float* __restrict__ state,
                                                        float* __restrict__ out, float* __restrict__ snaps,
                                                        int n_snap, int batch, int heads, int T, GateParams gp,
                                                        NormParams np = NormParams{}, FeParams fp = FeParams{})
{
    static_assert(!kNorm || NSLICE == 1, "the fused norm needs the whole row in one workgroup");
    constexpr bool kFE = FE_K > 0;
    static_assert(!kFE || (kNorm && !kPackedBf16 && THREADS >= 3 * 64), "front end: whole-head FP32 staging");
    using G = RecGeom<NSLICE, THREADS>;
    const int tid = threadIdx.x;
    // blocks come in groups of 8 * NSLICE: 8 heads, slice s of head j at 8 s + j
    const int r = blockIdx.x % (8 * NSLICE);
    const int slice = r / 8;
    const int bh = blockIdx.x / (8 * NSLICE) * 8 + r % 8;  // b * heads + h
    if (bh >= batch * heads) return;  // padding of the last group (the whole block leaves)
    const int b = bh / heads, h = bh % heads;
    const int cg = tid % G::kColGroups;
    const int rg = tid / G::kColGroups;
    const int wave = tid / 64;
    const int lane = tid % 64;
    const int col = slice * G::kCols + 4 * cg;

    __shared__ float s_k[kD], s_q[kD], s_a[kD];
    __shared__ float s_v[kFE ? kD : 1];
    __shared__ float s_red[G::kWaves][9][G::kColGroups];
    __shared__ float s_tot[G::kTwoStage ? 9 : 1][G::kColGroups];

    // per-head rate of the gate (kGated)
    const float rate = kGated ? __builtin_amdgcn_exp2f(1.4426950408889634f * gp.a_log[h]) : 0.f;
    const float dtb = kGated && tid < kD ? gp.dt_bias[h * kD + tid] : 0.f;  // the head's bias of channel tid

    // front end: wave p < 3 owns the head's vector of part p (q, k, v), channels lane and lane + 64
    const int Cdim = 3 * heads * kD;
    const size_t fe_cv = ((size_t)(wave < 3 ? wave : 0) * heads + h) * kD;  // first channel of the vector
    FeLane<kFE ? FE_K : 1> fl;
    if constexpr (kFE) {
        if (wave < 3) fe_load(fl, fp.conv_w, fp.conv_state + ((size_t)b * Cdim + fe_cv) * FE_K, fe_cv, lane);
    }

    // A row's inputs as loaded, still raw: the next row's are requested right after the current one
    // is staged (into the same registers), ahead of the current row's stores, so the wait for them
    // never covers a store (the vector memory counter counts loads and stores in order).  Widening, the gate's exponential and
    // the sigmoids happen only when a row is staged.
    struct RowIn {
        float q, k, g;      // FP32 q, k and the gate (FP32 forms)
        unsigned qb, kb;    // BF16 q, k (packed form), g_raw (gated form: in gb)
        unsigned gb;
        float b;            // beta, or its logit (gated form)
        float4 v;           // FP32 v
        uint2 vb;           // BF16 v (packed form)
        unsigned short x0, x1;  // front end: the raw projections of the wave's two channels
    };
    auto load_row = [&](int tt, RowIn& r) {
        const size_t rr = ((size_t)b * T + tt) * heads + h;  // (b, tt, h)
        if constexpr (kFE) {
            if (wave < 3) {
                const unsigned short* const x = qkv + ((size_t)b * T + tt) * Cdim + fe_cv + lane;
                r.x0 = x[0];
                r.x1 = x[64];
            }
            if (tid < kD) {
                if constexpr (kGated) r.gb = gp.g_raw[rr * kD + tid];
                else r.g = gate[rr * kD + tid];
            }
        } else if constexpr (kPackedBf16) {
            // q of head h in token (b, tt); k and v follow at a stride of heads * 128
            const unsigned short* const x = qkv + (((size_t)b * T + tt) * 3 * heads + h) * kD;
            const size_t part = (size_t)heads * kD;
            if (tid < kD) {
                r.kb = x[part + tid];
                r.qb = x[tid];
                r.g = gate[rr * kD + tid];
            }
            r.vb = *reinterpret_cast<const uint2*>(x + 2 * part + col);
        } else {
            if (tid < kD) {
                r.k = k[rr * kD + tid];
                r.q = q[rr * kD + tid];
                if constexpr (kGated) r.gb = gp.g_raw[rr * kD + tid];
                else r.g = gate[rr * kD + tid];
            }
            r.v = ld4(v + rr * kD + col);
        }
        r.b = beta[rr];
    };
    // the first row's inputs go out before the state: loads complete in order, so the row can be
    // staged (and, with the front end inside, its conv, SiLU and L2 computed) while the state streams in
    RowIn cur;
    load_row(0, cur);
    float* const S_head = state + (size_t)bh * kD * kD;
    float4 s[G::kRows];
#pragma unroll
    for (int m = 0; m < G::kRows; ++m) s[m] = state_ld(S_head + (size_t)(rg + G::kRowGroups * m) * kD + col);
    for (int t = 0; t < T; ++t) {
        const size_t row = ((size_t)b * T + t) * heads + h;  // (b, t, h)
        float bt;
        float4 vv;
        if constexpr (kFE) {
            if (wave < 3) {
                float y[2];
                fe_row(fl, cur.x0, cur.x1, wave < 2, fp.l2_eps, y);
                float* const dst = wave == 0 ? s_q : (wave == 1 ? s_k : s_v);
                dst[lane] = y[0];
                dst[lane + 64] = y[1];
                if (t < n_snap && fp.conv_snaps)
                    fe_store(fl, fp.conv_snaps + (((size_t)t * batch + b) * Cdim + fe_cv) * FE_K, lane);
            }
        }
        if (tid < kD) {
            if constexpr (kPackedBf16) {
                s_k[tid] = bf16_to_f32(cur.kb);
                s_q[tid] = bf16_to_f32(cur.qb);
            } else if constexpr (!kFE) {
                s_k[tid] = cur.k;
                s_q[tid] = cur.q;
            }
            if constexpr (kGated)
                s_a[tid] = expf(kda_gate_f32(bf16_to_f32(cur.gb), dtb, rate, gp.lower));
            else
                s_a[tid] = expf(cur.g);
        }
        bt = kGated ? sigmoid_f32(cur.b) : cur.b;
        if constexpr (kFE)
            vv = make_float4(0.f, 0.f, 0.f, 0.f);  // read from s_v after the barrier
        else if constexpr (kPackedBf16)
            vv = make_float4(bf16_to_f32(cur.vb.x & 0xffffu), bf16_to_f32(cur.vb.x >> 16),
                             bf16_to_f32(cur.vb.y & 0xffffu), bf16_to_f32(cur.vb.y >> 16));
        else
            vv = cur.v;
        __syncthreads();
        if constexpr (kFE) vv = make_float4(s_v[col], s_v[col + 1], s_v[col + 2], s_v[col + 3]);
        // the next row's inputs, into the registers the staging above has just consumed
        if (t + 1 < T) load_row(t + 1, cur);
        const float4 o = rec_row<G>(s, s_k, s_q, s_a, s_red, s_tot, vv, bt, cg, rg, wave, lane);
        if (rg == 0 && (!kNorm || out)) st4(out + row * kD + col, o);
        if constexpr (kNorm) {
            // row group 0 (lanes 0..31 of wave 0) holds the 128 outputs, 4 adjacent columns a lane
            if (rg == 0) {
                double ss = (double)o.x * o.x + (double)o.y * o.y + (double)o.z * o.z + (double)o.w * o.w;
#pragma unroll
                for (int off = 1; off < G::kColGroups; off <<= 1) ss += __shfl_xor(ss, off, G::kColGroups);
                const double r = norm_rsqrt(ss * (1.0 / kD) + np.eps);
                const uint2 g2 = *reinterpret_cast<const uint2*>(np.out_gate + row * kD + col);
                const uint2 w2 = *reinterpret_cast<const uint2*>(np.o_norm + col);
                const float x[4] = {o.x, o.y, o.z, o.w};
                const unsigned gb[4] = {g2.x & 0xffffu, g2.x >> 16, g2.y & 0xffffu, g2.y >> 16};
                const unsigned wb[4] = {w2.x & 0xffffu, w2.x >> 16, w2.y & 0xffffu, w2.y >> 16};
                unsigned yb[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    yb[e] = f32_to_bf16((float)(x[e] * r) * bf16_to_f32(wb[e]) * sigmoid_f32(bf16_to_f32(gb[e])));
                *reinterpret_cast<uint2*>(np.y + row * kD + col) = make_uint2(yb[0] | (yb[1] << 16), yb[2] | (yb[3] << 16));
            }
        }
        if (t < n_snap) {
            // snapshots are streamed like the state (non-temporal stores): at 512 threads x 4
            // slices that made decode_k ~2% faster than cacheable stores (interleaved A/B)
            float* snap = snaps + ((size_t)t * batch * heads + bh) * kD * kD;
#pragma unroll
            for (int m = 0; m < G::kRows; ++m) state_st(snap + (size_t)(rg + G::kRowGroups * m) * kD + col, s[m]);
        }
    }
#pragma unroll
    for (int m = 0; m < G::kRows; ++m) state_st(S_head + (size_t)(rg + G::kRowGroups * m) * kD + col, s[m]);
    if constexpr (kFE) {
        if (wave < 3) fe_store(fl, fp.conv_state + ((size_t)b * Cdim + fe_cv) * FE_K, lane);
    }
}

int launch_recurrent(const float* q, const float* k, const float* v, const uint16_t* qkv, const float* gate,
                     const float* beta, float* state, float* out, float* snaps, int n_snap, int batch, int heads,
                     int T, hipStream_t stream, const GateParams* gp)
{
    const unsigned grid = ((unsigned)batch * (unsigned)heads + 7u) / 8u * 8u * kRecSlices;
    const auto* x = reinterpret_cast<const unsigned short*>(qkv);
    if (gp)
        hipLaunchKernelGGL((recurrent_kernel<kRecSlices, false, kRecThreads, true>), dim3(grid), dim3(kRecThreads), 0,
                           stream, q, k, v, nullptr, nullptr, beta, state, out, snaps, n_snap, batch, heads, T, *gp);
    else if (qkv)
        hipLaunchKernelGGL((recurrent_kernel<kRecSlices, true, kRecThreads>), dim3(grid), dim3(kRecThreads), 0, stream,
                           nullptr, nullptr, nullptr, x, gate, beta, state, out, snaps, n_snap, batch, heads, T,
                           GateParams{});
    else
        hipLaunchKernelGGL((recurrent_kernel<kRecSlices, false, kRecThreads>), dim3(grid), dim3(kRecThreads), 0,
                           stream, q, k, v, nullptr, gate, beta, state, out, snaps, n_snap, batch, heads, T,
                           GateParams{});
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// A walk of several rows (each with its snapshots) runs one workgroup per compute unit: two per CU,
// which the kernel's registers allow, made the B=128 H=32 4-row walk with 4 snapshots 300 -> 320 us,
// while the single step (B=64 H=32) gains from them (50.5 -> 47.7 us).  Reserved LDS keeps it to one.
constexpr size_t kFusedWalkLdsPad = 72 * 1024;

// The decode step / k-row walk on BF16 q | k | v with the gated RMSNorm of every output row fused
// in: one 512-thread workgroup per (sequence, head), the whole row in one wave (measured per B=64
// H=32 step: 512 threads 47.6 us, 1024 threads 50.1, 256 threads 48.8).
constexpr int kNormRecThreads = 512;

int launch_recurrent_norm(const uint16_t* qkv, const float* gate, const float* beta, float* state, float* out,
                          float* snaps, int n_snap, int batch, int heads, int T, const uint16_t* out_gate,
                          const uint16_t* o_norm, uint16_t* y, float eps, hipStream_t stream)
{
    const unsigned grid = ((unsigned)batch * (unsigned)heads + 7u) / 8u * 8u;
    const NormParams np{reinterpret_cast<const unsigned short*>(out_gate),
                        reinterpret_cast<const unsigned short*>(o_norm), reinterpret_cast<unsigned short*>(y),
                        (double)eps};
    hipLaunchKernelGGL((recurrent_kernel<1, true, kNormRecThreads, false, true>), dim3(grid), dim3(kNormRecThreads),
                       T > 1 ? kFusedWalkLdsPad : 0,
                       stream, nullptr, nullptr, nullptr, reinterpret_cast<const unsigned short*>(qkv), gate, beta,
                       state, out, snaps, n_snap, batch, heads, T, GateParams{}, np);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// The whole decode step from the raw projections: front end, gate, core and gated RMSNorm in one
// kernel (the geometry of launch_recurrent_norm).
template <int K, bool kGated>
static void launch_fused_k(unsigned grid, const unsigned short* x, const float* gate, const float* beta, float* state,
                           float* out, float* snaps, int n_snap, int batch, int heads, int T, const GateParams& gp,
                           const NormParams& np, const FeParams& fp, hipStream_t stream)
{
    hipLaunchKernelGGL((recurrent_kernel<1, false, kNormRecThreads, kGated, true, K>), dim3(grid),
                       dim3(kNormRecThreads), T > 1 ? kFusedWalkLdsPad : 0, stream, nullptr, nullptr, nullptr, x,
                       gate, beta, state, out, snaps, n_snap, batch, heads, T, gp, np, fp);
}

int launch_decode_fused(const uint16_t* qkv_proj, const uint16_t* conv_w, float* conv_state, float* conv_snaps,
                        const float* gate, const float* beta, const GateParams* gp, float* state, float* out,
                        float* snaps, int n_snap, int batch, int heads, int T, int conv_kernel,
                        const uint16_t* out_gate, const uint16_t* o_norm, uint16_t* y, float eps, float l2_eps,
                        hipStream_t stream)
{
    const unsigned grid = ((unsigned)batch * (unsigned)heads + 7u) / 8u * 8u;
    const auto* x = reinterpret_cast<const unsigned short*>(qkv_proj);
    const NormParams np{reinterpret_cast<const unsigned short*>(out_gate),
                        reinterpret_cast<const unsigned short*>(o_norm), reinterpret_cast<unsigned short*>(y),
                        (double)eps};
    const FeParams fp{reinterpret_cast<const unsigned short*>(conv_w), conv_state, conv_snaps, (double)l2_eps};
    const GateParams g = gp ? *gp : GateParams{};
#define KDA_FUSED_CASE(K)                                                                                         \
    case K:                                                                                                       \
        if (gp) launch_fused_k<K, true>(grid, x, nullptr, beta, state, out, snaps, n_snap, batch, heads, T, g, np, fp, stream); \
        else launch_fused_k<K, false>(grid, x, gate, beta, state, out, snaps, n_snap, batch, heads, T, g, np, fp, stream); \
        break;
    switch (conv_kernel) {
        KDA_FUSED_CASE(1)
        KDA_FUSED_CASE(2)
        KDA_FUSED_CASE(3)
        KDA_FUSED_CASE(4)
    default: return -1;
    }
#undef KDA_FUSED_CASE
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

long long recurrent_max_units() { return 0x7fffffffLL / kRecSlices - 8; }

}  // namespace kda
