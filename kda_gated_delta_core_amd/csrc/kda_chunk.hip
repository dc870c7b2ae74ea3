// Chunked (prefill) form of the KDA gated delta-rule core, gfx950.
//
// Two kernels, as the kernel-table page splits the prefill (fields
// chunk_prepare and chunk_scan):
//
//  chunk_prepare  one workgroup per (sequence, head, chunk), all chunks in
//                 parallel.  Builds the chunk's WY/UT factors in LDS with FP32
//                 MFMA and writes one workspace record:
//                   W = T diag(beta)(e^G o K), U = T diag(beta) V,
//                   Qhat = e^G o Q, Ktil^T = (e^{G_last - G} o K)^T,
//                   M (lower-triangular decayed Q K^T), gamma = e^{G_last},
//                 with G the per-channel cumulative log-decay inside the chunk,
//                 A the strictly lower decayed K K^T scaled by beta and
//                 T = (I + A)^-1.
//  chunk_scan     one workgroup per (sequence, head, 16-column value slice),
//                 serial over chunks, its 128x16 state slice resident in
//                 registers.  Per chunk:
//                   Delta = U - W S,  O = Qhat S + M Delta,
//                   S <- diag(gamma) S + Ktil^T Delta
//                 all as 16x16x4 FP32 MFMA tiles.  Value columns never mix, so
//                 the eight slices of a head run independently; they are
//                 placed on one XCD so the head's records are fetched into
//                 that XCD's L2 once.
//
// Decay handling: G is accumulated in log2 units, separately inside each
// 16-row block, so no cumulative sum grows beyond 16 gates.  Every pairwise
// factor exp(G_r - G_s) in A and M is split about a reference row: the last
// row of the earlier block for off-diagonal blocks (both factors <= 1), row 7
// of the block for diagonal blocks (each factor spans at most 8 gates).  Pad
// rows (t >= T) are replaced by zeros with selects before any arithmetic, so
// NaN or inf there never reaches a result.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int C>
struct ChunkGeom {
    static constexpr int kTiles = C / 16;      // 16-row tiles per chunk
    static constexpr int kLd = kD + 4;         // LDS row stride of [C][128] tables (floats)
    static constexpr int kLdc = C + 4;         // LDS row stride of [C][C] tables
    static constexpr size_t kOffW = 0;
    static constexpr size_t kOffU = (size_t)C * kD;
    static constexpr size_t kOffQ = 2 * (size_t)C * kD;
    static constexpr size_t kOffKt = 3 * (size_t)C * kD;
    static constexpr size_t kOffM = 4 * (size_t)C * kD;
    static constexpr size_t kOffGam = kOffM + (size_t)C * C;
    static constexpr size_t kRecord = kOffGam + kD;
    static constexpr int kPairs = kTiles * (kTiles + 1) / 2;
    static_assert(kRecord == chunk_record_floats(C), "record layout");
};

__device__ __forceinline__ float4 lds4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void lds4_st(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ float comp(const float4& v, int e)
{
    return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
}

template <int C>
__global__ __launch_bounds__(256) void chunk_prepare_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                            const float* __restrict__ v,
                                                            const float* __restrict__ gate,
                                                            const float* __restrict__ beta, float* __restrict__ ws,
                                                            int heads, int T, int t_pad, int nchunks)
{
    using G = ChunkGeom<C>;
    constexpr int NT = G::kTiles, LD = G::kLd, LDC = G::kLdc;
    __shared__ float sK[C * LD];
    __shared__ float sQ[C * LD];    // q; later beta e^G k
    __shared__ float sL[C * LD];    // block-local log2 cumulative decay; later beta v
    __shared__ float sA[C * LDC];   // beta-scaled strictly lower A
    __shared__ float sT[C * LDC];   // (I + A)^-1
    __shared__ float sBlk[NT * kD]; // log2 decay of each whole 16-row block
    __shared__ float sBeta[C];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int c = blockIdx.x % nchunks;
    const int bh = blockIdx.x / nchunks;
    const int b = bh / heads, h = bh % heads;
    const int t0 = c * C;
    float* const rec = ws + (size_t)blockIdx.x * G::kRecord;
    const size_t row0 = ((size_t)b * t_pad + t0) * heads + h;  // (b, t0, h)
    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);

    // 1. stage K and Q; rows >= T are selected to zero
    for (int e = tid; e < C * 32; e += 256) {
        const int r = e >> 5, c4 = (e & 31) * 4;
        const bool ok = t0 + r < T;
        const size_t off = (row0 + (size_t)r * heads) * kD + c4;
        const float4 kk = ok ? ld4(k + off) : z4;
        const float4 qq = ok ? ld4(q + off) : z4;
        lds4_st(&sK[r * LD + c4], kk);
        lds4_st(&sQ[r * LD + c4], qq);
    }
    // block-local cumulative log2 decay
    for (int e = tid; e < NT * kD; e += 256) {
        const int j = e & (kD - 1), R = e >> 7;
        float acc = 0.f;
        for (int r = 16 * R; r < 16 * R + 16; ++r) {
            const bool ok = t0 + r < T;
            const float g = ok ? gate[(row0 + (size_t)r * heads) * kD + j] : 0.f;
            acc = fmaf(g, kLog2e, acc);
            sL[r * LD + j] = acc;
        }
        sBlk[R * kD + j] = acc;
    }
    if (tid < C) sBeta[tid] = (t0 + tid < T) ? beta[row0 + (size_t)tid * heads] : 0.f;
    __syncthreads();

    // 2. Qhat = e^G o Q, Ktil^T = (e^{G_last - G} o K)^T and gamma = e^{G_last}
    for (int e = tid; e < C * kD; e += 256) {
        const int r = e >> 7, j = e & (kD - 1), R = r >> 4;
        float pre = 0.f;
        for (int X = 0; X < R; ++X) pre += sBlk[X * kD + j];
        rec[G::kOffQ + e] = sQ[r * LD + j] * exp2_fast(pre + sL[r * LD + j]);
    }
    for (int e = tid; e < C * kD; e += 256) {
        const int j = e / C, r = e % C, R = r >> 4;
        float suf = 0.f;
        for (int X = R + 1; X < NT; ++X) suf += sBlk[X * kD + j];
        rec[G::kOffKt + e] = sK[r * LD + j] * exp2_fast(suf + (sBlk[R * kD + j] - sL[r * LD + j]));
    }
    if (tid < kD) {
        float tot = 0.f;
        for (int X = 0; X < NT; ++X) tot += sBlk[X * kD + tid];
        rec[G::kOffGam + tid] = exp2_fast(tot);
    }

    // 3. A and M, one 16x16 block pair (R, S <= R) per wave at a time
    for (int p = wave; p < G::kPairs; p += 4) {
        int R = 0;
        while ((R + 1) * (R + 2) / 2 <= p) ++R;
        const int S = p - R * (R + 1) / 2;
        const int ra = 16 * R + l16, sb = 16 * S + l16;
        floatx4 accA = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tau = 0; tau < 8; ++tau) {
            const int i0 = 16 * tau + 4 * q4;
            const float4 kr = lds4(&sK[ra * LD + i0]);
            const float4 qr = lds4(&sQ[ra * LD + i0]);
            const float4 lr = lds4(&sL[ra * LD + i0]);
            const float4 ks = lds4(&sK[sb * LD + i0]);
            const float4 ls = lds4(&sL[sb * LD + i0]);
            float4 er, es;  // log2 exponents of the row and column factors
            if (S < R) {
                float4 mid = z4;
                for (int X = S + 1; X < R; ++X) {
                    const float4 bx = lds4(&sBlk[X * kD + i0]);
                    mid.x += bx.x; mid.y += bx.y; mid.z += bx.z; mid.w += bx.w;
                }
                const float4 bs = lds4(&sBlk[S * kD + i0]);
                er = make_float4(lr.x + mid.x, lr.y + mid.y, lr.z + mid.z, lr.w + mid.w);
                es = make_float4(bs.x - ls.x, bs.y - ls.y, bs.z - ls.z, bs.w - ls.w);
            } else {
                const float4 lm = lds4(&sL[(16 * R + 7) * LD + i0]);
                er = make_float4(lr.x - lm.x, lr.y - lm.y, lr.z - lm.z, lr.w - lm.w);
                es = make_float4(lm.x - ls.x, lm.y - ls.y, lm.z - ls.z, lm.w - ls.w);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float xr = exp2_fast(comp(er, e));
                const float yc = comp(ks, e) * exp2_fast(comp(es, e));
                accA = mfma4(comp(kr, e) * xr, yc, accA);
                accM = mfma4(comp(qr, e) * xr, yc, accM);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * R + 4 * q4 + e, s = 16 * S + l16;
            sA[r * LDC + s] = (S < R || s < r) ? sBeta[r] * accA[e] : 0.f;
            rec[G::kOffM + (size_t)r * C + s] = (S < R || s <= r) ? accM[e] : 0.f;
        }
    }
    for (int e = tid; e < C * C; e += 256) {
        const int r = e / C, s = e % C;
        if ((s >> 4) > (r >> 4)) rec[G::kOffM + e] = 0.f;
    }
    __syncthreads();

    // 4a. T_RR = (I + A_RR)^-1 for each diagonal block, by forward substitution
    if (wave < NT && lane < 16) {
        const int base = 16 * wave;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float acc = (i == lane) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) acc = fmaf(-sA[(base + i) * LDC + base + m], x[m], acc);
            x[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sT[(base + i) * LDC + base + lane] = x[i];
    }
    __syncthreads();
    // 4b. off-diagonal blocks, by distance from the diagonal:
    //     T_RS = -T_RR sum_{X=S}^{R-1} A_RX T_XS
    for (int d = 1; d < NT; ++d) {
        const int S = wave, R = wave + d;
        if (R < NT) {
            floatx4 zacc = {0.f, 0.f, 0.f, 0.f};
            for (int X = S; X < R; ++X) {
                const float4 a4 = lds4(&sA[(16 * R + l16) * LDC + 16 * X + 4 * q4]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    zacc = mfma4(comp(a4, e), sT[(16 * X + 4 * q4 + e) * LDC + 16 * S + l16], zacc);
            }
            const float4 t4 = lds4(&sT[(16 * R + l16) * LDC + 16 * R + 4 * q4]);
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = mfma4(comp(t4, e), zacc[e], acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) sT[(16 * R + 4 * q4 + e) * LDC + 16 * S + l16] = -acc[e];
        }
        __syncthreads();
    }

    // 5. right-hand sides: beta e^G o K (over Q, now dead) and beta V (over the decay table)
    for (int e = tid; e < C * kD; e += 256) {
        const int r = e >> 7, j = e & (kD - 1), R = r >> 4;
        float pre = 0.f;
        for (int X = 0; X < R; ++X) pre += sBlk[X * kD + j];
        sQ[r * LD + j] = sBeta[r] * (exp2_fast(pre + sL[r * LD + j]) * sK[r * LD + j]);
    }
    __syncthreads();
    for (int e = tid; e < C * 32; e += 256) {
        const int r = e >> 5, c4 = (e & 31) * 4;
        const bool ok = t0 + r < T;
        const float4 vv = ok ? ld4(v + (row0 + (size_t)r * heads) * kD + c4) : z4;
        const float bb = sBeta[r];
        lds4_st(&sL[r * LD + c4], make_float4(bb * vv.x, bb * vv.y, bb * vv.z, bb * vv.w));
    }
    __syncthreads();

    // 6. W = T (beta e^G o K) and U = T (beta V), 16x16 output tiles
    for (int job = wave; job < 2 * NT * 8; job += 4) {
        const int which = job / (NT * 8);
        const int X = (job >> 3) % NT, cc = job & 7;
        const float* Bm = which ? sL : sQ;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int Y = 0; Y <= X; ++Y) {
            const float4 t4 = lds4(&sT[(16 * X + l16) * LDC + 16 * Y + 4 * q4]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc = mfma4(comp(t4, e), Bm[(16 * Y + 4 * q4 + e) * LD + 16 * cc + l16], acc);
        }
        float* dst = rec + (which ? G::kOffU : G::kOffW);
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(size_t)(16 * X + 4 * q4 + e) * kD + 16 * cc + l16] = acc[e];
    }
}

template <int C>
__global__ __launch_bounds__(256) void chunk_scan_kernel(const float* __restrict__ ws, float* __restrict__ state,
                                                         float* __restrict__ out, int n_bh, int heads, int T,
                                                         int t_pad, int nchunks)
{
    using G = ChunkGeom<C>;
    constexpr int NT = G::kTiles;
    // blockIdx -> (head, slice) so that all eight slices of a head share an XCD
    const int n = blockIdx.x;
    const int xcd = n & 7, k8 = n >> 3;
    const int slice = k8 & 7;
    const int bh = (k8 >> 3) * 8 + xcd;
    if (bh >= n_bh) return;
    const int b = bh / heads, h = bh % heads;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int v0 = 16 * slice;

    __shared__ floatx4 sDelta[NT][64];
    __shared__ floatx4 sS[8][64];

    // state slice as eight 16x16 accumulator tiles: tile s, element e of lane l
    // holds S[16 s + 4 (l / 16) + e][v0 + l % 16]; every wave keeps a full copy
    float* const S_head = state + (size_t)bh * kD * kD;
    floatx4 S[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[s][e] = S_head[(size_t)(16 * s + 4 * q4 + e) * kD + v0 + l16];

    int own = -1;  // output tile finished by this wave
    for (int j = NT; j < 2 * NT; ++j)
        if ((j & 3) == wave) own = j - NT;

    for (int c = 0; c < nchunks; ++c) {
        const float* rec = ws + ((size_t)bh * nchunks + c) * G::kRecord;
        floatx4 P = {0.f, 0.f, 0.f, 0.f};
        // phase 1: Delta tiles (W S) and the Qhat S part of the output tiles
        for (int job = wave; job < 2 * NT; job += 4) {
            const bool is_delta = job < NT;
            const int X = is_delta ? job : job - NT;
            const float* Am = rec + (is_delta ? G::kOffW : G::kOffQ) + (size_t)(16 * X + l16) * kD + 4 * q4;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int tau = 0; tau < 8; ++tau) {
                const float4 a4 = ld4(Am + 16 * tau);
                acc = mfma4(a4.x, S[tau][0], acc);
                acc = mfma4(a4.y, S[tau][1], acc);
                acc = mfma4(a4.z, S[tau][2], acc);
                acc = mfma4(a4.w, S[tau][3], acc);
            }
            if (is_delta) {
                floatx4 d;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    d[e] = rec[G::kOffU + (size_t)(16 * X + 4 * q4 + e) * kD + v0 + l16] - acc[e];
                sDelta[X][lane] = d;
            } else {
                P = acc;
            }
        }
        __syncthreads();
        // phase 2a: O = Qhat S + M Delta
        if (own >= 0) {
            const int X = own;
            const float* Mm = rec + G::kOffM + (size_t)(16 * X + l16) * C + 4 * q4;
            for (int Y = 0; Y <= X; ++Y) {
                const floatx4 d = sDelta[Y][lane];
                const float4 m4 = ld4(Mm + 16 * Y);
                P = mfma4(m4.x, d[0], P);
                P = mfma4(m4.y, d[1], P);
                P = mfma4(m4.z, d[2], P);
                P = mfma4(m4.w, d[3], P);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = c * C + 16 * X + 4 * q4 + e;
                if (t < T) out[(((size_t)b * t_pad + t) * heads + h) * kD + v0 + l16] = P[e];
            }
        }
        // phase 2b: S <- diag(gamma) S + Ktil^T Delta, tiles 2 wave and 2 wave + 1
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            if ((s >> 1) != wave) continue;
            const float4 g4 = ld4(rec + G::kOffGam + 16 * s + 4 * q4);
            floatx4 acc;
            acc[0] = g4.x * S[s][0];
            acc[1] = g4.y * S[s][1];
            acc[2] = g4.z * S[s][2];
            acc[3] = g4.w * S[s][3];
            const float* Km = rec + G::kOffKt + (size_t)(16 * s + l16) * C + 4 * q4;
#pragma unroll
            for (int Y = 0; Y < NT; ++Y) {
                const floatx4 d = sDelta[Y][lane];
                const float4 k4 = ld4(Km + 16 * Y);
                acc = mfma4(k4.x, d[0], acc);
                acc = mfma4(k4.y, d[1], acc);
                acc = mfma4(k4.z, d[2], acc);
                acc = mfma4(k4.w, d[3], acc);
            }
            sS[s][lane] = acc;
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < 8; ++s) S[s] = sS[s][lane];
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        if ((s >> 1) != wave) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) S_head[(size_t)(16 * s + 4 * q4 + e) * kD + v0 + l16] = S[s][e];
    }
}

template <int C>
static int launch_chunk(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                        float* state, float* out, int batch, int heads, int T, int t_pad, float* ws,
                        hipStream_t stream)
{
    const int nchunks = t_pad / C;
    const long long n_bh = (long long)batch * heads;
    hipLaunchKernelGGL(chunk_prepare_kernel<C>, dim3((unsigned)(n_bh * nchunks)), dim3(256), 0, stream, q, k, v,
                       gate, beta, ws, heads, T, t_pad, nchunks);
    if (hipGetLastError() != hipSuccess) return -1;
    const unsigned grid = (unsigned)(((n_bh + 7) / 8) * 64);
    hipLaunchKernelGGL(chunk_scan_kernel<C>, dim3(grid), dim3(256), 0, stream, ws, state, out, (int)n_bh, heads, T,
                       t_pad, nchunks);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_chunk_prefill(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                         float* state, float* out, int batch, int heads, int T, int t_pad, int chunk,
                         float* workspace, hipStream_t stream)
{
    switch (chunk) {
    case 16: return launch_chunk<16>(q, k, v, gate, beta, state, out, batch, heads, T, t_pad, workspace, stream);
    case 32: return launch_chunk<32>(q, k, v, gate, beta, state, out, batch, heads, T, t_pad, workspace, stream);
    case 64: return launch_chunk<64>(q, k, v, gate, beta, state, out, batch, heads, T, t_pad, workspace, stream);
    default: return -1;
    }
}

}  // namespace kda
