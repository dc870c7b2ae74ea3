// Chunked (prefill) form of the KDA gated delta-rule core, gfx950.
//
// Two kernels, as the kernel-table page splits the prefill (fields
// chunk_prepare and chunk_scan):
//
//  chunk_prepare  chunks are independent: one persistent workgroup per compute
//                 unit walks (sequence, head, chunk) triples.  Builds the
//                 chunk's WY/UT factors in LDS with FP32 MFMA: G the
//                 per-channel cumulative log-decay inside the chunk, A the
//                 strictly lower decayed K K^T scaled by beta, T = (I + A)^-1
//                 (only its 16x16 diagonal blocks are inverted; the rest is
//                 block forward substitution on the right-hand sides), M the
//                 lower-triangular decayed Q K^T,
//                   W = T diag(beta)(e^G o K),  U = T diag(beta) V,
//                 and writes one workspace record with W, U,
//                   P = e^G o Q - M W,  R = M U,
//                   Ktil^T = (e^{G_last - G} o K)^T,  gamma = e^{G_last}.
//                 (O = (e^G o Q) S + M (U - W S) = P S + R, so the output no
//                 longer waits for Delta inside the scan.)
//  chunk_scan     one workgroup per (sequence, head, group of 16 or 32 value
//                 columns), serial over chunks, its 128-row state slice
//                 resident on chip.  Per chunk:
//                   Delta = U - W S,  O = P S + R,
//                   S <- diag(gamma) S + Ktil^T Delta
//                 all as 16x16x4 FP32 MFMA tiles.  Value columns never mix, so
//                 the column groups of a head run independently (and the group
//                 width does not change a bit of the result); they are placed
//                 on one XCD so the head's records are fetched into that XCD's
//                 L2 once.
//
// Both kernels take a layout: DenseLayout (sequences of one length, padded to
// whole chunks) or VarlenLayout (sequences of their own lengths packed back
// to back, located through offsets a one-workgroup set-up kernel clamps and
// counts into the workspace).  Only the index arithmetic differs; a sequence
// gets the same bits either way.
//
// Decay handling: the gate is accumulated in log2 units, separately inside
// each 16-row block (L), so no running sum grows beyond 16 gates.  One pass
// turns K and Q into tables decayed about row 7 of their own block,
//   Kr = K o 2^(L - L7),  Qr = Q o 2^(L - L7),  Kc = K o 2^(L7 - L)
// (each factor spans at most 8 gates), with two exponentials per element.
// That keeps every factor a normal float while each gate is >= -12 in log2
// units; a chunk with a steeper gate (checked while it is staged, so the
// choice is uniform over the workgroup) takes the steep-gate path instead:
// K, Q and L stay as they are and each operand is decayed by one exponential
// of an exponent sum <= 0 (two products, about two reference rows, on the
// diagonal blocks; see am_below_steep, am_diag_steep), with gates clamped at
// -kSteepGateClampLog2.
// Everything else needs only per-channel factors on top of those tables:
//   diagonal blocks of A, M   Kr Kc^T, Qr Kc^T              (no rescaling)
//   block pair S < R          (Kr o X_RS)(Kc o Y_S)^T      X_RS = 2^(G7_R - Gend_S),
//                             Y_S = 2^(Gend_S - G7_S): both operands are then
//                             decayed about the last row of block S, every
//                             factor <= 1, so an underflow drops only terms
//                             below the smallest normal float
//   e^G o K, e^G o Q          Kr o 2^(G7_R), Qr o 2^(G7_R)
//   Ktil                      Kc o 2^(Glast - G7_R)
// (G: cumulative log2 decay from the chunk start; G7_R, Gend_R: at row 7 and
// at the last row of block R).  Pad rows (t >= T) are replaced by zeros with
// selects before any arithmetic, so NaN or inf there never reaches a result.
#include "kda_common.h"
#include "kda_front_end.h"
#include "kda_internal.h"

namespace kda {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int C>
struct ChunkGeom {
    static constexpr int kTiles = C / 16;      // 16-row tiles per chunk
    static constexpr int kLd = kD + 4;         // LDS row stride of [C][128] tables (floats)
    static constexpr int kLdc = C + 4;         // LDS row stride of [C][C] tables
    static constexpr size_t kOffW = 0;                      // W     A tiles [C/16][8]
    static constexpr size_t kOffU = (size_t)C * kD;         // U     accumulator tiles [C/16][8]
    static constexpr size_t kOffP = 2 * (size_t)C * kD;     // P     A tiles [C/16][8]
    static constexpr size_t kOffR = 3 * (size_t)C * kD;     // R     accumulator tiles [C/16][8]
    static constexpr size_t kOffKt = 4 * (size_t)C * kD;    // Ktil^T A tiles [8][C/16]
    static constexpr size_t kOffGam = 5 * (size_t)C * kD;   // gamma [128]
    static constexpr size_t kRecord = kOffGam + kD;
    static constexpr int kPairs = kTiles * (kTiles + 1) / 2;
    static_assert(kRecord == chunk_record_floats(C), "record layout");
};

__device__ __forceinline__ float4 lds4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// Where the inputs of one chunk record are, and which record it is.  Rows are
// [token][head] rows of 128 floats: row0 = first token * heads + head.  nvalid
// = tokens of the sequence in the chunk (the rest are selected away); span =
// rows readable from row0 before the end of the input buffers, at most
// C * heads; rec = the record's index in the workspace.
struct ChunkPos {
    size_t row0;
    int nvalid;
    int span;
    int rec;
    int b, t0, h;  // sequence, first token of the chunk within it, head (for the fused front end)
    size_t tok0;   // the sequence's first token in the token stream of the front end's inputs
    int len;       // the sequence's length
};
// One (sequence, head) of the scan: its first token, its length, its chunks
// and the index of its first record.
struct SeqPos {
    size_t tok0;
    int T;
    int nchunks;
    size_t rec0;
};

// Sequences of one common length T, each padded to t_pad = nchunks * C rows:
// inputs [B][t_pad][heads][128]; records stored in (sequence, head, chunk)
// order.  The prepare takes them in (sequence, chunk, head) order: the records
// in flight at one time then read every head of a run of consecutive tokens,
// a dense region of the inputs, rather than every chunk of a few heads,
// 512-byte rows scattered over the whole sequence.
struct DenseLayout {
    int heads, T, t_pad, nchunks, n_total;
    __device__ int records() const { return n_total; }
    template <int C>
    __device__ ChunkPos chunk(int i) const  // i-th record in processing order
    {
        const int per_seq = nchunks * heads;
        const int b = i / per_seq, c = (i % per_seq) / heads, h = i % heads;
        ChunkPos p;
        p.row0 = ((size_t)b * t_pad + (size_t)c * C) * heads + h;
        p.nvalid = T - c * C < C ? T - c * C : C;
        p.span = C * heads;
        p.rec = (b * heads + h) * nchunks + c;
        p.b = b;
        p.t0 = c * C;
        p.h = h;
        p.tok0 = (size_t)b * T;
        p.len = T;
        return p;
    }
    __device__ SeqPos seq(int bh) const
    {
        return {(size_t)(bh / heads) * t_pad, T, nchunks, (size_t)bh * nchunks};
    }
};

// Sequences of their own lengths packed back to back: inputs [total][heads][128],
// sequence s at tokens cu[s] .. cu[s + 1] - 1; cb[s] = chunks of the sequences
// before s; records stored in (sequence, head, chunk) order and prepared in
// (sequence, chunk, head) order, as for DenseLayout.  cu and cb are the
// clamped, non-decreasing copies the setup kernel writes into the workspace.
struct VarlenLayout {
    int heads, total, n_seqs;
    const int* cu;
    const int* cb;
    __device__ int records() const { return cb[n_seqs] * heads; }
    template <int C>
    __device__ ChunkPos chunk(int i) const  // i-th record in processing order
    {
        // the sequence: the last s with cb[s] <= i / heads (it has at least one chunk)
        const int x = i / heads;
        int lo = 0, hi = n_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (cb[mid] <= x) lo = mid;
            else hi = mid - 1;
        }
        const int ns = cb[lo + 1] - cb[lo], local = i - cb[lo] * heads;
        const int c = local / heads, h = local % heads;
        const int tok = cu[lo] + c * C, len = cu[lo + 1] - cu[lo];
        ChunkPos p;
        p.row0 = (size_t)tok * heads + h;
        p.nvalid = len - c * C < C ? len - c * C : C;
        const long long left = (long long)(total - tok) * heads - h;
        p.span = left < C * heads ? (int)left : C * heads;
        p.rec = cb[lo] * heads + h * ns + c;
        p.b = lo;
        p.t0 = c * C;
        p.h = h;
        p.tok0 = (size_t)cu[lo];
        p.len = len;
        return p;
    }
    __device__ SeqPos seq(int bh) const
    {
        const int s = bh / heads, h = bh % heads;
        const int ns = cb[s + 1] - cb[s];
        return {(size_t)cu[s], cu[s + 1] - cu[s], ns, (size_t)cb[s] * heads + (size_t)h * ns};
    }
};
__device__ __forceinline__ void lds4_st(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ float comp(const float4& v, int e)
{
    return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
}

// A-operand tile order.  A matrix stored as 16x16 tiles, tile t = a * n_cols + b
// covering rows 16a.. and columns 16b.., each tile as [lane][4]: lane l holds
// the four consecutive columns 16b + 4 (l / 16) + 0..3 of row 16a + l % 16, which
// is what lane l feeds to four successive 16x16x4 MFMA steps.  A wave then
// loads one tile with a single contiguous 1 KiB access.
__device__ __forceinline__ size_t atile_index(int tile, int row_in, int col_in)
{
    const int lane = (col_in >> 2) * 16 + row_in;
    return ((size_t)tile * 64 + lane) * 4 + (col_in & 3);
}
// inverse: element e of an A-tiled matrix with n_cols column tiles -> (row, col)
__device__ __forceinline__ void atile_coords(int e, int n_cols, int& row, int& col)
{
    const int tile = e >> 8, lane = (e >> 2) & 63;
    row = (tile / n_cols) * 16 + (lane & 15);
    col = (tile % n_cols) * 16 + (lane >> 4) * 4 + (e & 3);
}

constexpr int kPrepThreads = 512;  // 8 waves: one per 16-column block in the W/U stage

__device__ __forceinline__ uint2 buf_ld_b64(rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

// Inputs of one chunk as one thread of chunk_prepare loads them.  With kda_gate inside the prepare (kGate), gr holds the BF16 g_raw pieces in
// place of g, dt the thread's four dt_bias values and a_log the head's a_log;
// beta then holds the logit.
template <int C>
struct PrepInputs {
    static constexpr int NV4 = C * 32 / kPrepThreads;
    float4 k[NV4], q[NV4], g[NV4];  // row-major [C][128] pieces
    float beta;
    uint2 gr[NV4];
    float4 dt;
    float a_log;
};

// With BF16 q, k, v: the k and q pieces of the chunk being staged as loaded (four
// BF16 values each) and this chunk's v values, raw; empty for FP32 inputs.
template <int C, bool kB16>
struct PrepRaw16 {
};
template <int C>
struct PrepRaw16<C, true> {
    uint2 kb[PrepInputs<C>::NV4], qb[PrepInputs<C>::NV4];
    unsigned short vr[C / 16][4];
};

// Raw buffer descriptors over the rows of one chunk of one (sequence, head) in
// each input, from row p.row0 and p.span rows long (rows past the end of the
// buffers read as zeros).  With `live` false the descriptors cover zero bytes:
// loads through them return zeros without touching memory, so a wave can
// issue its usual load sequence for no chunk.
struct PrepSrc {
    rsrc_t q, k, g, v, b;
};
__device__ __forceinline__ PrepSrc prep_src(const float* q, const float* k, const float* v, const float* gate,
                                            const float* beta, const ChunkPos& p, bool live = true)
{
    const uint32_t vec = live ? (uint32_t)p.span * (kD * 4) : 0u, sca = live ? (uint32_t)p.span * 4 : 0u;
    const size_t row0 = p.row0;
    return {make_rsrc(q + row0 * kD, vec), make_rsrc(k + row0 * kD, vec), make_rsrc(gate + row0 * kD, vec),
            make_rsrc(v + row0 * kD, vec), make_rsrc(beta + row0, sca)};
}

// One row-major input of a chunk as thread tid holds it: rows tid/32 + 16 i,
// columns 4 (tid % 32) + 0..3.  Pad rows are loaded like the others and masked
// when staged.
template <int C>
__device__ __forceinline__ void prep_load_part(float4 (&dst)[PrepInputs<C>::NV4], rsrc_t src, int heads, int tid)
{
    const int voff = ((tid >> 5) * heads * kD + (tid & 31) * 4) * 4;
#pragma unroll
    for (int i = 0; i < PrepInputs<C>::NV4; ++i) dst[i] = buf_ld4(src, voff, i * 16 * heads * kD * 4);
}
template <int C>
__device__ __forceinline__ float prep_load_beta(rsrc_t src, int heads, int tid)
{
    return tid < C ? buf_ld1(src, tid * heads * 4, 0) : 0.f;
}

// BF16 q, k, v packed per token as [tokens][3][heads][128] (the FP32 forms'
// rows with the three parts side by side): descriptors over part `part` of
// head p.h for the tokens the chunk can read (p.span rows of the FP32 layout:
// C tokens, fewer at the end of packed sequences), 3 heads 128 values apart
// from token to token.
template <int C>
__device__ __forceinline__ rsrc_t prep_src_b16(const unsigned short* qkv, int part, int heads, const ChunkPos& p,
                                               bool live)
{
    const size_t tok = (p.row0 - (size_t)p.h) / (size_t)heads;             // the chunk's first token
    const size_t avail = ((size_t)p.span + (size_t)p.h) / (size_t)heads;   // tokens from there to the end
    const size_t base = (tok * 3 + (size_t)part) * heads * kD + (size_t)p.h * kD;
    const uint32_t bytes = live && avail ? (uint32_t)(((avail - 1) * 3 * heads * kD + kD) * 2) : 0u;
    return make_rsrc(qkv + base, bytes);
}
// prep_load_part for BF16 rows: the same pieces (rows tid/32 + 16 i, columns 4 (tid % 32) + 0..3), 8 bytes each
template <int C>
__device__ __forceinline__ void prep_load_part_b16(uint2 (&dst)[PrepInputs<C>::NV4], rsrc_t src, int heads, int tid)
{
    const int voff = ((tid >> 5) * 3 * heads * kD + (tid & 31) * 4) * 2;
#pragma unroll
    for (int i = 0; i < PrepInputs<C>::NV4; ++i) dst[i] = buf_ld_b64(src, voff, i * 16 * 3 * heads * kD * 2);
}
__device__ __forceinline__ float4 bf16x4(uint2 u)
{
    return make_float4(bf16_to_f32(u.x & 0xffffu), bf16_to_f32(u.x >> 16), bf16_to_f32(u.y & 0xffffu),
                       bf16_to_f32(u.y >> 16));
}

// kGate: the g_raw pieces of the thread's gate rows (BF16, 8 bytes per row: columns 4 (tid % 32) +
// 0..3), its four dt_bias values and the head's a_log.  live false: the g_raw descriptor covers
// zero bytes (loads return zeros) and the parameters are those of head p.h as ever.
template <int C>
__device__ __forceinline__ void prep_load_gate(PrepInputs<C>& in, const GateParams& gp, const ChunkPos& p, int heads,
                                               int tid, bool live = true)
{
    const rsrc_t src = make_rsrc(gp.g_raw + p.row0 * kD, live ? (uint32_t)p.span * (kD * 2) : 0u);
    const int voff = ((tid >> 5) * heads * kD + (tid & 31) * 4) * 2;
#pragma unroll
    for (int i = 0; i < PrepInputs<C>::NV4; ++i) in.gr[i] = buf_ld_b64(src, voff, i * 16 * heads * kD * 2);
    in.dt = ld4(gp.dt_bias + p.h * kD + 4 * (tid & 31));
    in.a_log = gp.a_log[p.h];
}

// V of one chunk in the B-operand layout of this wave's U tiles (rows
// 16 y + 4 q4 + e, column 16 wave + l16).  Rows >= T are selected away where
// the values are used, so that nothing here waits for the loads.
template <int C>
__device__ __forceinline__ void prep_load_v(float (&vb)[C / 16][4], rsrc_t src, int heads, int wave, int l16, int q4)
{
    const int voff = (4 * q4 * heads * kD + 16 * wave + l16) * 4;
#pragma unroll
    for (int y = 0; y < C / 16; ++y)
#pragma unroll
        for (int e = 0; e < 4; ++e) vb[y][e] = buf_ld1(src, voff, (16 * y + e) * heads * kD * 4);
}
// prep_load_v for BF16 rows: the raw values, widened where they are used
template <int C>
__device__ __forceinline__ void prep_load_v_b16(unsigned short (&vr)[C / 16][4], rsrc_t src, int heads, int wave,
                                                int l16, int q4)
{
    const int voff = (4 * q4 * 3 * heads * kD + 16 * wave + l16) * 2;
#pragma unroll
    for (int y = 0; y < C / 16; ++y)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            vr[y][e] = __builtin_amdgcn_raw_buffer_load_b16(src, voff, (16 * y + e) * 3 * heads * kD * 2, 0);
}

// Rows >= T (nvalid and beyond) are replaced by zeros with selects, then the
// chunk goes to LDS (gate in log2 units).
// kFE: k and q are in the fused row order (rows NV4 (tid / 32) + i), the gate
// in the usual one.
// index of block pair (R, S < R) among the pairs below the diagonal
__device__ __forceinline__ int below_index(int R, int S) { return R * (R - 1) / 2 + S; }

// The decayed tables of the fast path (factors about row 7 of each 16-row
// block, spanning up to 8 gates) stay inside the normal FP32 range, with room
// for small key and query components, while every gate of the chunk is at or
// above -kFastGateLog2 in log2 units (about -8.3 in natural units): 8 gates
// then span at most 2^96.  A chunk with a steeper gate takes the steep-gate
// path instead (see chunk_prepare_kernel).
constexpr float kFastGateLog2 = 12.f;
// On the steep-gate path every log2 gate below -kSteepGateClampLog2 counts as
// that value (about -19.4 in natural units): a decay factor of 2^-28 instead of
// a smaller one, a change below 2^-28 of the decayed state, far under FP32's
// own rounding of the terms it is added to.  It bounds the factors of the
// diagonal blocks (4 gates about a reference row) by 2^112.
constexpr float kSteepGateClampLog2 = 28.f;

// Rows >= T (nvalid and beyond) are replaced by zeros with selects, then the
// chunk goes to LDS (gate in log2 units).  Each wave also records in
// sSteep[wave] whether any gate it staged is below -kFastGateLog2 (log2).
// kFE: k and q are in the fused row order (rows NV4 (tid / 32) + i), the gate
// in the usual one.
// kGate: the gate is kda_gate of the g_raw pieces (with `lower`) and beta the sigmoid of the logit.
// kB16: k and q are BF16 pieces (kb, qb), widened exactly here.
template <int C, bool kFE = false, bool kGate = false, bool kB16 = false>
__device__ __forceinline__ void prep_stage(const PrepInputs<C>& in, float* sK, float* sQ, float* sL, float* sBeta,
                                           int* sSteep, int nvalid, int tid, float lower = 0.f,
                                           const PrepRaw16<C, kB16>& raw = {})
{
    using G = ChunkGeom<C>;
    constexpr int NV4 = PrepInputs<C>::NV4, LD = G::kLd;
    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
    bool steep = false;
    const float rate = kGate ? exp2_fast(kLog2e * in.a_log) : 0.f;
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
        const int e = tid + kPrepThreads * i, r = e >> 5, c4 = (e & 31) * 4;
        const bool ok = r < nvalid;
        const int rq = kFE ? NV4 * (tid >> 5) + i : r;
        const bool okq = rq < nvalid;
        if constexpr (kB16) {
            lds4_st(&sK[rq * LD + c4], okq ? bf16x4(raw.kb[i]) : z4);
            lds4_st(&sQ[rq * LD + c4], okq ? bf16x4(raw.qb[i]) : z4);
        } else {
            lds4_st(&sK[rq * LD + c4], okq ? in.k[i] : z4);
            lds4_st(&sQ[rq * LD + c4], okq ? in.q[i] : z4);
        }
        float4 g;
        if constexpr (kGate) {
            const uint2 u = in.gr[i];
            g = make_float4(kda_gate_f32(bf16_to_f32(u.x & 0xffffu), in.dt.x, rate, lower),
                            kda_gate_f32(bf16_to_f32(u.x >> 16), in.dt.y, rate, lower),
                            kda_gate_f32(bf16_to_f32(u.y & 0xffffu), in.dt.z, rate, lower),
                            kda_gate_f32(bf16_to_f32(u.y >> 16), in.dt.w, rate, lower));
        } else {
            g = in.g[i];
        }
        // per-component selects (a select of whole float4 values went through scratch memory)
        const float4 l = make_float4(ok ? g.x * kLog2e : 0.f, ok ? g.y * kLog2e : 0.f, ok ? g.z * kLog2e : 0.f,
                                     ok ? g.w * kLog2e : 0.f);
        steep |= (l.x < -kFastGateLog2) | (l.y < -kFastGateLog2) | (l.z < -kFastGateLog2) | (l.w < -kFastGateLog2);
        lds4_st(&sL[r * LD + c4], l);
    }
    if (tid < C) sBeta[tid] = tid < nvalid ? (kGate ? sigmoid_f32(in.beta) : in.beta) : 0.f;
    const bool any = __builtin_amdgcn_ballot_w64(steep) != 0;
    if ((tid & 63) == 0) sSteep[tid >> 6] = any ? 1 : 0;
}

// Steep-gate path.  The LDS tables hold K and Q as staged and L, the
// block-local cumulative log2 decay (clamped gates), and every operand is
// decayed by one exponential of an exponent sum, each <= 0 except on the
// diagonal blocks (below):
//   pair S < R   row r:    K o 2^(L_r + sX_RS),  sX_RS = sum of the block totals strictly between S and R
//                column s: K o 2^(sY_S - L_s),   sY_S  = block total of S
// (both equal the fast path's operands decayed about the last row of block S).
template <int C, int TAU0, int TAU1>
__device__ __forceinline__ void am_below_steep(int R, int S, const float* sK, const float* sQ, const float* sL,
                                               const float* sX, const float* sY, int l16, int q4, floatx4& accA,
                                               floatx4& accM)
{
    constexpr int LD = ChunkGeom<C>::kLd;
    const int ra = 16 * R + l16, sb = 16 * S + l16;
    const float* const xv = sX + below_index(R, S) * kD;
    const float* const yv = sY + S * kD;
#pragma unroll
    for (int tau = TAU0; tau < TAU1; ++tau) {
        const int i0 = 16 * tau + 4 * q4;
        const float4 kr = lds4(&sK[ra * LD + i0]), qr = lds4(&sQ[ra * LD + i0]), lr = lds4(&sL[ra * LD + i0]);
        const float4 ks = lds4(&sK[sb * LD + i0]), ls = lds4(&sL[sb * LD + i0]);
        const float4 x = lds4(&xv[i0]), y = lds4(&yv[i0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float fa = exp2_fast(comp(lr, e) + comp(x, e)), fb = exp2_fast(comp(y, e) - comp(ls, e));
            const float b = comp(ks, e) * fb;
            accA = mfma4(comp(kr, e) * fa, b, accA);
            accM = mfma4(comp(qr, e) * fa, b, accM);
        }
    }
}

// Steep-gate path, diagonal block R: no single reference row keeps both
// factors of every pair s <= r in range, so two products are taken and
// selected per element.  Pairs inside one 8-row half use that half's row 3 as
// the reference (factors span at most 4 gates, so with clamped gates at most
// 2^112); pairs across the halves (r in rows 8..15, s in rows 0..7) use row 7,
// the boundary, where both factors are <= 1.  The rows and columns a product
// must not use are selected to zero; the cross-half elements of the first
// product can overflow and are discarded by the select.
template <int C>
__device__ __forceinline__ void am_diag_steep(int R, const float* sK, const float* sQ, const float* sL, int l16,
                                              int q4, floatx4& accA, floatx4& accM)
{
    constexpr int LD = ChunkGeom<C>::kLd;
    const int ra = 16 * R + l16, half = l16 >> 3;
    const int ref = 16 * R + 3 + 8 * half, mid = 16 * R + 7;
    floatx4 a2 = {0.f, 0.f, 0.f, 0.f}, m2 = {0.f, 0.f, 0.f, 0.f};
    floatx4 a1 = {0.f, 0.f, 0.f, 0.f}, m1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tau = 0; tau < 8; ++tau) {
        const int i0 = 16 * tau + 4 * q4;
        const float4 kr = lds4(&sK[ra * LD + i0]), qr = lds4(&sQ[ra * LD + i0]), lr = lds4(&sL[ra * LD + i0]);
        const float4 lref = lds4(&sL[ref * LD + i0]), lmid = lds4(&sL[mid * LD + i0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // the A operand is row ra of this lane, the B operand column ra: the same K row
            const float k = comp(kr, e), q = comp(qr, e), l = comp(lr, e);
            const float f2a = exp2_fast(l - comp(lref, e)), f2b = exp2_fast(comp(lref, e) - l);
            const float f1a = half ? exp2_fast(l - comp(lmid, e)) : 0.f;
            const float f1b = half ? 0.f : exp2_fast(comp(lmid, e) - l);
            a2 = mfma4(k * f2a, k * f2b, a2);
            m2 = mfma4(q * f2a, k * f2b, m2);
            a1 = mfma4(k * f1a, k * f1b, a1);
            m1 = mfma4(q * f1a, k * f1b, m1);
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bool same = ((4 * q4 + e) >> 3) == half;  // row 4 q4 + e and column l16 of the block
        accA[e] = same ? a2[e] : a1[e];
        accM[e] = same ? m2[e] : m1[e];
    }
}


// Partial A and M tile of block pair (R, S <= R) over the channel steps
// [16 TAU0, 16 TAU1), from the decayed tables: lane l accumulates rows
// 16R + 4(l/16) + e, columns 16S + l%16.
template <int C, int TAU0, int TAU1>
__device__ __forceinline__ void am_pair(int R, int S, const float* sKr, const float* sQr, const float* sKc,
                                        const float* sX, const float* sY, int l16, int q4, floatx4& accA,
                                        floatx4& accM)
{
    constexpr int LD = ChunkGeom<C>::kLd;
    const int ra = 16 * R + l16, sb = 16 * S + l16;
    const float* const xv = sX + (S < R ? below_index(R, S) : 0) * kD;
#pragma unroll
    for (int tau = TAU0; tau < TAU1; ++tau) {
        const int i0 = 16 * tau + 4 * q4;
        float4 kr = lds4(&sKr[ra * LD + i0]);
        float4 qr = lds4(&sQr[ra * LD + i0]);
        float4 kc = lds4(&sKc[sb * LD + i0]);
        if (S < R) {
            // move both factors to the last row of block S
            const float4 x = lds4(&xv[i0]);
            const float4 y = lds4(&sY[S * kD + i0]);
            kr = make_float4(kr.x * x.x, kr.y * x.y, kr.z * x.z, kr.w * x.w);
            qr = make_float4(qr.x * x.x, qr.y * x.y, qr.z * x.z, qr.w * x.w);
            kc = make_float4(kc.x * y.x, kc.y * y.y, kc.z * y.z, kc.w * y.w);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            accA = mfma4(comp(kr, e), comp(kc, e), accA);
            accM = mfma4(comp(qr, e), comp(kc, e), accM);
        }
    }
}

// beta row scaling and the triangular masks, then A and M tiles to LDS
template <int C>
__device__ __forceinline__ void am_store(int R, int S, const floatx4& accA, const floatx4& accM, float* sA,
                                         float* sM, const float* sBeta, int l16, int q4)
{
    constexpr int LDC = ChunkGeom<C>::kLdc;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = 16 * R + 4 * q4 + e, s = 16 * S + l16;
        sA[r * LDC + s] = (S < R || s < r) ? sBeta[r] * accA[e] : 0.f;
        sM[r * LDC + s] = (S < R || s <= r) ? accM[e] : 0.f;
    }
}

// An accumulator tile (lane l, element e = row 4(l/16) + e, column l%16) rewritten
// in A-tile lane order (lane L = row L%16, columns 4(L/16) + 0..3) through a
// wave-private 1 KiB LDS scratch, so the tile leaves with one float4 store per
// lane.  Lane L's four values sit in float4 slot L ^ (2 (L >> 4) + ((L >> 3) & 1))
// rather than slot L: each scalar write of the 64 lanes then spreads over all
// banks instead of 8 of them, and the float4 read back stays conflict-free.
__device__ __forceinline__ int atile_slot(int L) { return L ^ (2 * (L >> 4) + ((L >> 3) & 1)); }

__device__ __forceinline__ float4 acc_to_atile(const floatx4& acc, float* scratch, int lane)
{
    const int l16 = lane & 15, q4 = lane >> 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        // element (row 4 q4 + e, column l16) belongs to A-lane (l16 / 4) * 16 + 4 q4 + e, position l16 % 4
        scratch[atile_slot((l16 >> 2) * 16 + 4 * q4 + e) * 4 + (l16 & 3)] = acc[e];
    }
    __builtin_amdgcn_wave_barrier();
    const float4 r = lds4(&scratch[atile_slot(lane) * 4]);
    __builtin_amdgcn_wave_barrier();
    return r;
}

// block pair (R, S < R) with below-diagonal index j (the inverse of below_index)
__device__ __forceinline__ void below_pair(int j, int& R, int& S)
{
    R = 1;
    while (R * (R + 1) / 2 <= j) ++R;
    S = j - R * (R - 1) / 2;
}

// Record stores of chunk_prepare are non-temporal: a prefill's records are
// written once and read back by the scan only after the whole prepare, by which
// time the caches hold the last records written, not the first ones the scan
// wants (T=8192, H=32: 673 MB of records).  Streaming them past the caches made
// the T=8192 prefill 3.8% faster.
__device__ __forceinline__ void rec_st4(float* p, float4 v)
{
    __builtin_nontemporal_store(floatx4{v.x, v.y, v.z, v.w}, reinterpret_cast<floatx4*>(p));
}

// ---------------------------------------------------------------------------
// Front end fused into the prepare (dense layout, conv_kernel 4).  Instead of
// FP32 q, k, v rows the prepare reads the BF16 projections q | k | v
// [B][T][3][H][128] (workspace page, qkv_proj), and computes for every staged
// row the front end of the module page's pipeline line: the depthwise causal
// conv over the token and the three before it (conv weights [3 H 128][4]
// BF16, slot 3 the newest; tokens before the call from the conv state
// [B][3 H 128][4] FP32), SiLU, and for q and k the scale 1 / sqrt(sum y^2 +
// l2_eps) over the head's 128 channels.  q and k are formed in the staging
// layout (32 lanes of a wave hold one row, 4 channels each; the sum of
// squares is FP64, reduced over those 32 lanes), v directly in the B-operand
// layout of the U tiles.  The conv state itself is advanced by a separate
// launch after the whole prefill.
struct FeSrc {
    const unsigned short* qkv;     // [tokens][3][H][128] BF16: sequence b at rows tok0 .. tok0 + len - 1
    const unsigned short* conv_w;  // [3 H 128][4] BF16
    const float* conv_state;       // [sequences][3 H 128][4] FP32, read only here
    double eps;                    // l2_eps
};
constexpr int kFeK = 4;  // conv taps of the fused form

__device__ __forceinline__ uint4 buf_ld_b128u(rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ float fe_bf16(unsigned w, int half) { return bf16_to_f32(half ? (w >> 16) : (w & 0xffffu)); }
__device__ __forceinline__ float fe_silu(float a)
{
    return a * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504f * a));
}

// The raw inputs of q or k for the rows one thread stages in the fused form:
// NV4 consecutive rows NV4 (tid / 32) + i of the chunk (not the rows tid / 32
// + 16 i of the unfused staging), so that one window of NV4 + kFeK - 1 input
// rows, channels 4 (tid % 32) + 0..3, feeds all their taps; the conv state of
// those channels (for the first chunk of a sequence, else not read) and their
// weights.
template <int C>
struct FeRaw {
    static constexpr int NW = PrepInputs<C>::NV4 + kFeK - 1;  // window rows
    uint2 x[NW];
    float4 st[4];
    uint4 w[2];
};

// live false: descriptors of zero bytes (loads return zeros, touch nothing)
template <int C>
__device__ __forceinline__ void fe_load_qk(FeRaw<C>& r, const FeSrc& fe, int part, const ChunkPos& p, int heads,
                                           int tid, bool live)
{
    const int rowbytes = 3 * heads * kD * 2;
    const int col = 4 * (tid & 31);
    const int ch = (part * heads + p.h) * kD + col;  // first channel of the four
    const rsrc_t src = make_rsrc(fe.qkv + p.tok0 * 3 * heads * kD, live ? (uint32_t)p.len * rowbytes : 0u);
#pragma unroll
    for (int m = 0; m < FeRaw<C>::NW; ++m) {
        // rows before the call (t < 0) wrap to offsets at or above 2^31 and rows at or past T
        // reach the size: both read zeros
        const int t = p.t0 + PrepInputs<C>::NV4 * (tid >> 5) - (kFeK - 1) + m;
        r.x[m] = buf_ld_b64(src, (int)((uint32_t)t * (uint32_t)rowbytes + (uint32_t)(ch * 2)), 0);
    }
    // descriptors over the head's 128 channels (wave-uniform), the lane's channels as offsets
    const int ch0 = (part * heads + p.h) * kD;
    const rsrc_t ss = make_rsrc(fe.conv_state + ((size_t)p.b * 3 * heads * kD + ch0) * kFeK,
                                live && p.t0 == 0 ? (uint32_t)kD * kFeK * 4u : 0u);
#pragma unroll
    for (int j = 0; j < 4; ++j) r.st[j] = buf_ld4(ss, (col + j) * kFeK * 4, 0);
    const rsrc_t ws = make_rsrc(fe.conv_w + (size_t)ch0 * kFeK, live ? (uint32_t)kD * kFeK * 2u : 0u);
    r.w[0] = buf_ld_b128u(ws, col * kFeK * 2, 0);
    r.w[1] = buf_ld_b128u(ws, col * kFeK * 2, 16);
}

// conv, SiLU and the per-row scale 1 / sqrt(sum y^2 + eps) for the rows of k
// and q (FeRaw), to the float4 pieces prep_stage takes (in the fused row
// order).  The sum of squares is FP64, reduced over the 32 lanes of each half
// of a wave (quads, eights, rows of 16 by DPP, then row 0 into row 1 and row 2
// into row 3 through the row broadcast of lane 15); the 2 NV4 rows' reductions
// are taken step by step side by side, independent chains the scheduler
// overlaps.
template <int C>
__device__ __forceinline__ void fe_finish_kq(const FeRaw<C>& rk, const FeRaw<C>& rq, float4 (&ok)[PrepInputs<C>::NV4],
                                             float4 (&oq)[PrepInputs<C>::NV4], int t0, int tid, double eps)
{
    constexpr int NV4 = PrepInputs<C>::NV4, N = 2 * NV4;
    const int lane = tid & 63;
    float y[N][4];
    double x[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const FeRaw<C>& r = n < NV4 ? rk : rq;
        const int i = n % NV4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const unsigned wj0 = j < 2 ? (j == 0 ? r.w[0].x : r.w[0].z) : (j == 2 ? r.w[1].x : r.w[1].z);
            const unsigned wj1 = j < 2 ? (j == 0 ? r.w[0].y : r.w[0].w) : (j == 2 ? r.w[1].y : r.w[1].w);
            float a = 0.f;
#pragma unroll
            for (int k = 0; k < kFeK; ++k) {
                const int t = t0 + NV4 * (tid >> 5) + i - (kFeK - 1) + k;
                float xv = fe_bf16(j < 2 ? r.x[i + k].x : r.x[i + k].y, j & 1);
                if (i + k + 1 < kFeK && t0 == 0) {
                    const float sv = t == -3 ? r.st[j].y : (t == -2 ? r.st[j].z : r.st[j].w);
                    xv = t < 0 ? sv : xv;
                }
                const float w = fe_bf16(k < 2 ? wj0 : wj1, k & 1);
                a = k == 0 ? w * xv : fmaf(w, xv, a);
            }
            y[n][j] = fe_silu(a);
        }
        x[n] = (double)y[n][0] * y[n][0] + (double)y[n][1] * y[n][1] + (double)y[n][2] * y[n][2] +
               (double)y[n][3] * y[n][3];
    }
    // the reduction steps, each over all rows before the next
#pragma unroll
    for (int n = 0; n < N; ++n) x[n] += dpp_f64<0xB1>(x[n]);
#pragma unroll
    for (int n = 0; n < N; ++n) x[n] += dpp_f64<0x4E>(x[n]);
#pragma unroll
    for (int n = 0; n < N; ++n) x[n] += dpp_f64<0x141>(x[n]);
#pragma unroll
    for (int n = 0; n < N; ++n) x[n] += dpp_f64<0x140>(x[n]);
#pragma unroll
    for (int n = 0; n < N; ++n) x[n] += dpp_f64<0x142, 0xa>(x[n]);
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const unsigned long long u = (unsigned long long)__double_as_longlong(x[n]);
        const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)u, 31);
        const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(u >> 32), 31);
        const unsigned lo2 = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)u, 63);
        const unsigned hi2 = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(u >> 32), 63);
        const unsigned a = lane < 32 ? lo : lo2, b = lane < 32 ? hi : hi2;
        const double tot = __longlong_as_double((long long)(((unsigned long long)b << 32) | a)) + eps;
        double rs = __builtin_amdgcn_rsq(tot);
        rs = rs * (1.5 - 0.5 * (tot * rs) * rs);  // one Newton step
        const float4 o = make_float4((float)(y[n][0] * rs), (float)(y[n][1] * rs), (float)(y[n][2] * rs),
                                     (float)(y[n][3] * rs));
        if (n < NV4) ok[n % NV4] = o;
        else oq[n % NV4] = o;
    }
}

// v of the current chunk in the B-operand layout of this wave's U tiles
// (rows 16 y + 4 q4 + e, channel 16 wave + l16): the seven input rows
// 16 y + 4 q4 - 3 .. 16 y + 4 q4 + 3 per row block, the channel's conv state
// (first chunk only) and weights
template <int C>
struct FeV {
    unsigned short x[C / 16][7];
    float4 st;
    uint2 w;
};
template <int C>
__device__ __forceinline__ void fe_load_v(FeV<C>& r, const FeSrc& fe, const ChunkPos& p, int heads, int wave, int l16,
                                          int q4)
{
    const int rowbytes = 3 * heads * kD * 2;
    const int ch = (2 * heads + p.h) * kD + 16 * wave + l16;
    const rsrc_t src = make_rsrc(fe.qkv + p.tok0 * 3 * heads * kD, (uint32_t)p.len * rowbytes);
#pragma unroll
    for (int y = 0; y < C / 16; ++y)
#pragma unroll
        for (int j = 0; j < 7; ++j) {
            const int t = p.t0 + 16 * y + 4 * q4 - 3 + j;  // out of range as in fe_load_qk
            r.x[y][j] = __builtin_amdgcn_raw_buffer_load_b16(
                src, (int)((uint32_t)t * (uint32_t)rowbytes + (uint32_t)(ch * 2)), 0, 0);
        }
    // descriptors over the head's v channels (wave-uniform), the lane's channel as the offset
    const int ch0 = (2 * heads + p.h) * kD, cl = 16 * wave + l16;
    r.st = buf_ld4(make_rsrc(fe.conv_state + ((size_t)p.b * 3 * heads * kD + ch0) * kFeK,
                             p.t0 == 0 ? (uint32_t)kD * kFeK * 4u : 0u), cl * kFeK * 4, 0);
    r.w = buf_ld_b64(make_rsrc(fe.conv_w + (size_t)ch0 * kFeK, (uint32_t)kD * kFeK * 2u), cl * kFeK * 2, 0);
}
template <int C>
__device__ __forceinline__ void fe_finish_v(const FeV<C>& r, float (&vb)[C / 16][4], int t0, int q4)
{
#pragma unroll
    for (int y = 0; y < C / 16; ++y)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float a = 0.f;
#pragma unroll
            for (int k = 0; k < kFeK; ++k) {
                const int t = t0 + 16 * y + 4 * q4 + e - (kFeK - 1) + k;
                float x = bf16_to_f32(r.x[y][e + k]);
                if (y == 0 && e + k < kFeK - 1 && t0 == 0) {  // rows that can precede the call, as in fe_finish_kq
                    const float sv = t == -3 ? r.st.y : (t == -2 ? r.st.z : r.st.w);
                    x = t < 0 ? sv : x;
                }
                const float w = fe_bf16(k < 2 ? r.w.x : r.w.y, k & 1);
                a = k == 0 ? w * x : fmaf(w, x, a);
            }
            vb[y][e] = fe_silu(a);
        }
}

// Persistent: one workgroup per CU walks the records gc = blockIdx.x, +gridDim.x,
// ... of the layout's processing order (the layout gives each one's inputs and
// its place in the workspace).  The inputs of the next chunk are read into
// registers while the current one is computed and are staged into LDS at its
// end.
//
// kFE: the front end is fused in (dense layout): q, k and v are formed from
// the BF16 projections in `fe` (see FeSrc) instead of read as FP32 rows; the
// q, k, v pointers are then not read.
// kB16: q, k, v are BF16, packed per token as [B][T_pad][3][heads][128] (dense) or
// [total][3][heads][128] (packed sequences) at `q` (k and v unused), and widened
// exactly where they are staged.
template <int C, class Layout, bool kFE = false, bool kGate = false, bool kB16 = false>
__global__ __launch_bounds__(kPrepThreads) void chunk_prepare_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ gate, const float* __restrict__ beta, float* __restrict__ ws, int heads,
    Layout layout, FeSrc fe, GateParams gp)
{
    using G = ChunkGeom<C>;
    constexpr int NT = G::kTiles, LD = G::kLd, LDC = G::kLdc;
    constexpr int NW = kPrepThreads / 64;
    // block pairs below the diagonal: the first four whole on waves 0..3, the rest
    // in two channel halves on waves 0..2 kSplit-1; diagonal pair R on wave 4 + R
    constexpr int kBelow = NT * (NT - 1) / 2;
    constexpr int kSplit = kBelow > 4 ? kBelow - 4 : 0;
    constexpr int LDT = 20;  // row stride of the inverted diagonal blocks
    static_assert(PrepInputs<C>::NV4 >= 1 && NW == 8 && NT <= 4 && kSplit <= 2, "geometry");
    constexpr int NX = NT > 1 ? NT * (NT - 1) / 2 : 1;  // block pairs below the diagonal
    __shared__ float sKr[C * LD];    // K, then K o 2^(L - L7)
    __shared__ float sQr[C * LD];    // Q, then Q o 2^(L - L7)
    __shared__ float sKc[C * LD];    // log2 gates, then K o 2^(L7 - L); transpose scratch after step 3
    __shared__ float sA[C * LDC];    // beta-scaled strictly lower A
    __shared__ float sTd[NT * 16 * LDT];  // the inverted diagonal blocks (I + A_RR)^-1
    __shared__ floatx4 sPart[(kSplit > 0 ? kSplit : 1) * 2 * 64];  // first channel halves of the split pairs
    __shared__ float sM[C * LDC];    // lower-triangular decayed Q K^T
    __shared__ float sE[NT * kD];    // 2^(G7_R)          (L7 of each block during step 2)
    __shared__ float sF[NT * kD];    // 2^(Glast - G7_R)  (block totals during step 2)
    __shared__ float sY[NT * kD];    // 2^(Gend_R - G7_R)
    __shared__ float sX[NX * kD];    // 2^(G7_R - Gend_S), S < R
    __shared__ float sBeta[C];
    __shared__ int sSteep[NW];       // per wave: a staged gate below -kFastGateLog2 (log2)

    const int stride = gridDim.x;

    const int n_total = layout.records();
    int gc = blockIdx.x;
    PrepInputs<C> in;
    PrepRaw16<C, kB16> raw;
    ChunkPos pos;  // of the gc-th record in processing order
    if (gc < n_total) {
        pos = layout.template chunk<C>(gc);
        const PrepSrc src = prep_src(q, k, v, gate, beta, pos);
        if constexpr (kFE) {
            FeRaw<C> rk, rq;
            fe_load_qk<C>(rk, fe, 1, pos, heads, threadIdx.x, true);
            fe_load_qk<C>(rq, fe, 0, pos, heads, threadIdx.x, true);
            fe_finish_kq<C>(rk, rq, in.k, in.q, pos.t0, threadIdx.x, fe.eps);
        } else if constexpr (kB16) {
            const auto* qkv = reinterpret_cast<const unsigned short*>(q);
            prep_load_part_b16<C>(raw.kb, prep_src_b16<C>(qkv, 1, heads, pos, true), heads, threadIdx.x);
            prep_load_part_b16<C>(raw.qb, prep_src_b16<C>(qkv, 0, heads, pos, true), heads, threadIdx.x);
        } else {
            prep_load_part<C>(in.k, src.k, heads, threadIdx.x);
            prep_load_part<C>(in.q, src.q, heads, threadIdx.x);
        }
        if constexpr (kGate) prep_load_gate<C>(in, gp, pos, heads, threadIdx.x);
        else prep_load_part<C>(in.g, src.g, heads, threadIdx.x);
        in.beta = prep_load_beta<C>(src.b, heads, threadIdx.x);
        prep_stage<C, kFE, kGate, kB16>(in, sKr, sQr, sKc, sBeta, sSteep, pos.nvalid, threadIdx.x, gp.lower, raw);
    }
    __syncthreads();

    for (; gc < n_total; gc += stride) {
        // Lane indices re-derived behind an opaque copy: address arithmetic is
        // then recomputed in each phase instead of being hoisted out of the loop
        // (dozens of hoisted lane-dependent addresses would spill, and their
        // reloads would wait behind the in-flight loads of the next chunk).
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, l16 = lane & 15, q4 = lane >> 4;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        float* const rec = ws + (size_t)pos.rec * G::kRecord;
        float vb[NT][4];  // needed only at step 4c: its latency hides behind steps 2-4
        FeV<C> fv;        // (fused front end: the raw v inputs instead)
        if constexpr (kFE) fe_load_v<C>(fv, fe, pos, heads, wave, l16, q4);
        else if constexpr (kB16)
            prep_load_v_b16<C>(raw.vr, prep_src_b16<C>(reinterpret_cast<const unsigned short*>(q), 2, heads, pos, true),
                               heads, wave, l16, q4);
        else prep_load_v<C>(vb, prep_src(q, k, v, gate, beta, pos).v, heads, wave, l16, q4);
        const int nvalid = pos.nvalid;
        // The next chunk's inputs are read in three parts, at steps 3, 5 and 6,
        // so the vector-memory path takes them while the matrix cores work.
        // After a workgroup's last chunk the loads go through empty descriptors
        // instead of being branched around, which keeps every wave's load
        // sequence, and so its wait counts, fixed.
        const int gn = gc + stride;
        const ChunkPos npos = gn < n_total ? layout.template chunk<C>(gn) : pos;
        const PrepSrc nsrc = prep_src(q, k, v, gate, beta, npos, gn < n_total);

        // Whether any gate of this chunk is steeper than the fast path's tables allow
        // (uniform over the workgroup: the staging waves' flags, read into a scalar).
        int flags = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) flags |= sSteep[w];
        const bool steep = __builtin_amdgcn_readfirstlane(flags) != 0;
        if (steep) {
            // 2'. steep gates: L, the block-local cumulative log2 decay of each
            //     column with every gate clamped at -kSteepGateClampLog2, replaces
            //     the gates; K and Q stay as staged.  Block totals wait in sE.
            if (tid < NT * kD) {
                const int j = tid & (kD - 1), R = tid >> 7;
                float acc = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int o = (16 * R + r) * LD + j;
                    const float g = sKc[o];
                    acc += g < -kSteepGateClampLog2 ? -kSteepGateClampLog2 : g;  // (a NaN gate stays NaN)
                    sKc[o] = acc;
                }
                sE[R * kD + j] = acc;
            }
            __syncthreads();
            //    per-channel exponents (not factors): sE = the block totals before
            //    R, sF = those from R on (G_last - G_r = sF_R - L_r), sY = block
            //    total of S, sX = the totals strictly between S and R
            if (tid < kD) {
                float bl[NT];
#pragma unroll
                for (int R = 0; R < NT; ++R) bl[R] = sE[R * kD + tid];
                float pre = 0.f, tot = 0.f;
#pragma unroll
                for (int R = 0; R < NT; ++R) tot += bl[R];
#pragma unroll
                for (int R = 0; R < NT; ++R) {
                    sE[R * kD + tid] = pre;
                    sF[R * kD + tid] = tot - pre;
                    sY[R * kD + tid] = bl[R];
                    float mid = 0.f;
#pragma unroll
                    for (int S = R - 1; S >= 0; --S) {
                        sX[below_index(R, S) * kD + tid] = mid;
                        mid += bl[S];
                    }
                    pre += bl[R];
                }
                rec[G::kOffGam + tid] = exp2_fast(tot);  // gamma = e^{G_last}
            }
            __syncthreads();
        } else {
            // 2. block-local cumulative log2 decay L of each column, then the tables
            //    decayed about row 7 of the block (L7 and the block totals wait in sE, sF)
            if (tid < NT * kD) {
                const int j = tid & (kD - 1), R = tid >> 7;
                float L[16];
                float acc = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    acc += sKc[(16 * R + r) * LD + j];
                    L[r] = acc;
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int o = (16 * R + r) * LD + j;
                    const float er = exp2_fast(L[r] - L[7]), ec = exp2_fast(L[7] - L[r]);
                    const float kk = sKr[o];
                    sKr[o] = kk * er;
                    sQr[o] = sQr[o] * er;
                    sKc[o] = kk * ec;
                }
                sE[R * kD + j] = L[7];
                sF[R * kD + j] = L[15];
            }
            __syncthreads();
            //    per-channel factors, each exponent summed from block-local pieces
            if (tid < kD) {
                float l7[NT], bl[NT];
#pragma unroll
                for (int R = 0; R < NT; ++R) {
                    l7[R] = sE[R * kD + tid];
                    bl[R] = sF[R * kD + tid];
                }
                float pre = 0.f;
#pragma unroll
                for (int R = 0; R < NT; ++R) {
                    float suf = 0.f;
#pragma unroll
                    for (int X = R + 1; X < NT; ++X) suf += bl[X];
                    sE[R * kD + tid] = exp2_fast(pre + l7[R]);
                    sF[R * kD + tid] = exp2_fast((bl[R] - l7[R]) + suf);
                    sY[R * kD + tid] = exp2_fast(bl[R] - l7[R]);
                    float mid = 0.f;  // blocks strictly between S and R, summed from R down
#pragma unroll
                    for (int S = R - 1; S >= 0; --S) {
                        sX[below_index(R, S) * kD + tid] = exp2_fast(l7[R] + mid);
                        mid += bl[S];
                    }
                    pre += bl[R];
                }
                rec[G::kOffGam + tid] = exp2_fast(pre);  // gamma = e^{G_last}
            }
            __syncthreads();
        }

        // 3a. A and M on the 16x16 block pairs (R, S <= R).  Waves 4.. take the
        //     diagonal pairs and, as soon as their block of A is in LDS, invert
        //     it, (I + A_RR)^-1 by forward substitution (one lane per column),
        //     while waves 0..3 are still on the pairs below the diagonal.
        __builtin_amdgcn_sched_barrier(0);
        FeRaw<C> rk, rq;  // (fused front end: the next chunk's raw k and q)
        if constexpr (kFE) fe_load_qk<C>(rk, fe, 1, npos, heads, tid, gn < n_total);
        else if constexpr (kB16)
            prep_load_part_b16<C>(raw.kb,
                                  prep_src_b16<C>(reinterpret_cast<const unsigned short*>(q), 1, heads, npos,
                                                  gn < n_total),
                                  heads, tid);
        else prep_load_part<C>(in.k, nsrc.k, heads, tid);
        __builtin_amdgcn_sched_barrier(0);
        int R, S;
        if (wave >= 4) {
            R = S = wave - 4;
            if (R < NT) {
                floatx4 accA = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
                if (steep) am_diag_steep<C>(R, sKr, sQr, sKc, l16, q4, accA, accM);
                else am_pair<C, 0, 8>(R, S, sKr, sQr, sKc, sX, sY, l16, q4, accA, accM);
                am_store<C>(R, S, accA, accM, sA, sM, sBeta, l16, q4);
                __builtin_amdgcn_wave_barrier();  // the wave reads back the block it wrote
                if (lane < 16) {
                    const int base = 16 * R;
                    float x[16];
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        float acc = (i == lane) ? 1.f : 0.f;
#pragma unroll
                        for (int m = 0; m < i; ++m) acc = fmaf(-sA[(base + i) * LDC + base + m], x[m], acc);
                        x[i] = acc;
                    }
#pragma unroll
                    for (int i = 0; i < 16; ++i) sTd[(16 * R + i) * LDT + lane] = x[i];
                }
            }
        } else if (wave < kBelow) {
            floatx4 accA = {0.f, 0.f, 0.f, 0.f}, accM = {0.f, 0.f, 0.f, 0.f};
            below_pair(wave, R, S);
            if (steep) am_below_steep<C, 0, 8>(R, S, sKr, sQr, sKc, sX, sY, l16, q4, accA, accM);
            else am_pair<C, 0, 8>(R, S, sKr, sQr, sKc, sX, sY, l16, q4, accA, accM);
            am_store<C>(R, S, accA, accM, sA, sM, sBeta, l16, q4);
        }
        floatx4 hA = {0.f, 0.f, 0.f, 0.f}, hM = {0.f, 0.f, 0.f, 0.f};
        const bool split = wave < 2 * kSplit;
        if (split) {
            below_pair(4 + (wave >> 1), R, S);
            if (wave & 1) {
                if (steep) am_below_steep<C, 4, 8>(R, S, sKr, sQr, sKc, sX, sY, l16, q4, hA, hM);
                else am_pair<C, 4, 8>(R, S, sKr, sQr, sKc, sX, sY, l16, q4, hA, hM);
            } else {
                if (steep) am_below_steep<C, 0, 4>(R, S, sKr, sQr, sKc, sX, sY, l16, q4, hA, hM);
                else am_pair<C, 0, 4>(R, S, sKr, sQr, sKc, sX, sY, l16, q4, hA, hM);
                sPart[((wave >> 1) * 2 + 0) * 64 + lane] = hA;
                sPart[((wave >> 1) * 2 + 1) * 64 + lane] = hM;
            }
        }
        // 3b. Ktil^T = (e^{G_last - G} o K)^T as A tiles: wave w builds tiles (row
        //     block s of key channels, column block y of chunk rows) for s = w,
        //     one float4 store per lane (lane l: channel 16 s + l%16, rows 16 y + 4(l/16)..)
        //     (steep gates: K o 2^(G_last - G_r) directly, sF holding G_last - G at the block start;
        //     whole loops in each branch, so the fast path carries none of the steep path's work)
        auto ktil_put = [&](int y, const float4& o) {
            rec_st4(rec + G::kOffKt + ((size_t)(wave * NT + y) * 64 + lane) * 4, o);
        };
        if (steep) {
#pragma unroll
            for (int y = 0; y < NT; ++y) {
                const int i = 16 * wave + l16, r = 16 * y + 4 * q4;
                const float f = sF[y * kD + i];
                ktil_put(y, make_float4(sKr[r * LD + i] * exp2_fast(f - sKc[r * LD + i]),
                                        sKr[(r + 1) * LD + i] * exp2_fast(f - sKc[(r + 1) * LD + i]),
                                        sKr[(r + 2) * LD + i] * exp2_fast(f - sKc[(r + 2) * LD + i]),
                                        sKr[(r + 3) * LD + i] * exp2_fast(f - sKc[(r + 3) * LD + i])));
            }
        } else {
#pragma unroll
            for (int y = 0; y < NT; ++y) {
                const int i = 16 * wave + l16, r = 16 * y + 4 * q4;
                const float f = sF[y * kD + i];
                ktil_put(y, make_float4(sKc[r * LD + i] * f, sKc[(r + 1) * LD + i] * f, sKc[(r + 2) * LD + i] * f,
                                        sKc[(r + 3) * LD + i] * f));
            }
        }
        __syncthreads();
        // finish the split pairs
        if (split && (wave & 1)) {
            const floatx4 pa = sPart[((wave >> 1) * 2 + 0) * 64 + lane];
            const floatx4 pm = sPart[((wave >> 1) * 2 + 1) * 64 + lane];
            floatx4 a, m;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a[e] = pa[e] + hA[e];
                m[e] = pm[e] + hM[e];
            }
            am_store<C>(R, S, a, m, sA, sM, sBeta, l16, q4);
        }
        __syncthreads();

        // 4c. right-hand sides of W and U in the B-operand layout of this wave's
        //     column block: beta e^G o K and beta V at rows 16 y + 4 q4 + e, and
        //     e^G o Q at the same positions (the accumulator layout of the P tiles)
        float bw[NT][4], bu[NT][4], qh[NT][4];
        if constexpr (kFE) fe_finish_v<C>(fv, vb, pos.t0, q4);
        //     e^{G_s} at row s_ as a factor on the table: the per-channel 2^(G7) of the block on the
        //     fast path; on the steep path 2^(G_s) itself, formed from the exponent (sKr, sQr then
        //     holding K and Q as staged)
        float ev[NT][4];
        if (steep) {
#pragma unroll
            for (int y = 0; y < NT; ++y)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s_ = 16 * y + 4 * q4 + e, i = 16 * wave + l16;
                    ev[y][e] = exp2_fast(sE[y * kD + i] + sKc[s_ * LD + i]);
                }
        } else {
#pragma unroll
            for (int y = 0; y < NT; ++y) {
                const float f = sE[y * kD + 16 * wave + l16];
#pragma unroll
                for (int e = 0; e < 4; ++e) ev[y][e] = f;
            }
        }
#pragma unroll
        for (int y = 0; y < NT; ++y)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s_ = 16 * y + 4 * q4 + e, i = 16 * wave + l16;
                const float bb = sBeta[s_];
                bw[y][e] = bb * (sKr[s_ * LD + i] * ev[y][e]);
                if constexpr (kB16) bu[y][e] = bb * (s_ < nvalid ? bf16_to_f32(raw.vr[y][e]) : 0.f);
                else bu[y][e] = bb * (s_ < nvalid ? vb[y][e] : 0.f);
                qh[y][e] = sQr[s_ * LD + i] * ev[y][e];
            }

        // 5. W = T (beta e^G o K) and U = T (beta V) for this wave's 16-column block,
        //    by block forward substitution on the right-hand sides,
        //      Z_X = RHS_X - sum_{Y < X} A_XY W_Y,   W_X = T_XX Z_X,
        //    so the blocks of T below the diagonal are never formed.  The
        //    accumulator tiles stay in registers for step 6.  The Kc table is dead
        //    from step 3 until the next chunk is staged: its LDS holds the
        //    wave-private transpose scratch.
        static_assert(C * LD >= NW * 256, "transpose scratch");
        // (steep gates: step 4c read L from the Kc table, which the transposes now overwrite)
        if (steep) __syncthreads();
        float* const xpose = sKc + wave * 256;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kFE) fe_load_qk<C>(rq, fe, 0, npos, heads, tid, gn < n_total);
        else if constexpr (kB16)
            prep_load_part_b16<C>(raw.qb,
                                  prep_src_b16<C>(reinterpret_cast<const unsigned short*>(q), 0, heads, npos,
                                                  gn < n_total),
                                  heads, tid);
        else prep_load_part<C>(in.q, nsrc.q, heads, tid);
        __builtin_amdgcn_sched_barrier(0);
        floatx4 wt[NT], ut[NT];
#pragma unroll
        for (int X = 0; X < NT; ++X) {
            floatx4 zw, zu;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                zw[e] = bw[X][e];
                zu[e] = bu[X][e];
            }
#pragma unroll
            for (int Y = 0; Y < X; ++Y) {
                const float4 a4 = lds4(&sA[(16 * X + l16) * LDC + 16 * Y + 4 * q4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    zw = mfma4(-comp(a4, e), wt[Y][e], zw);
                    zu = mfma4(-comp(a4, e), ut[Y][e], zu);
                }
            }
            const float4 t4 = lds4(&sTd[(16 * X + l16) * LDT + 4 * q4]);
            floatx4 accW = {0.f, 0.f, 0.f, 0.f}, accU = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                accW = mfma4(comp(t4, e), zw[e], accW);
                accU = mfma4(comp(t4, e), zu[e], accU);
            }
            wt[X] = accW;
            ut[X] = accU;
            rec_st4(rec + G::kOffW + ((size_t)(X * 8 + wave) * 64 + lane) * 4, acc_to_atile(accW, xpose, lane));
            // U in the scan's accumulator layout: [row tile][16-column block][lane][4]
            rec_st4(rec + G::kOffU + ((size_t)(X * 8 + wave) * 64 + lane) * 4,
                make_float4(accU[0], accU[1], accU[2], accU[3]));
        }
        // 6. P = e^G o Q - M W and R = M U.  The W and U accumulator tiles are, lane
        //    for lane, the B operands of the products over the chunk rows.
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kGate) prep_load_gate<C>(in, gp, npos, heads, tid, gn < n_total);
        else prep_load_part<C>(in.g, nsrc.g, heads, tid);
        in.beta = prep_load_beta<C>(nsrc.b, heads, tid);
        __builtin_amdgcn_sched_barrier(0);
        // (fused front end) the next chunk's k and q from their raw inputs, which arrived during
        // steps 3-5; independent of this step's products, so the VALU work can fill the MFMA gaps
        if constexpr (kFE) fe_finish_kq<C>(rk, rq, in.k, in.q, npos.t0, tid, fe.eps);
        //    Row blocks X and NT - 1 - X go together (equal work, 4 (NT + 1) MFMAs
        //    each way), so four independent accumulation chains keep the matrix
        //    core busy instead of two; each block's sum runs in the same order.
        auto put_pr = [&](int X, const floatx4& mw, const floatx4& mu) {
            floatx4 pt;
#pragma unroll
            for (int e = 0; e < 4; ++e) pt[e] = qh[X][e] - mw[e];
            rec_st4(rec + G::kOffP + ((size_t)(X * 8 + wave) * 64 + lane) * 4, acc_to_atile(pt, xpose, lane));
            rec_st4(rec + G::kOffR + ((size_t)(X * 8 + wave) * 64 + lane) * 4, make_float4(mu[0], mu[1], mu[2], mu[3]));
        };
#pragma unroll
        for (int X0 = 0; X0 < (NT + 1) / 2; ++X0) {
            const int X1 = NT - 1 - X0;  // == X0 for the middle block of an odd count
            floatx4 mw0 = {0.f, 0.f, 0.f, 0.f}, mu0 = {0.f, 0.f, 0.f, 0.f};
            floatx4 mw1 = {0.f, 0.f, 0.f, 0.f}, mu1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int y = 0; y <= X1; ++y) {
                const float4 m1 = lds4(&sM[(16 * X1 + l16) * LDC + 16 * y + 4 * q4]);
                float4 m0 = m1;
                if (X1 != X0 && y <= X0) m0 = lds4(&sM[(16 * X0 + l16) * LDC + 16 * y + 4 * q4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    mw1 = mfma4(comp(m1, e), wt[y][e], mw1);
                    mu1 = mfma4(comp(m1, e), ut[y][e], mu1);
                    if (X1 != X0 && y <= X0) {
                        mw0 = mfma4(comp(m0, e), wt[y][e], mw0);
                        mu0 = mfma4(comp(m0, e), ut[y][e], mu0);
                    }
                }
            }
            if (X1 != X0) put_pr(X0, mw0, mu0);
            put_pr(X1, mw1, mu1);
        }
        __syncthreads();
        // stage the next chunk (loaded during this one; after the last chunk the
        // staged copy is unused)
        prep_stage<C, kFE, kGate, kB16>(in, sKr, sQr, sKc, sBeta, sSteep, npos.nvalid, tid, gp.lower, raw);
        pos = npos;
        __syncthreads();
    }
}

constexpr int kScanThreads = 512;  // 8 waves, two per SIMD
constexpr int kOutRow = 20;                // LDS row stride (floats) of a staged 16x16 output tile
constexpr int kOutTile = 16 * kOutRow;

// Operands one wave of the scan reads from a chunk record, prefetched two
// chunks ahead into registers.  A workgroup owns NCT adjacent 16-column tiles
// of the value index (16 NCT columns of one head).  Wave roles inside a chunk
// (NT = C / 16 row tiles):
//   wave < NT           Delta tile xd = wave:          Delta = U - W S
//   NT <= wave < 2 NT   output tile xp = wave - NT:    O = P S + R
//   every wave          state tile row block `wave`:   S <- diag(gamma) S + Ktil^T Delta
//   wave < NT           after that, stores output tile xd (staged in LDS by
//                       the output wave): the output waves are the younger
//                       ones on each SIMD, whose MFMAs issue last, so the
//                       stores go to the waves that wait for them.
// The A operands (W or P rows, Ktil^T rows) serve all NCT column tiles; each
// column tile is an independent MFMA chain.
template <int C, int NCT>
struct ScanOps {
    static constexpr int NT = C / 16;
    float4 a[8];       // W rows of the Delta tile, or P rows of the output tile
    float4 x[NCT];     // U tiles (Delta waves) or R tiles (output waves), accumulator layout
    float4 kt[NT];     // Ktil^T rows of this wave's state row block
    float4 g;          // gamma at those rows
};

// Byte offsets of one wave's operands inside a chunk record; they do not
// change from chunk to chunk, so they are computed once.
struct ScanOffsets {
    int a;   // W rows of the Delta tile or P rows of the output tile (8 A tiles, 1 KiB apart)
    int x;   // first U or R tile of this workgroup's columns (NCT tiles, 1 KiB apart)
    int kt;  // Ktil^T rows of the state row block (NT A tiles, 1 KiB apart)
    int g;   // gamma at those rows
};

template <int C>
__device__ __forceinline__ ScanOffsets scan_offsets(bool is_d, int xd, bool is_p, int xp, int wave, int lane, int q4,
                                                    int ct0)
{
    using G = ChunkGeom<C>;
    constexpr int NT = C / 16;
    const int xa = is_d ? xd : (is_p ? xp : 0);
    ScanOffsets o;
    o.a = (int)((is_d ? G::kOffW : G::kOffP) + ((size_t)xa * 8 * 64 + lane) * 4) * 4;
    o.x = (int)((is_d ? G::kOffU : G::kOffR) + ((size_t)(xa * 8 + ct0) * 64 + lane) * 4) * 4;
    o.kt = (int)(G::kOffKt + ((size_t)wave * NT * 64 + lane) * 4) * 4;
    o.g = (int)(G::kOffGam + 16 * wave + 4 * q4) * 4;
    return o;
}

// Every wave issues the same load sequence (only its lane offsets depend on
// its role), so the wait counts the compiler derives stay exact across the
// loop; the record address lives in scalar registers, so issuing the loads
// needs no vector registers beyond their destinations.
template <int C, int NCT>
__device__ __forceinline__ void scan_load(ScanOps<C, NCT>& o, rsrc_t rec, const ScanOffsets& off)
{
    constexpr int NT = C / 16;
#pragma unroll
    for (int tau = 0; tau < 8; ++tau) o.a[tau] = buf_ld4(rec, off.a, tau * 1024);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) o.x[ct] = buf_ld4(rec, off.x, ct * 1024);
#pragma unroll
    for (int y = 0; y < NT; ++y) o.kt[y] = buf_ld4(rec, off.kt, y * 1024);
    o.g = buf_ld4(rec, off.g, 0);
}

// One chunk of the scan for one wave.  The state lives in LDS only, in two
// buffers: sIn holds the chunk's incoming state, sOut receives the outgoing
// one.  Tile (s, ct), element e of lane l is S[16 s + 4 (l / 16) + e][v0 + 16 ct + l % 16],
// which is directly the B operand of the 16x16x4 MFMA over the key index.
// The operands of a later chunk are loaded into `nxt` one tile after every
// group of MFMAs, so the compute unit's vector-memory path takes them while
// the matrix core works instead of in one burst that the waves wait behind.
// kTrans: the transition form (no output tiles, no output waves); with homog
// the chunk's U is taken as zero (Delta = -W S), the homogeneous part of the
// update.
template <int C, int NCT, bool kTrans = false>
__device__ __forceinline__ void scan_chunk(const ScanOps<C, NCT>& cur, ScanOps<C, NCT>& nxt, rsrc_t nrec,
                                           const ScanOffsets& off, floatx4 (*sIn)[NCT][64],
                                           floatx4 (*sOut)[NCT][64], floatx4 (*sDelta)[NCT][64],
                                           float (*sO)[NCT][kOutTile], float* __restrict__ out_b, int out_voff,
                                           int c, bool is_d, int xd, bool is_p, int xp, int wave, int lane, int q4,
                                           int heads, int T, bool homog = false)
{
    constexpr int NT = C / 16;
    // at C = 64 every wave has a role in step A: no branch, so the wait counts
    // the compiler derives never merge a path that issued loads with one that did not
    constexpr bool kAllRoles = !kTrans && 2 * NT == kScanThreads / 64;
    // A. Delta = U - W S (Delta waves) and O = R + P S (output waves)
    if (kAllRoles || is_d || is_p) {
        floatx4 st[8][NCT];
#pragma unroll
        for (int tau = 0; tau < 8; ++tau)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) st[tau][ct] = sIn[tau][ct][lane];
        __builtin_amdgcn_sched_barrier(0);  // all eight reads in flight before the first MFMA
        // two independent accumulation chains per column tile (even and odd
        // key steps), so that a wave left alone on its SIMD still keeps the
        // matrix core busy instead of waiting out each MFMA's latency
        floatx4 acc[NCT], acc2[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            acc[ct][0] = is_p ? cur.x[ct].x : 0.f;
            acc[ct][1] = is_p ? cur.x[ct].y : 0.f;
            acc[ct][2] = is_p ? cur.x[ct].z : 0.f;
            acc[ct][3] = is_p ? cur.x[ct].w : 0.f;
            acc2[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int tau = 0; tau < 8; ++tau) {
#pragma unroll
            for (int e = 0; e < 4; e += 2)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    acc[ct] = mfma4(comp(cur.a[tau], e), st[tau][ct][e], acc[ct]);
                    acc2[ct] = mfma4(comp(cur.a[tau], e + 1), st[tau][ct][e + 1], acc2[ct]);
                }
            nxt.a[tau] = buf_ld4(nrec, off.a, tau * 1024);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acc[ct] += acc2[ct];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) nxt.x[ct] = buf_ld4(nrec, off.x, ct * 1024);
        if (is_d) {
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const float4 u = homog ? make_float4(0.f, 0.f, 0.f, 0.f) : cur.x[ct];
                floatx4 d;
                d[0] = u.x - acc[ct][0];
                d[1] = u.y - acc[ct][1];
                d[2] = u.z - acc[ct][2];
                d[3] = u.w - acc[ct][3];
                sDelta[xd][ct][lane] = d;
            }
        } else {
            // output tile xp to LDS, row-major (row stride kOutRow: the 64
            // lanes' writes of one element e hit 64 different banks)
            const int l16 = lane & 15;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) sO[xp][ct][(4 * q4 + e) * kOutRow + l16] = acc[ct][e];
        }
    } else {
#pragma unroll
        for (int tau = 0; tau < 8; ++tau) nxt.a[tau] = buf_ld4(nrec, off.a, tau * 1024);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) nxt.x[ct] = buf_ld4(nrec, off.x, ct * 1024);
    }
    __syncthreads();

    // B. state row block `wave`, all NCT column tiles
    {
        floatx4 dl[NT][NCT];
#pragma unroll
        for (int y = 0; y < NT; ++y)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) dl[y][ct] = sDelta[y][ct][lane];
        floatx4 acc[NCT], acc2[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const floatx4 so = sIn[wave][ct][lane];
            acc[ct][0] = cur.g.x * so[0];
            acc[ct][1] = cur.g.y * so[1];
            acc[ct][2] = cur.g.z * so[2];
            acc[ct][3] = cur.g.w * so[3];
            acc2[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int y = 0; y < NT; ++y) {
#pragma unroll
            for (int e = 0; e < 4; e += 2)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    acc[ct] = mfma4(comp(cur.kt[y], e), dl[y][ct][e], acc[ct]);
                    acc2[ct] = mfma4(comp(cur.kt[y], e + 1), dl[y][ct][e + 1], acc2[ct]);
                }
            nxt.kt[y] = buf_ld4(nrec, off.kt, y * 1024);
            __builtin_amdgcn_sched_barrier(0);
        }
        nxt.g = buf_ld4(nrec, off.g, 0);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acc[ct] += acc2[ct];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) sOut[wave][ct][lane] = acc[ct];
    }
    // C. output tile xd: row lane / 4 of the tile, columns 4 (lane % 4) + 0..3 of
    // each 16-column tile, one 16-byte store per lane and column tile
    if (!kTrans && is_d) {
        const int r = lane >> 2, j = lane & 3;
        const int t = c * C + 16 * xd + r;
        if (t < T) {
            const rsrc_t ob = make_rsrc(out_b + (size_t)c * C * heads * kD, (uint32_t)(C * heads * kD * 4));
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                buf_st4(ob, out_voff, 64 * ct, lds4(&sO[xd][ct][r * kOutRow + 4 * j]));
        }
    }
    __syncthreads();
}

// One workgroup per (sequence, head, group of 16 NCT value columns); the 8 / NCT
// groups of a head are mapped to one XCD (blockIdx % 8) so the head's records
// are fetched into that XCD's L2 once.
//
// kTrans: the segment transition instead of the scan, with `state` the Q
// output and `out` the P output, both [n_bh][128][128] and written whole.  A
// head gets twice the groups: the first 8 / NCT run the update from the zero
// state (Q, the final state of the segment from S = 0), the others run its
// homogeneous part (U taken as zero) from the identity, one column per key
// (P: the final state from S is P S + Q).  No outputs are produced.
template <int C, int NCT, class Layout, bool kTrans = false>
__global__ __launch_bounds__(kScanThreads) void chunk_scan_kernel(const float* __restrict__ ws,
                                                                  float* __restrict__ state, float* __restrict__ out,
                                                                  int n_bh, int heads, Layout layout)
{
    using G = ChunkGeom<C>;
    constexpr int NT = G::kTiles;
    constexpr int kGroups = 8 / NCT;  // column groups per head
    constexpr int kSlots = kTrans ? 2 * kGroups : kGroups;
    const int n = blockIdx.x;
    const int xcd = n & 7, k8 = n >> 3;
    const int slot = k8 % kSlots;
    const bool homog = kTrans && slot >= kGroups;
    const int slice = homog ? slot - kGroups : slot;
    const int bh = (k8 / kSlots) * 8 + xcd;
    if (bh >= n_bh) return;
    const SeqPos sq = layout.seq(bh);
    const int nchunks = sq.nchunks, T = sq.T;
    if (nchunks == 0) return;  // an empty sequence: its state is left as it is
    const int h = bh % heads;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int ct0 = NCT * slice, v0 = 16 * ct0;
    const bool is_d = wave < NT, is_p = !kTrans && wave >= NT && wave < 2 * NT;
    const int xd = wave, xp = wave - NT;

    __shared__ floatx4 sDelta[NT][NCT][64];
    __shared__ floatx4 sS[2][8][NCT][64];
    __shared__ __attribute__((aligned(16))) float sO[NT][NCT][kOutTile];

    float* const S_head = (homog ? out : state) + (size_t)bh * kD * kD;
    float* const out_b = kTrans ? nullptr : out + sq.tok0 * heads * kD;
    // byte offset of this lane's output row (16 xd + lane / 4) and columns
    // v0 + 4 (lane % 4) + 0..3 inside a chunk's output rows
    const int out_voff = ((16 * xd + (lane >> 2)) * heads * kD + h * kD + v0 + 4 * (lane & 3)) * 4;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        floatx4 st;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * wave + 4 * q4 + e, col = v0 + 16 * ct + l16;
            if constexpr (kTrans) st[e] = homog && row == col ? 1.f : 0.f;
            else st[e] = S_head[(size_t)row * kD + col];
        }
        sS[0][wave][ct][lane] = st;
    }
    const float* const rec0 = ws + sq.rec0 * G::kRecord;
    auto rec = [&](int cc) {
        return make_rsrc(rec0 + (size_t)(cc < nchunks ? cc : nchunks - 1) * G::kRecord, (uint32_t)(G::kRecord * 4));
    };
    const ScanOffsets off = scan_offsets<C>(is_d, xd, is_p, xp, wave, lane, q4, ct0);
    // Three operand buffers in rotation: while one chunk is computed, the loads
    // of the next are in flight and those of the one after are being issued
    // (no register copies between the buffers, so no wait on a prefetch
    // before it is needed).
    ScanOps<C, NCT> op0, op1, op2;
    scan_load<C, NCT>(op0, rec(0), off);
    scan_load<C, NCT>(op1, rec(1), off);
    __syncthreads();
    // Whole rounds of three chunks, then the remaining one or two: the loop has
    // a single back edge, so the wait counts at its head see only the state in
    // which a round ends.
    int c = 0;
    for (; c + 3 <= nchunks; c += 3) {
        scan_chunk<C, NCT, kTrans>(op0, op2, rec(c + 2), off, sS[c & 1], sS[(c + 1) & 1], sDelta, sO, out_b, out_voff, c, is_d,
                           xd, is_p, xp, wave, lane, q4, heads, T, homog);
        scan_chunk<C, NCT, kTrans>(op1, op0, rec(c + 3), off, sS[(c + 1) & 1], sS[c & 1], sDelta, sO, out_b, out_voff, c + 1,
                           is_d, xd, is_p, xp, wave, lane, q4, heads, T, homog);
        scan_chunk<C, NCT, kTrans>(op2, op1, rec(c + 4), off, sS[c & 1], sS[(c + 1) & 1], sDelta, sO, out_b, out_voff, c + 2,
                           is_d, xd, is_p, xp, wave, lane, q4, heads, T, homog);
    }
    if (c < nchunks)
        scan_chunk<C, NCT, kTrans>(op0, op2, rec(c + 2), off, sS[c & 1], sS[(c + 1) & 1], sDelta, sO, out_b, out_voff, c, is_d,
                           xd, is_p, xp, wave, lane, q4, heads, T, homog);
    if (c + 1 < nchunks)
        scan_chunk<C, NCT, kTrans>(op1, op0, rec(c + 3), off, sS[(c + 1) & 1], sS[c & 1], sDelta, sO, out_b, out_voff, c + 1,
                           is_d, xd, is_p, xp, wave, lane, q4, heads, T, homog);
    // the final state is in sS[nchunks & 1]
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        const floatx4 st = sS[nchunks & 1][wave][ct][lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) S_head[(size_t)(16 * wave + 4 * q4 + e) * kD + v0 + 16 * ct + l16] = st[e];
    }
}

template <int C, int NCT, class Layout, bool kTrans = false>
static int launch_scan(const float* ws, float* state, float* out, long long n_bh, int heads, const Layout& layout,
                       hipStream_t stream)
{
    const unsigned grid = (unsigned)(((n_bh + 7) / 8) * 64 / NCT * (kTrans ? 2 : 1));
    hipLaunchKernelGGL((chunk_scan_kernel<C, NCT, Layout, kTrans>), dim3(grid), dim3(kScanThreads), 0, stream, ws,
                       state, out, (int)n_bh, heads, layout);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

static int compute_units()
{
    int dev = 0, n_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 1)
        return -1;
    return n_cu;
}

// The scan with its column-group width: 32-column workgroups when 16-column
// ones would not fit the compute units in one round and 32-column ones still
// fill them (results are the same bits either way: value columns never mix).
template <int C, class Layout, bool kTrans = false>
static int launch_scan_auto(const float* ws, float* state, float* out, long long n_bh, int heads,
                            const Layout& layout, int n_cu, hipStream_t stream)
{
    const long long slots = kTrans ? 2 : 1;  // the transition form runs P and Q groups
    if constexpr (C == 64) {
        if (n_bh * 8 * slots > n_cu && n_bh * 4 * slots >= n_cu)
            return launch_scan<C, 2, Layout, kTrans>(ws, state, out, n_bh, heads, layout, stream);
    }
    return launch_scan<C, 1, Layout, kTrans>(ws, state, out, n_bh, heads, layout, stream);
}

// max_records bounds the layout's record count (exact for the dense layout).
// kTrans: state is the Q output and out the P output of the transition form.
// kFE: the prepare with the front end fused in (q, k, v unused; fe its inputs).
// kGate: kda_gate and the beta sigmoid inside the prepare (gate unused, beta the logits; gp its inputs).
template <int C, class Layout, bool kTrans = false, bool kFE = false, bool kGate = false, bool kB16 = false>
static int launch_chunk(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                        float* state, float* out, long long n_bh, int heads, long long max_records, float* ws,
                        const Layout& layout, hipStream_t stream, const FeSrc& fe = FeSrc{},
                        const GateParams& gp = GateParams{})
{
    // persistent prepare workgroups, as many per compute unit as its resources allow (one at C = 64,
    // where the LDS tables take all but 5 KiB; more at the narrower chunks, so that more chunks'
    // latency chains overlap).  Which workgroup takes which record does not change a bit.
    const int n_cu = compute_units();
    if (n_cu < 1) return -1;
    int per_cu = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chunk_prepare_kernel<C, Layout, kFE, kGate, kB16>,
                                                     kPrepThreads, 0) != hipSuccess || per_cu < 1) {
        (void)hipGetLastError();  // a failed query leaves no error behind for the launch check below
        per_cu = 1;
    }
    const long long slots = (long long)n_cu * per_cu;
    const int grid_p = (int)(max_records < slots ? max_records : slots);
    if (grid_p > 0) {
        hipLaunchKernelGGL((chunk_prepare_kernel<C, Layout, kFE, kGate, kB16>), dim3((unsigned)grid_p), dim3(kPrepThreads),
                           0, stream, q, k, v, gate, beta, ws, heads, layout, fe, gp);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    return launch_scan_auto<C, Layout, kTrans>(ws, state, out, n_bh, heads, layout, n_cu, stream);
}

template <int C, bool kTrans = false>
static int launch_dense(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                        float* state, float* out, int batch, int heads, int T, int t_pad, float* ws,
                        hipStream_t stream)
{
    const int nchunks = t_pad / C;
    const long long n_bh = (long long)batch * heads;
    const DenseLayout layout{heads, T, t_pad, nchunks, (int)(n_bh * nchunks)};
    return launch_chunk<C, DenseLayout, kTrans>(q, k, v, gate, beta, state, out, n_bh, heads, n_bh * nchunks, ws,
                                                layout, stream);
}

int launch_chunk_prefill(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                         float* state, float* out, int batch, int heads, int T, int t_pad, int chunk,
                         float* workspace, hipStream_t stream)
{
    switch (chunk) {
    case 16: return launch_dense<16>(q, k, v, gate, beta, state, out, batch, heads, T, t_pad, workspace, stream);
    case 32: return launch_dense<32>(q, k, v, gate, beta, state, out, batch, heads, T, t_pad, workspace, stream);
    case 64: return launch_dense<64>(q, k, v, gate, beta, state, out, batch, heads, T, t_pad, workspace, stream);
    default: return -1;
    }
}

// The prefill on BF16 q | k | v rows ([B][T_pad][3][heads][128]), passed to the prepare as its q pointer.
template <int C>
static int launch_dense_b16(const uint16_t* qkv, const float* gate, const float* beta, float* state, float* out,
                            int batch, int heads, int T, int t_pad, float* ws, hipStream_t stream)
{
    const int nchunks = t_pad / C;
    const long long n_bh = (long long)batch * heads;
    const DenseLayout layout{heads, T, t_pad, nchunks, (int)(n_bh * nchunks)};
    const float* const x = reinterpret_cast<const float*>(qkv);
    return launch_chunk<C, DenseLayout, false, false, false, true>(x, x, x, gate, beta, state, out, n_bh, heads,
                                                                  n_bh * nchunks, ws, layout, stream);
}

int launch_chunk_prefill_bf16(const uint16_t* qkv, const float* gate, const float* beta, float* state, float* out,
                              int batch, int heads, int T, int t_pad, int chunk, float* workspace, hipStream_t stream)
{
    switch (chunk) {
    case 16: return launch_dense_b16<16>(qkv, gate, beta, state, out, batch, heads, T, t_pad, workspace, stream);
    case 32: return launch_dense_b16<32>(qkv, gate, beta, state, out, batch, heads, T, t_pad, workspace, stream);
    case 64: return launch_dense_b16<64>(qkv, gate, beta, state, out, batch, heads, T, t_pad, workspace, stream);
    default: return -1;
    }
}

// The prefill with kda_gate and the beta sigmoid inside the prepare (dense layout): beta holds the
// logits, the gate comes from gp.
template <int C>
static int launch_dense_gated(const float* q, const float* k, const float* v, const float* beta_logit,
                              const GateParams& gp, float* state, float* out, int batch, int heads, int T, int t_pad,
                              float* ws, hipStream_t stream)
{
    const int nchunks = t_pad / C;
    const long long n_bh = (long long)batch * heads;
    const DenseLayout layout{heads, T, t_pad, nchunks, (int)(n_bh * nchunks)};
    // the gate pointer of the plain form is not read: q stands in for it (only its rows' descriptor is made)
    return launch_chunk<C, DenseLayout, false, false, true>(q, k, v, q, beta_logit, state, out, n_bh, heads,
                                                            n_bh * nchunks, ws, layout, stream, FeSrc{}, gp);
}

int launch_chunk_prefill_gated(const float* q, const float* k, const float* v, const float* beta_logit,
                               const GateParams& gp, float* state, float* out, int batch, int heads, int T, int t_pad,
                               int chunk, float* workspace, hipStream_t stream)
{
    switch (chunk) {
    case 16: return launch_dense_gated<16>(q, k, v, beta_logit, gp, state, out, batch, heads, T, t_pad, workspace, stream);
    case 32: return launch_dense_gated<32>(q, k, v, beta_logit, gp, state, out, batch, heads, T, t_pad, workspace, stream);
    case 64: return launch_dense_gated<64>(q, k, v, beta_logit, gp, state, out, batch, heads, T, t_pad, workspace, stream);
    default: return -1;
    }
}

// The scan alone, from the records a dense prepare left in ws.
template <int C>
static int launch_dense_scan(const float* ws, float* state, float* out, int batch, int heads, int T, int t_pad,
                             hipStream_t stream)
{
    const int nchunks = t_pad / C;
    const long long n_bh = (long long)batch * heads;
    const DenseLayout layout{heads, T, t_pad, nchunks, (int)(n_bh * nchunks)};
    const int n_cu = compute_units();
    if (n_cu < 1) return -1;
    return launch_scan_auto<C, DenseLayout>(ws, state, out, n_bh, heads, layout, n_cu, stream);
}

int launch_chunk_scan(const float* workspace, float* state, float* out, int batch, int heads, int T, int t_pad,
                      int chunk, hipStream_t stream)
{
    switch (chunk) {
    case 16: return launch_dense_scan<16>(workspace, state, out, batch, heads, T, t_pad, stream);
    case 32: return launch_dense_scan<32>(workspace, state, out, batch, heads, T, t_pad, stream);
    case 64: return launch_dense_scan<64>(workspace, state, out, batch, heads, T, t_pad, stream);
    default: return -1;
    }
}

// The prefill with the front end fused into the prepare (dense layout).  q, k,
// v are not read in this form: the gate pointer stands in for them.
// With gp, kda_gate and the beta sigmoid are inside the prepare too (gate not read, beta the logits),
// and beta stands in for every unread pointer.
template <int C>
static int launch_dense_fused(const FeSrc& fe, const float* gate, const float* beta, const GateParams* gp,
                              float* state, float* out, int batch, int heads, int T, int t_pad, float* ws,
                              hipStream_t stream)
{
    const int nchunks = t_pad / C;
    const long long n_bh = (long long)batch * heads;
    const DenseLayout layout{heads, T, t_pad, nchunks, (int)(n_bh * nchunks)};
    if (gp)
        return launch_chunk<C, DenseLayout, false, true, true>(beta, beta, beta, beta, beta, state, out, n_bh, heads,
                                                               n_bh * nchunks, ws, layout, stream, fe, *gp);
    return launch_chunk<C, DenseLayout, false, true>(gate, gate, gate, gate, beta, state, out, n_bh, heads,
                                                     n_bh * nchunks, ws, layout, stream, fe);
}

int launch_chunk_prefill_fused(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state, const float* gate,
                               const float* beta, const GateParams* gp, float* state, float* out, int batch, int heads,
                               int T, int t_pad, int chunk, float l2_eps, float* workspace, hipStream_t stream)
{
    const FeSrc fe{reinterpret_cast<const unsigned short*>(qkv), reinterpret_cast<const unsigned short*>(conv_w),
                   conv_state, (double)l2_eps};
    int rc = -1;
    switch (chunk) {
    case 16: rc = launch_dense_fused<16>(fe, gate, beta, gp, state, out, batch, heads, T, t_pad, workspace, stream); break;
    case 32: rc = launch_dense_fused<32>(fe, gate, beta, gp, state, out, batch, heads, T, t_pad, workspace, stream); break;
    case 64: rc = launch_dense_fused<64>(fe, gate, beta, gp, state, out, batch, heads, T, t_pad, workspace, stream); break;
    default: return -1;
    }
    if (rc != 0) return rc;
    // every prepare workgroup has read the conv state by now (stream order)
    return launch_conv_state_advance(qkv, conv_state, batch, heads, T, kFeK, stream);
}

int launch_chunk_prefill_transition(const float* q, const float* k, const float* v, const float* gate,
                                    const float* beta, float* trans_p, float* trans_q, int batch, int heads, int T,
                                    int t_pad, int chunk, float* workspace, hipStream_t stream)
{
    switch (chunk) {
    case 16: return launch_dense<16, true>(q, k, v, gate, beta, trans_q, trans_p, batch, heads, T, t_pad, workspace, stream);
    case 32: return launch_dense<32, true>(q, k, v, gate, beta, trans_q, trans_p, batch, heads, T, t_pad, workspace, stream);
    case 64: return launch_dense<64, true>(q, k, v, gate, beta, trans_q, trans_p, batch, heads, T, t_pad, workspace, stream);
    default: return -1;
    }
}

// S <- P S + Q for n independent 128 x 128 states (Q null: S <- P S): the
// fold of segment transitions, and their composition (P2 P1, P2 Q1 + Q2).
// The value columns of a state are independent (column j of the result needs
// column j of S and Q and all of P), so each state is split over
// kApplyGroups workgroups of 16 kApplyNct columns; they take block indices 8
// apart, which the dispatcher places on one XCD, so P is fetched into one L2.
// A workgroup stages its columns of the incoming state in LDS before any of
// them is overwritten, so S is updated in place; wave w computes rows
// 16 w .. 16 w + 15 of its columns with the 16x16x4 FP32 MFMA, the key index
// as the reduction, two chains per 16-column tile (even and odd key steps).
constexpr int kApplyThreads = 512;
constexpr int kApplyNct = 4;                 // 16-column tiles per workgroup
constexpr int kApplyGroups = 8 / kApplyNct;  // workgroups per state

__global__ __launch_bounds__(kApplyThreads) void transition_apply_kernel(const float* __restrict__ P,
                                                                         const float* __restrict__ Q, float* S, int n)
{
    // block b: state 8 (b / (8 G)) + b % 8, column group (b / 8) % G
    const int b = blockIdx.x;
    const int u = 8 * (b / (8 * kApplyGroups)) + b % 8, grp = (b / 8) % kApplyGroups;
    if (u >= n) return;  // the whole workgroup leaves together, before its barrier
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;
    const int c0 = 16 * kApplyNct * grp;  // first column of the group
    // tile (row block rb, column tile ct), element e of lane l: S[16 rb + 4 (l / 16) + e][c0 + 16 ct + l % 16]
    __shared__ floatx4 sS[8][kApplyNct][64];
    float* const Su = S + (size_t)u * kD * kD;
    const float* const Pu = P + (size_t)u * kD * kD;
#pragma unroll
    for (int ct = 0; ct < kApplyNct; ++ct) {
        floatx4 st;
#pragma unroll
        for (int e = 0; e < 4; ++e) st[e] = Su[(size_t)(16 * wave + 4 * q4 + e) * kD + c0 + 16 * ct + l16];
        sS[wave][ct][lane] = st;
    }
    __syncthreads();
    floatx4 acc[kApplyNct], acc2[kApplyNct];
#pragma unroll
    for (int ct = 0; ct < kApplyNct; ++ct) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc[ct][e] = Q ? Q[(size_t)u * kD * kD + (size_t)(16 * wave + 4 * q4 + e) * kD + c0 + 16 * ct + l16]
                           : 0.f;
        acc2[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int tau = 0; tau < 8; ++tau) {
        // A operand: P[16 w + l % 16][16 tau + 4 (l / 16) + e] for the e-th key step
        const float4 a = ld4(Pu + (size_t)(16 * wave + l16) * kD + 16 * tau + 4 * q4);
#pragma unroll
        for (int e = 0; e < 4; e += 2)
#pragma unroll
            for (int ct = 0; ct < kApplyNct; ++ct) {
                acc[ct] = mfma4(comp(a, e), sS[tau][ct][lane][e], acc[ct]);
                acc2[ct] = mfma4(comp(a, e + 1), sS[tau][ct][lane][e + 1], acc2[ct]);
            }
    }
#pragma unroll
    for (int ct = 0; ct < kApplyNct; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            Su[(size_t)(16 * wave + 4 * q4 + e) * kD + c0 + 16 * ct + l16] = acc[ct][e] + acc2[ct][e];
}

int launch_transition_apply(const float* P, const float* Q, float* S, int n, hipStream_t stream)
{
    const long long blocks = (long long)((n + 7) / 8) * 8 * kApplyGroups;  // n padded to whole groups of 8
    hipLaunchKernelGGL(transition_apply_kernel, dim3((unsigned)blocks), dim3(kApplyThreads), 0, stream, P, Q, S, n);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Varlen set-up, one workgroup: token offsets clamped to [0, total] and made
// non-decreasing (so no later access leaves the buffers whatever the caller
// passed), and the chunk offsets cb[s] = sum over s' < s of ceil(len(s') / C).
constexpr int kSetupThreads = 1024;
__global__ __launch_bounds__(kSetupThreads) void varlen_setup_kernel(const int* __restrict__ cu_in, int n_seqs,
                                                                     int total, int C, int* __restrict__ cu,
                                                                     int* __restrict__ cb)
{
    __shared__ int s_max[kSetupThreads], s_sum[kSetupThreads];
    const int tid = threadIdx.x, n = n_seqs + 1;
    const int per = (n + kSetupThreads - 1) / kSetupThreads, i0 = tid * per, i1 = i0 + per < n ? i0 + per : n;
    auto clamp = [&](int x) { return x < 0 ? 0 : (x > total ? total : x); };
    // pass 1: the running maximum of this thread's entries
    int m = 0;
    for (int i = i0; i < i1; ++i) m = max(m, clamp(cu_in[i]));
    s_max[tid] = m;
    __syncthreads();
    for (int off = 1; off < kSetupThreads; off <<= 1) {  // inclusive max-scan over the threads
        const int o = tid >= off ? s_max[tid - off] : 0;
        __syncthreads();
        s_max[tid] = max(s_max[tid], o);
        __syncthreads();
    }
    // pass 2: offsets and this thread's chunk count
    int run = tid > 0 ? s_max[tid - 1] : 0, chunks = 0;
    for (int i = i0; i < i1; ++i) {
        const int prev = run;
        run = max(run, clamp(cu_in[i]));
        cu[i] = run;
        if (i > 0) chunks += (run - prev + C - 1) / C;  // sequence i - 1 ends at run
    }
    s_sum[tid] = chunks;
    __syncthreads();
    for (int off = 1; off < kSetupThreads; off <<= 1) {  // inclusive sum-scan over the threads
        const int o = tid >= off ? s_sum[tid - off] : 0;
        __syncthreads();
        s_sum[tid] += o;
        __syncthreads();
    }
    // pass 3: chunk offsets (this thread's own offsets, read back; the one
    // before its range is the previous thread's running maximum)
    int prev = tid > 0 ? s_max[tid - 1] : 0, acc = tid > 0 ? s_sum[tid - 1] : 0;
    for (int i = i0; i < i1; ++i) {
        const int cur = cu[i];
        if (i > 0) acc += (cur - prev + C - 1) / C;
        cb[i] = acc;
        prev = cur;
    }
}

int launch_chunk_prefill_varlen_fused(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state,
                                      const float* gate, const float* beta, float* state, float* out,
                                      const int* cu_seqlens, int n_seqs, int heads, int total, int chunk,
                                      float l2_eps, float* workspace, size_t meta_offset_floats,
                                      long long max_records, hipStream_t stream)
{
    int* const cu = reinterpret_cast<int*>(workspace + meta_offset_floats);
    int* const cb = cu + (n_seqs + 1);
    hipLaunchKernelGGL(varlen_setup_kernel, dim3(1), dim3(kSetupThreads), 0, stream, cu_seqlens, n_seqs, total,
                       chunk, cu, cb);
    if (hipGetLastError() != hipSuccess) return -1;
    const VarlenLayout layout{heads, total, n_seqs, cu, cb};
    const long long n_bh = (long long)n_seqs * heads;
    const FeSrc fe{reinterpret_cast<const unsigned short*>(qkv), reinterpret_cast<const unsigned short*>(conv_w),
                   conv_state, (double)l2_eps};
    int rc = -1;
    // q, k, v are not read in this form: the gate pointer stands in for them
    switch (chunk) {
    case 16: rc = launch_chunk<16, VarlenLayout, false, true>(gate, gate, gate, gate, beta, state, out, n_bh, heads, max_records, workspace, layout, stream, fe); break;
    case 32: rc = launch_chunk<32, VarlenLayout, false, true>(gate, gate, gate, gate, beta, state, out, n_bh, heads, max_records, workspace, layout, stream, fe); break;
    case 64: rc = launch_chunk<64, VarlenLayout, false, true>(gate, gate, gate, gate, beta, state, out, n_bh, heads, max_records, workspace, layout, stream, fe); break;
    default: return -1;
    }
    if (rc != 0) return rc;
    return launch_conv_state_advance_varlen(qkv, conv_state, cu_seqlens, n_seqs, heads, total, 4, stream);
}

template <bool kB16>
static int launch_varlen(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                         float* state, float* out, const int* cu_seqlens, int n_seqs, int heads, int total, int chunk,
                         float* workspace, size_t meta_offset_floats, long long max_records, hipStream_t stream)
{
    int* const cu = reinterpret_cast<int*>(workspace + meta_offset_floats);
    int* const cb = cu + (n_seqs + 1);
    hipLaunchKernelGGL(varlen_setup_kernel, dim3(1), dim3(kSetupThreads), 0, stream, cu_seqlens, n_seqs, total,
                       chunk, cu, cb);
    if (hipGetLastError() != hipSuccess) return -1;
    const VarlenLayout layout{heads, total, n_seqs, cu, cb};
    const long long n_bh = (long long)n_seqs * heads;
    switch (chunk) {
    case 16:
        return launch_chunk<16, VarlenLayout, false, false, false, kB16>(q, k, v, gate, beta, state, out, n_bh, heads,
                                                                         max_records, workspace, layout, stream);
    case 32:
        return launch_chunk<32, VarlenLayout, false, false, false, kB16>(q, k, v, gate, beta, state, out, n_bh, heads,
                                                                         max_records, workspace, layout, stream);
    case 64:
        return launch_chunk<64, VarlenLayout, false, false, false, kB16>(q, k, v, gate, beta, state, out, n_bh, heads,
                                                                         max_records, workspace, layout, stream);
    default: return -1;
    }
}

int launch_chunk_prefill_varlen_bf16(const uint16_t* qkv, const float* gate, const float* beta, float* state,
                                     float* out, const int* cu_seqlens, int n_seqs, int heads, int total, int chunk,
                                     float* workspace, size_t meta_offset_floats, long long max_records,
                                     hipStream_t stream)
{
    const float* const x = reinterpret_cast<const float*>(qkv);
    return launch_varlen<true>(x, x, x, gate, beta, state, out, cu_seqlens, n_seqs, heads, total, chunk, workspace,
                               meta_offset_floats, max_records, stream);
}

int launch_chunk_prefill_varlen(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                                float* state, float* out, const int* cu_seqlens, int n_seqs, int heads, int total,
                                int chunk, float* workspace, size_t meta_offset_floats, long long max_records,
                                hipStream_t stream)
{
    return launch_varlen<false>(q, k, v, gate, beta, state, out, cu_seqlens, n_seqs, heads, total, chunk, workspace,
                                meta_offset_floats, max_records, stream);
}

}  // namespace kda
