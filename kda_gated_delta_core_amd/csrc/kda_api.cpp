// C ABI of the KDA core (declared in include/kda.h): argument checks on the
// host, then launches on the caller's stream.  Nothing here allocates.
#include "kda.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "kda_common.h"
#include "kda_internal.h"

#define KDA_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int64_t kMaxElems = INT64_C(1) << 46;  // keeps every byte offset far inside int64

// a * b * ..., or -1 when any factor is < 0 or the product passes kMaxElems
int64_t mul(std::initializer_list<int64_t> xs)
{
    int64_t p = 1;
    for (int64_t x : xs) {
        if (x < 0) return -1;
        if (x != 0 && p > kMaxElems / x) return -1;
        p *= x;
    }
    return p;
}

struct Range {
    const void* p;
    int64_t bytes;
};

bool overlap(const Range& a, const Range& b)
{
    if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + (uintptr_t)b.bytes && b0 < a0 + (uintptr_t)a.bytes;
}

// every written range against every other range
bool any_overlap(const Range* ranges, int n, int n_written)
{
    for (int i = 0; i < n_written; ++i)
        for (int j = 0; j < n; ++j)
            if (j != i && overlap(ranges[i], ranges[j])) return true;
    return false;
}

// the kernels move tensors with 16-byte vector accesses (beta with 4-byte ones)
bool aligned(std::initializer_list<const void*> ps, uintptr_t a = 16)
{
    for (const void* p : ps)
        if ((uintptr_t)p % a) return false;
    return true;
}

bool chunk_ok(int chunk) { return chunk == 16 || chunk == 32 || chunk == 64; }

// the gate inputs of the *_gated entry points: g_raw [rows][heads][128] BF16 (8-byte aligned),
// dt_bias [heads][128] (16-byte aligned), a_log [heads], a finite lower bound <= 0
bool gate_inputs_ok(const uint16_t* g_raw, const float* dt_bias, const float* a_log, float lower)
{
    return g_raw && dt_bias && a_log && aligned({g_raw}, 8) && aligned({dt_bias}) && aligned({a_log}, 4) &&
           isfinite(lower) && lower <= 0.f;
}

int64_t prefill_ws_bytes(int batch, int heads, int T, int chunk)
{
    if (batch < 1 || heads < 1 || T < 1 || !chunk_ok(chunk)) return -1;
    const int64_t nchunks = ((int64_t)T + chunk - 1) / chunk;
    const int64_t recs = mul({batch, heads, nchunks});
    if (recs < 0 || recs > 0x7fffffffLL) return -1;  // one prepare workgroup per record
    const int64_t floats = mul({recs, (int64_t)kda::chunk_record_floats(chunk)});
    return floats < 0 ? -1 : floats * 4;
}

}  // namespace

KDA_API const char* kda_status_string(int status)
{
    switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG: null pointer, size out of range or overlapping buffers";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: chunk must be 16, 32 or 64";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace smaller than kda_chunk_prefill_workspace_bytes()";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: the HIP runtime refused a launch";
    default: return "unknown kda status";
    }
}

KDA_API size_t kda_chunk_prefill_workspace_bytes(int batch, int heads, int T, int chunk)
{
    const int64_t b = prefill_ws_bytes(batch, heads, T, chunk);
    return b < 0 ? 0 : (size_t)b;
}

KDA_API int kda_chunk_prefill(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                              float* state, float* out, int batch, int heads, int T, int chunk, void* workspace,
                              size_t workspace_bytes, void* stream)
{
    if (!q || !k || !v || !gate || !beta || !state || !out) return KDA_ERR_INVALID_ARG;
    if (!aligned({q, k, v, gate, state, out, workspace}) || !aligned({beta}, 4)) return KDA_ERR_INVALID_ARG;
    if (batch < 1 || heads < 1 || T < 1) return KDA_ERR_INVALID_ARG;
    if (!chunk_ok(chunk)) return KDA_ERR_UNSUPPORTED;
    const int64_t need = prefill_ws_bytes(batch, heads, T, chunk);
    const int64_t t_pad = ((int64_t)T + chunk - 1) / chunk * chunk;
    const int64_t vec = mul({batch, t_pad, heads, KDA_HEAD_DIM});
    const int64_t sca = mul({batch, t_pad, heads});
    const int64_t st = mul({batch, heads, KDA_HEAD_DIM, KDA_HEAD_DIM});
    if (need < 0 || vec < 0 || sca < 0 || st < 0 || t_pad > 0x7fffffffLL) return KDA_ERR_INVALID_ARG;
    if ((int64_t)batch * heads > 0x7fffffffLL / 64) return KDA_ERR_INVALID_ARG;  // scan grid
    if (heads > KDA_PREFILL_MAX_HEADS) return KDA_ERR_INVALID_ARG;  // 32-bit in-chunk byte offsets
    if ((int64_t)batch * heads * (t_pad / chunk) > (1LL << 30)) return KDA_ERR_INVALID_ARG;  // chunk index
    if (!workspace || workspace_bytes < (size_t)need) return KDA_ERR_WORKSPACE;
    const Range r[] = {{out, vec * 4}, {state, st * 4}, {workspace, need}, {q, vec * 4}, {k, vec * 4},
                       {v, vec * 4},   {gate, vec * 4}, {beta, sca * 4}};
    if (any_overlap(r, 8, 3)) return KDA_ERR_INVALID_ARG;
    const int rc = kda::launch_chunk_prefill(q, k, v, gate, beta, state, out, batch, heads, T, (int)t_pad, chunk,
                                             static_cast<float*>(workspace), static_cast<hipStream_t>(stream));
    return rc == 0 ? KDA_OK : KDA_ERR_HIP;
}

KDA_API int kda_chunk_prefill_bf16(const uint16_t* qkv, const float* gate, const float* beta, float* state, float* out,
                                   int batch, int heads, int T, int chunk, void* workspace, size_t workspace_bytes,
                                   void* stream)
{
    if (!qkv || !gate || !beta || !state || !out) return KDA_ERR_INVALID_ARG;
    if (!aligned({qkv, gate, state, out, workspace}) || !aligned({beta}, 4)) return KDA_ERR_INVALID_ARG;
    if (batch < 1 || heads < 1 || T < 1) return KDA_ERR_INVALID_ARG;
    if (!chunk_ok(chunk)) return KDA_ERR_UNSUPPORTED;
    const int64_t need = prefill_ws_bytes(batch, heads, T, chunk);
    const int64_t t_pad = ((int64_t)T + chunk - 1) / chunk * chunk;
    const int64_t x = mul({batch, t_pad, 3, heads, KDA_HEAD_DIM});
    const int64_t vec = mul({batch, t_pad, heads, KDA_HEAD_DIM});
    const int64_t sca = mul({batch, t_pad, heads});
    const int64_t st = mul({batch, heads, KDA_HEAD_DIM, KDA_HEAD_DIM});
    if (need < 0 || x < 0 || vec < 0 || sca < 0 || st < 0 || t_pad > 0x7fffffffLL) return KDA_ERR_INVALID_ARG;
    if ((int64_t)batch * heads > 0x7fffffffLL / 64) return KDA_ERR_INVALID_ARG;  // scan grid
    if (heads > KDA_PREFILL_MAX_HEADS) return KDA_ERR_INVALID_ARG;  // 32-bit in-chunk byte offsets
    if ((int64_t)batch * heads * (t_pad / chunk) > (1LL << 30)) return KDA_ERR_INVALID_ARG;  // chunk index
    if (!workspace || workspace_bytes < (size_t)need) return KDA_ERR_WORKSPACE;
    const Range r[] = {{out, vec * 4}, {state, st * 4}, {workspace, need}, {qkv, x * 2}, {gate, vec * 4},
                       {beta, sca * 4}};
    if (any_overlap(r, 6, 3)) return KDA_ERR_INVALID_ARG;
    const int rc = kda::launch_chunk_prefill_bf16(qkv, gate, beta, state, out, batch, heads, T, (int)t_pad, chunk,
                                                  static_cast<float*>(workspace), static_cast<hipStream_t>(stream));
    return rc == 0 ? KDA_OK : KDA_ERR_HIP;
}

KDA_API int kda_chunk_prefill_gated(const float* q, const float* k, const float* v, const uint16_t* g_raw,
                                    const float* beta_logit, const float* dt_bias, const float* a_log,
                                    float gate_lower_bound, float* state, float* out, int batch, int heads, int T,
                                    int chunk, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!q || !k || !v || !beta_logit || !state || !out) return KDA_ERR_INVALID_ARG;
    if (!gate_inputs_ok(g_raw, dt_bias, a_log, gate_lower_bound)) return KDA_ERR_INVALID_ARG;
    if (!aligned({q, k, v, state, out, workspace}) || !aligned({beta_logit}, 4)) return KDA_ERR_INVALID_ARG;
    if (batch < 1 || heads < 1 || T < 1) return KDA_ERR_INVALID_ARG;
    if (!chunk_ok(chunk)) return KDA_ERR_UNSUPPORTED;
    const int64_t need = prefill_ws_bytes(batch, heads, T, chunk);
    const int64_t t_pad = ((int64_t)T + chunk - 1) / chunk * chunk;
    const int64_t vec = mul({batch, t_pad, heads, KDA_HEAD_DIM});
    const int64_t sca = mul({batch, t_pad, heads});
    const int64_t st = mul({batch, heads, KDA_HEAD_DIM, KDA_HEAD_DIM});
    if (need < 0 || vec < 0 || sca < 0 || st < 0 || t_pad > 0x7fffffffLL) return KDA_ERR_INVALID_ARG;
    if ((int64_t)batch * heads > 0x7fffffffLL / 64) return KDA_ERR_INVALID_ARG;
    if (heads > KDA_PREFILL_MAX_HEADS) return KDA_ERR_INVALID_ARG;
    if ((int64_t)batch * heads * (t_pad / chunk) > (1LL << 30)) return KDA_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < (size_t)need) return KDA_ERR_WORKSPACE;
    const Range r[] = {{out, vec * 4},        {state, st * 4},          {workspace, need},
                       {q, vec * 4},          {k, vec * 4},             {v, vec * 4},
                       {g_raw, vec * 2},      {beta_logit, sca * 4},    {dt_bias, (int64_t)heads * KDA_HEAD_DIM * 4},
                       {a_log, (int64_t)heads * 4}};
    if (any_overlap(r, 10, 3)) return KDA_ERR_INVALID_ARG;
    const kda::GateParams gp{reinterpret_cast<const unsigned short*>(g_raw), dt_bias, a_log, gate_lower_bound};
    const int rc = kda::launch_chunk_prefill_gated(q, k, v, beta_logit, gp, state, out, batch, heads, T, (int)t_pad,
                                                   chunk, static_cast<float*>(workspace),
                                                   static_cast<hipStream_t>(stream));
    return rc == 0 ? KDA_OK : KDA_ERR_HIP;
}

// The chunk records of kda_chunk_prefill_noalloc: a static device array, one
// copy per GPU at its own address.  In host code `scratch` names a host-side
// stand-in, never the device memory: every host use goes through the address
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept.
static __device__ __align__(256) float scratch[KDA_STATIC_WORKSPACE_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices];

// this device's copy of `scratch` (looked up on its first use), or nullptr
float* scratch_address()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch[dev] = static_cast<float*>(p);
    }
    return g_scratch[dev];
}

}  // namespace

KDA_API int kda_chunk_prefill_noalloc(const float* q, const float* k, const float* v, const float* gate,
                                      const float* beta, float* state, float* out, int batch, int heads, int T,
                                      int chunk, void* stream)
{
    // the argument checks of kda_chunk_prefill, with the array's size in place of a workspace size
    if (!q || !k || !v || !gate || !beta || !state || !out) return KDA_ERR_INVALID_ARG;
    if (!aligned({q, k, v, gate, state, out}) || !aligned({beta}, 4)) return KDA_ERR_INVALID_ARG;
    if (batch < 1 || heads < 1 || T < 1) return KDA_ERR_INVALID_ARG;
    if (!chunk_ok(chunk)) return KDA_ERR_UNSUPPORTED;
    const int64_t need = prefill_ws_bytes(batch, heads, T, chunk);
    const int64_t t_pad = ((int64_t)T + chunk - 1) / chunk * chunk;
    const int64_t vec = mul({batch, t_pad, heads, KDA_HEAD_DIM});
    const int64_t sca = mul({batch, t_pad, heads});
    const int64_t st = mul({batch, heads, KDA_HEAD_DIM, KDA_HEAD_DIM});
    if (need < 0 || vec < 0 || sca < 0 || st < 0 || t_pad > 0x7fffffffLL) return KDA_ERR_INVALID_ARG;
    if ((int64_t)batch * heads > 0x7fffffffLL / 64) return KDA_ERR_INVALID_ARG;
    if (heads > KDA_PREFILL_MAX_HEADS) return KDA_ERR_INVALID_ARG;
    if ((int64_t)batch * heads * (t_pad / chunk) > (1LL << 30)) return KDA_ERR_INVALID_ARG;
    if (need > (int64_t)KDA_STATIC_WORKSPACE_BYTES) return KDA_ERR_WORKSPACE;
    const Range r[] = {{out, vec * 4}, {state, st * 4}, {q, vec * 4}, {k, vec * 4},
                       {v, vec * 4},   {gate, vec * 4}, {beta, sca * 4}};
    if (any_overlap(r, 7, 2)) return KDA_ERR_INVALID_ARG;
    float* const ws = scratch_address();
    if (!ws) return KDA_ERR_HIP;
    const int rc = kda::launch_chunk_prefill(q, k, v, gate, beta, state, out, batch, heads, T, (int)t_pad, chunk, ws,
                                             static_cast<hipStream_t>(stream));
    return rc == 0 ? KDA_OK : KDA_ERR_HIP;
}

KDA_API int kda_chunk_prefill_transition(const float* q, const float* k, const float* v, const float* gate,
                                         const float* beta, float* trans_p, float* trans_q, int batch, int heads,
                                         int T, int chunk, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!q || !k || !v || !gate || !beta || !trans_p || !trans_q) return KDA_ERR_INVALID_ARG;
    if (!aligned({q, k, v, gate, trans_p, trans_q, workspace}) || !aligned({beta}, 4)) return KDA_ERR_INVALID_ARG;
    if (batch < 1 || heads < 1 || T < 1) return KDA_ERR_INVALID_ARG;
    if (!chunk_ok(chunk)) return KDA_ERR_UNSUPPORTED;
    const int64_t need = prefill_ws_bytes(batch, heads, T, chunk);
    const int64_t t_pad = ((int64_t)T + chunk - 1) / chunk * chunk;
    const int64_t vec = mul({batch, t_pad, heads, KDA_HEAD_DIM});
    const int64_t sca = mul({batch, t_pad, heads});
    const int64_t st = mul({batch, heads, KDA_HEAD_DIM, KDA_HEAD_DIM});
    if (need < 0 || vec < 0 || sca < 0 || st < 0 || t_pad > 0x7fffffffLL) return KDA_ERR_INVALID_ARG;
    if ((int64_t)batch * heads > 0x7fffffffLL / 128) return KDA_ERR_INVALID_ARG;  // scan grid (P and Q groups)
    if (heads > KDA_PREFILL_MAX_HEADS) return KDA_ERR_INVALID_ARG;
    if ((int64_t)batch * heads * (t_pad / chunk) > (1LL << 30)) return KDA_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < (size_t)need) return KDA_ERR_WORKSPACE;
    const Range r[] = {{trans_p, st * 4}, {trans_q, st * 4}, {workspace, need}, {q, vec * 4}, {k, vec * 4},
                       {v, vec * 4},      {gate, vec * 4},   {beta, sca * 4}};
    if (any_overlap(r, 8, 3)) return KDA_ERR_INVALID_ARG;
    const int rc = kda::launch_chunk_prefill_transition(q, k, v, gate, beta, trans_p, trans_q, batch, heads, T,
                                                        (int)t_pad, chunk, static_cast<float*>(workspace),
                                                        static_cast<hipStream_t>(stream));
    return rc == 0 ? KDA_OK : KDA_ERR_HIP;
}

KDA_API int kda_chunk_scan(float* state, float* out, int batch, int heads, int T, int chunk, const void* workspace,
                           size_t workspace_bytes, void* stream)
{
    if (!state || !out) return KDA_ERR_INVALID_ARG;
    if (!aligned({state, out, workspace})) return KDA_ERR_INVALID_ARG;
    if (batch < 1 || heads < 1 || T < 1) return KDA_ERR_INVALID_ARG;
    if (!chunk_ok(chunk)) return KDA_ERR_UNSUPPORTED;
    const int64_t need = prefill_ws_bytes(batch, heads, T, chunk);
    const int64_t t_pad = ((int64_t)T + chunk - 1) / chunk * chunk;
    const int64_t vec = mul({batch, t_pad, heads, KDA_HEAD_DIM});
    const int64_t st = mul({batch, heads, KDA_HEAD_DIM, KDA_HEAD_DIM});
    if (need < 0 || vec < 0 || st < 0 || t_pad > 0x7fffffffLL) return KDA_ERR_INVALID_ARG;
    if ((int64_t)batch * heads > 0x7fffffffLL / 64) return KDA_ERR_INVALID_ARG;
    if (heads > KDA_PREFILL_MAX_HEADS) return KDA_ERR_INVALID_ARG;
    if ((int64_t)batch * heads * (t_pad / chunk) > (1LL << 30)) return KDA_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < (size_t)need) return KDA_ERR_WORKSPACE;
    const Range r[] = {{out, vec * 4}, {state, st * 4}, {workspace, need}};
    if (any_overlap(r, 3, 2)) return KDA_ERR_INVALID_ARG;
    const int rc = kda::launch_chunk_scan(static_cast<const float*>(workspace), state, out, batch, heads, T,
                                          (int)t_pad, chunk, static_cast<hipStream_t>(stream));
    return rc == 0 ? KDA_OK : KDA_ERR_HIP;
}

KDA_API int kda_state_transition_apply(const float* trans_p, const float* trans_q, float* state, int batch,
                                       int heads, void* stream)
{
    if (!trans_p || !state) return KDA_ERR_INVALID_ARG;
    if (!aligned({trans_p, trans_q, state})) return KDA_ERR_INVALID_ARG;
    // two workgroups of 512 threads per state: the grid's work-items stay below 2^32
    if (batch < 1 || heads < 1 || (int64_t)batch * heads > (1LL << 22) - 8) return KDA_ERR_INVALID_ARG;
    const int64_t st = mul({batch, heads, KDA_HEAD_DIM, KDA_HEAD_DIM});
    if (st < 0) return KDA_ERR_INVALID_ARG;
    const Range r[] = {{state, st * 4}, {trans_p, st * 4}, {trans_q, trans_q ? st * 4 : 0}};
    if (any_overlap(r, 3, 1)) return KDA_ERR_INVALID_ARG;
    const int rc = kda::launch_transition_apply(trans_p, trans_q, state, batch * heads,
                                                static_cast<hipStream_t>(stream));
    return rc == 0 ? KDA_OK : KDA_ERR_HIP;
}

namespace {

// records and metadata of the varlen workspace: (record floats, byte size) or -1
struct VarlenWs {
    int64_t max_records, meta_offset_floats, bytes;
};
VarlenWs varlen_ws(int n_seqs, int heads, int total, int chunk)
{
    VarlenWs w{-1, -1, -1};
    if (n_seqs < 1 || heads < 1 || total < 1 || !chunk_ok(chunk) || n_seqs > KDA_VARLEN_MAX_SEQS) return w;
    const int64_t recs = mul({heads, (int64_t)total / chunk + n_seqs});  // >= heads * sum ceil(len / chunk)
    if (recs < 0 || recs > (1LL << 30)) return w;
    const int64_t floats = mul({recs, (int64_t)kda::chunk_record_floats(chunk)});
    if (floats < 0) return w;
    const int64_t meta = (floats + 63) / 64 * 64;  // 256-byte aligned
    w.max_records = recs;
    w.meta_offset_floats = meta;
    w.bytes = meta * 4 + 2 * ((int64_t)n_seqs + 1) * 4;
    return w;
}

}  // namespace

KDA_API size_t kda_chunk_prefill_varlen_workspace_bytes(int n_seqs, int heads, int total_tokens, int chunk)
{
    const VarlenWs w = varlen_ws(n_seqs, heads, total_tokens, chunk);
    return w.bytes < 0 ? 0 : (size_t)w.bytes;
}

KDA_API int kda_chunk_prefill_varlen(const float* q, const float* k, const float* v, const float* gate,
                                     const float* beta, float* state, float* out, const int* cu_seqlens, int n_seqs,
                                     int heads, int total_tokens, int chunk, void* workspace, size_t workspace_bytes,
                                     void* stream)
{
    if (!q || !k || !v || !gate || !beta || !state || !out || !cu_seqlens) return KDA_ERR_INVALID_ARG;
    if (!aligned({q, k, v, gate, state, out, workspace}) || !aligned({beta, cu_seqlens}, 4))
        return KDA_ERR_INVALID_ARG;
    if (n_seqs < 1 || heads < 1 || total_tokens < 1 || n_seqs > KDA_VARLEN_MAX_SEQS) return KDA_ERR_INVALID_ARG;
    if (!chunk_ok(chunk)) return KDA_ERR_UNSUPPORTED;
    if (heads > KDA_PREFILL_MAX_HEADS) return KDA_ERR_INVALID_ARG;
    if ((int64_t)n_seqs * heads > 0x7fffffffLL / 64) return KDA_ERR_INVALID_ARG;  // scan grid
    const VarlenWs w = varlen_ws(n_seqs, heads, total_tokens, chunk);
    const int64_t vec = mul({total_tokens, heads, KDA_HEAD_DIM});
    const int64_t sca = mul({total_tokens, heads});
    const int64_t st = mul({n_seqs, heads, KDA_HEAD_DIM, KDA_HEAD_DIM});
    if (w.bytes < 0 || vec < 0 || sca < 0 || st < 0) return KDA_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < (size_t)w.bytes) return KDA_ERR_WORKSPACE;
    const Range r[] = {{out, vec * 4}, {state, st * 4}, {workspace, w.bytes}, {q, vec * 4},
                       {k, vec * 4},   {v, vec * 4},    {gate, vec * 4},      {beta, sca * 4},
                       {cu_seqlens, ((int64_t)n_seqs + 1) * 4}};
    if (any_overlap(r, 9, 3)) return KDA_ERR_INVALID_ARG;
    const int rc = kda::launch_chunk_prefill_varlen(q, k, v, gate, beta, state, out, cu_seqlens, n_seqs, heads,
                                                    total_tokens, chunk, static_cast<float*>(workspace),
                                                    (size_t)w.meta_offset_floats, w.max_records,
                                                    static_cast<hipStream_t>(stream));
    return rc == 0 ? KDA_OK : KDA_ERR_HIP;
}

KDA_API int kda_chunk_prefill_varlen_bf16(const uint16_t* qkv, const float* gate, const float* beta, float* state,
                                          float* out, const int* cu_seqlens, int n_seqs, int heads, int total_tokens,
                                          int chunk, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!qkv || !gate || !beta || !state || !out || !cu_seqlens) return KDA_ERR_INVALID_ARG;
    if (!aligned({qkv, gate, state, out, workspace}) || !aligned({beta, cu_seqlens}, 4)) return KDA_ERR_INVALID_ARG;
    if (n_seqs < 1 || heads < 1 || total_tokens < 1 || n_seqs > KDA_VARLEN_MAX_SEQS) return KDA_ERR_INVALID_ARG;
    if (!chunk_ok(chunk)) return KDA_ERR_UNSUPPORTED;
    if (heads > KDA_PREFILL_MAX_HEADS) return KDA_ERR_INVALID_ARG;
    if ((int64_t)n_seqs * heads > 0x7fffffffLL / 64) return KDA_ERR_INVALID_ARG;  // scan grid
    const VarlenWs w = varlen_ws(n_seqs, heads, total_tokens, chunk);
    const int64_t x = mul({total_tokens, 3, heads, KDA_HEAD_DIM});
    const int64_t vec = mul({total_tokens, heads, KDA_HEAD_DIM});
    const int64_t sca = mul({total_tokens, heads});
    const int64_t st = mul({n_seqs, heads, KDA_HEAD_DIM, KDA_HEAD_DIM});
    if (w.bytes < 0 || x < 0 || vec < 0 || sca < 0 || st < 0) return KDA_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < (size_t)w.bytes) return KDA_ERR_WORKSPACE;
    const Range r[] = {{out, vec * 4},  {state, st * 4}, {workspace, w.bytes}, {qkv, x * 2},
                       {gate, vec * 4}, {beta, sca * 4}, {cu_seqlens, ((int64_t)n_seqs + 1) * 4}};
    if (any_overlap(r, 7, 3)) return KDA_ERR_INVALID_ARG;
    const int rc = kda::launch_chunk_prefill_varlen_bf16(qkv, gate, beta, state, out, cu_seqlens, n_seqs, heads,
                                                         total_tokens, chunk, static_cast<float*>(workspace),
                                                         (size_t)w.meta_offset_floats, w.max_records,
                                                         static_cast<hipStream_t>(stream));
    return rc == 0 ? KDA_OK : KDA_ERR_HIP;
}

KDA_API int kda_chunk_prefill_varlen_fused(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state,
                                           const float* gate, const float* beta, float* state, float* out,
                                           const int* cu_seqlens, int n_seqs, int heads, int total_tokens, int chunk,
                                           int conv_kernel, float l2_eps, void* workspace, size_t workspace_bytes,
                                           void* stream)
{
    if (!qkv || !conv_w || !conv_state || !gate || !beta || !state || !out || !cu_seqlens) return KDA_ERR_INVALID_ARG;
    if (!aligned({qkv, conv_w, conv_state, gate, state, out, workspace}) || !aligned({beta, cu_seqlens}, 4))
        return KDA_ERR_INVALID_ARG;
    if (n_seqs < 1 || heads < 1 || total_tokens < 1 || n_seqs > KDA_VARLEN_MAX_SEQS) return KDA_ERR_INVALID_ARG;
    if (heads > KDA_PREFILL_MAX_HEADS || conv_kernel < 1) return KDA_ERR_INVALID_ARG;
    if (!(isfinite(l2_eps) && l2_eps >= KDA_GATED_RMSNORM_MIN_EPS)) return KDA_ERR_INVALID_ARG;
    if (!chunk_ok(chunk) || conv_kernel != 4) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)n_seqs * heads > 0x7fffffffLL / 64) return KDA_ERR_INVALID_ARG;  // scan grid
    const VarlenWs w = varlen_ws(n_seqs, heads, total_tokens, chunk);
    const int64_t C = 3 * (int64_t)heads * KDA_HEAD_DIM;
    const int64_t x = mul({total_tokens, C});
    const int64_t cw = mul({C, conv_kernel});
    const int64_t cs = mul({n_seqs, C, conv_kernel});
    const int64_t vec = mul({total_tokens, heads, KDA_HEAD_DIM});
    const int64_t sca = mul({total_tokens, heads});
    const int64_t st = mul({n_seqs, heads, KDA_HEAD_DIM, KDA_HEAD_DIM});
    if (w.bytes < 0 || x < 0 || cw < 0 || cs < 0 || vec < 0 || sca < 0 || st < 0) return KDA_ERR_INVALID_ARG;
    if (mul({total_tokens, C, 2}) > 0x7fffffffLL || mul({n_seqs, C}) > 0x7fffffffLL) return KDA_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < (size_t)w.bytes) return KDA_ERR_WORKSPACE;
    const Range r[] = {{out, vec * 4},   {state, st * 4}, {conv_state, cs * 4}, {workspace, w.bytes},
                       {qkv, x * 2},     {conv_w, cw * 2}, {gate, vec * 4},     {beta, sca * 4},
                       {cu_seqlens, ((int64_t)n_seqs + 1) * 4}};
    if (any_overlap(r, 9, 4)) return KDA_ERR_INVALID_ARG;
    const int rc = kda::launch_chunk_prefill_varlen_fused(qkv, conv_w, conv_state, gate, beta, state, out, cu_seqlens,
                                                          n_seqs, heads, total_tokens, chunk, l2_eps,
                                                          static_cast<float*>(workspace), (size_t)w.meta_offset_floats,
                                                          w.max_records, static_cast<hipStream_t>(stream));
    return rc == 0 ? KDA_OK : KDA_ERR_HIP;
}

namespace {

// decode_k with FP32 q, k, v or, when qkv is not null, packed BF16 q | k | v rows; with gp, the gate
// from kda_gate of gp->g_raw (gate must be null) and beta holding logits
int recurrent_checked(const float* q, const float* k, const float* v, const uint16_t* qkv, const float* gate,
                      const float* beta, float* state, float* out, float* snapshots, int n_snapshots, int batch,
                      int heads, int T, void* stream, const kda::GateParams* gp = nullptr)
{
    if ((!qkv && (!q || !k || !v)) || !(gate || gp) || !beta || !state || !out) return KDA_ERR_INVALID_ARG;
    if (gp && (qkv || !gate_inputs_ok(gp->g_raw, gp->dt_bias, gp->a_log, gp->lower))) return KDA_ERR_INVALID_ARG;
    if (!aligned({q, k, v, qkv, gate, state, out, snapshots}) || !aligned({beta}, 4)) return KDA_ERR_INVALID_ARG;
    if (batch < 1 || heads < 1 || T < 1) return KDA_ERR_INVALID_ARG;
    if (n_snapshots < 0 || n_snapshots > T || (n_snapshots > 0 && !snapshots)) return KDA_ERR_INVALID_ARG;
    const int64_t vec = mul({batch, T, heads, KDA_HEAD_DIM});
    const int64_t sca = mul({batch, T, heads});
    const int64_t st = mul({batch, heads, KDA_HEAD_DIM, KDA_HEAD_DIM});
    const int64_t sn = mul({n_snapshots, batch, heads, KDA_HEAD_DIM, KDA_HEAD_DIM});
    if (vec < 0 || sca < 0 || st < 0 || sn < 0) return KDA_ERR_INVALID_ARG;
    if ((int64_t)batch * heads > kda::recurrent_max_units()) return KDA_ERR_INVALID_ARG;
    const int64_t hd = mul({heads, KDA_HEAD_DIM});
    const Range r[] = {{out, vec * 4},  {state, st * 4}, {n_snapshots ? snapshots : nullptr, sn * 4},
                       {q, vec * 4},    {k, vec * 4},    {v, vec * 4},
                       {qkv, vec * 6},  {gate, vec * 4}, {beta, sca * 4},
                       {gp ? gp->g_raw : nullptr, vec * 2}, {gp ? gp->dt_bias : nullptr, hd * 4},
                       {gp ? gp->a_log : nullptr, (int64_t)heads * 4}};
    if (any_overlap(r, 12, 3)) return KDA_ERR_INVALID_ARG;
    const int rc = kda::launch_recurrent(qkv ? nullptr : q, qkv ? nullptr : k, qkv ? nullptr : v, qkv, gate, beta,
                                         state, out, n_snapshots ? snapshots : nullptr, n_snapshots, batch, heads, T,
                                         static_cast<hipStream_t>(stream), gp);
    return rc == 0 ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

KDA_API int kda_recurrent_k(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                            float* state, float* out, float* snapshots, int n_snapshots, int batch, int heads,
                            int T, void* stream)
{
    if (!q || !k || !v) return KDA_ERR_INVALID_ARG;
    return recurrent_checked(q, k, v, nullptr, gate, beta, state, out, snapshots, n_snapshots, batch, heads, T,
                             stream);
}

KDA_API int kda_recurrent_step(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                               float* state, float* out, int batch, int heads, void* stream)
{
    return kda_recurrent_k(q, k, v, gate, beta, state, out, nullptr, 0, batch, heads, 1, stream);
}

KDA_API int kda_recurrent_k_gated(const float* q, const float* k, const float* v, const uint16_t* g_raw,
                                  const float* beta_logit, const float* dt_bias, const float* a_log,
                                  float gate_lower_bound, float* state, float* out, float* snapshots, int n_snapshots,
                                  int batch, int heads, int T, void* stream)
{
    if (!q || !k || !v) return KDA_ERR_INVALID_ARG;
    const kda::GateParams gp{reinterpret_cast<const unsigned short*>(g_raw), dt_bias, a_log, gate_lower_bound};
    if (!gate_inputs_ok(g_raw, dt_bias, a_log, gate_lower_bound)) return KDA_ERR_INVALID_ARG;
    return recurrent_checked(q, k, v, nullptr, nullptr, beta_logit, state, out, snapshots, n_snapshots, batch, heads,
                             T, stream, &gp);
}

KDA_API int kda_recurrent_step_gated(const float* q, const float* k, const float* v, const uint16_t* g_raw,
                                     const float* beta_logit, const float* dt_bias, const float* a_log,
                                     float gate_lower_bound, float* state, float* out, int batch, int heads,
                                     void* stream)
{
    return kda_recurrent_k_gated(q, k, v, g_raw, beta_logit, dt_bias, a_log, gate_lower_bound, state, out, nullptr, 0,
                                 batch, heads, 1, stream);
}

KDA_API int kda_recurrent_k_bf16(const uint16_t* qkv, const float* gate, const float* beta, float* state, float* out,
                                 float* snapshots, int n_snapshots, int batch, int heads, int T, void* stream)
{
    if (!qkv) return KDA_ERR_INVALID_ARG;
    return recurrent_checked(nullptr, nullptr, nullptr, qkv, gate, beta, state, out, snapshots, n_snapshots, batch,
                             heads, T, stream);
}

KDA_API int kda_recurrent_step_bf16(const uint16_t* qkv, const float* gate, const float* beta, float* state,
                                    float* out, int batch, int heads, void* stream)
{
    return kda_recurrent_k_bf16(qkv, gate, beta, state, out, nullptr, 0, batch, heads, 1, stream);
}

KDA_API int kda_recurrent_k_bf16_norm(const uint16_t* qkv, const float* gate, const float* beta, float* state,
                                      float* out, const uint16_t* out_gate, const uint16_t* o_norm, float eps,
                                      uint16_t* y, float* snapshots, int n_snapshots, int batch, int heads, int T,
                                      void* stream)
{
    if (!qkv || !gate || !beta || !state || !out_gate || !o_norm || !y) return KDA_ERR_INVALID_ARG;
    if (!aligned({qkv, gate, state, out, snapshots, out_gate, o_norm, y}) || !aligned({beta}, 4))
        return KDA_ERR_INVALID_ARG;
    if (!(isfinite(eps) && eps >= KDA_GATED_RMSNORM_MIN_EPS)) return KDA_ERR_INVALID_ARG;
    if (batch < 1 || heads < 1 || T < 1) return KDA_ERR_INVALID_ARG;
    if (n_snapshots < 0 || n_snapshots > T || (n_snapshots > 0 && !snapshots)) return KDA_ERR_INVALID_ARG;
    const int64_t vec = mul({batch, T, heads, KDA_HEAD_DIM});
    const int64_t sca = mul({batch, T, heads});
    const int64_t st = mul({batch, heads, KDA_HEAD_DIM, KDA_HEAD_DIM});
    const int64_t sn = mul({n_snapshots, batch, heads, KDA_HEAD_DIM, KDA_HEAD_DIM});
    if (vec < 0 || sca < 0 || st < 0 || sn < 0) return KDA_ERR_INVALID_ARG;
    if ((int64_t)batch * heads > 0x7fffffffLL - 8) return KDA_ERR_INVALID_ARG;  // one workgroup per head
    const Range r[] = {{y, vec * 2},       {state, st * 4},        {out, vec * 4},
                       {n_snapshots ? snapshots : nullptr, sn * 4}, {qkv, vec * 6}, {gate, vec * 4},
                       {beta, sca * 4},    {out_gate, vec * 2},    {o_norm, KDA_HEAD_DIM * 2}};
    if (any_overlap(r, 9, 4)) return KDA_ERR_INVALID_ARG;
    const int rc = kda::launch_recurrent_norm(qkv, gate, beta, state, out, n_snapshots ? snapshots : nullptr,
                                              n_snapshots, batch, heads, T, out_gate, o_norm, y, eps,
                                              static_cast<hipStream_t>(stream));
    return rc == 0 ? KDA_OK : KDA_ERR_HIP;
}

KDA_API int kda_recurrent_step_bf16_norm(const uint16_t* qkv, const float* gate, const float* beta, float* state,
                                         float* out, const uint16_t* out_gate, const uint16_t* o_norm, float eps,
                                         uint16_t* y, int batch, int heads, void* stream)
{
    return kda_recurrent_k_bf16_norm(qkv, gate, beta, state, out, out_gate, o_norm, eps, y, nullptr, 0, batch, heads,
                                     1, stream);
}

KDA_API int kda_gated_rmsnorm(const float* core, const uint16_t* out_gate, const uint16_t* o_norm, uint16_t* out,
                              int rows, int heads, float eps, void* stream)
{
    if (!core || !out_gate || !o_norm || !out || rows < 1 || heads < 1) return KDA_ERR_INVALID_ARG;
    if (!aligned({core, out_gate, o_norm, out})) return KDA_ERR_INVALID_ARG;
    if (!(isfinite(eps) && eps >= KDA_GATED_RMSNORM_MIN_EPS)) return KDA_ERR_INVALID_ARG;
    const int64_t n_vec = mul({rows, heads});
    const int64_t elems = mul({n_vec, KDA_HEAD_DIM});
    if (n_vec < 0 || elems < 0 || n_vec > INT64_C(0x7fffffff) * 8) return KDA_ERR_INVALID_ARG;  // grid bound
    const Range r[] = {{out, elems * 2}, {core, elems * 4}, {out_gate, elems * 2}, {o_norm, KDA_HEAD_DIM * 2}};
    if (any_overlap(r, 4, 1)) return KDA_ERR_INVALID_ARG;
    const int rc = kda::launch_gated_rmsnorm(core, out_gate, o_norm, out, n_vec, eps, static_cast<hipStream_t>(stream));
    return rc == 0 ? KDA_OK : KDA_ERR_HIP;
}

namespace {

// the front end with FP32 q, k, v outputs or, when conv_out is not null, BF16 conv_out
int front_end_checked(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state, float* q, float* k, float* v,
                      uint16_t* conv_out, float* conv_snapshots, int n_snapshots, int batch, int heads, int T,
                      int conv_kernel, float l2_eps, void* stream)
{
    if (!qkv || !conv_w || !conv_state || (!conv_out && (!q || !k || !v))) return KDA_ERR_INVALID_ARG;
    if (!aligned({qkv, conv_w, conv_state, q, k, v, conv_out, conv_snapshots})) return KDA_ERR_INVALID_ARG;
    if (batch < 1 || heads < 1 || T < 1 || heads > KDA_PREFILL_MAX_HEADS) return KDA_ERR_INVALID_ARG;
    if (n_snapshots < 0 || n_snapshots > T || (n_snapshots > 0 && !conv_snapshots)) return KDA_ERR_INVALID_ARG;
    if (conv_kernel < 1) return KDA_ERR_INVALID_ARG;
    if (conv_kernel > KDA_FRONT_END_MAX_CONV_KERNEL) return KDA_ERR_UNSUPPORTED;
    if (!(isfinite(l2_eps) && l2_eps >= KDA_GATED_RMSNORM_MIN_EPS)) return KDA_ERR_INVALID_ARG;
    const int64_t C = 3 * (int64_t)heads * KDA_HEAD_DIM;
    const int64_t x = mul({batch, T, C});
    const int64_t w = mul({C, conv_kernel});
    const int64_t st = mul({batch, C, conv_kernel});
    const int64_t sn = mul({n_snapshots, batch, C, conv_kernel});
    const int64_t vec = mul({batch, T, heads, KDA_HEAD_DIM});
    if (x < 0 || w < 0 || st < 0 || sn < 0 || vec < 0) return KDA_ERR_INVALID_ARG;
    if (mul({batch, 3, heads}) > 0x7fffffffLL) return KDA_ERR_INVALID_ARG;  // one wave per head vector
    if (conv_out) q = k = v = nullptr;
    const Range r[] = {{q, vec * 4},          {k, vec * 4}, {v, vec * 4}, {conv_out, x * 2},
                       {conv_state, st * 4}, {n_snapshots ? conv_snapshots : nullptr, sn * 4},
                       {qkv, x * 2},          {conv_w, w * 2}};
    if (any_overlap(r, 8, 6)) return KDA_ERR_INVALID_ARG;
    const int rc = kda::launch_front_end(qkv, conv_w, conv_state, q, k, v, conv_out,
                                         n_snapshots ? conv_snapshots : nullptr, n_snapshots, batch, heads, T,
                                         conv_kernel, l2_eps, static_cast<hipStream_t>(stream));
    return rc == 0 ? KDA_OK : KDA_ERR_HIP;
}

// The decode step from the raw projections (front end, gate, core, gated RMSNorm in one kernel).
int decode_fused_checked(const uint16_t* qkv_proj, const uint16_t* conv_w, float* conv_state, float* conv_snapshots,
                         const float* gate, const float* beta, const kda::GateParams* gp, float* state,
                         float* snapshots, int n_snapshots, const uint16_t* out_gate, const uint16_t* o_norm,
                         float norm_eps, float l2_eps, uint16_t* y, float* out, int batch, int heads, int T,
                         int conv_kernel, void* stream)
{
    if (!qkv_proj || !conv_w || !conv_state || !beta || !state || !out_gate || !o_norm || !y)
        return KDA_ERR_INVALID_ARG;
    if (gp ? !gate_inputs_ok(gp->g_raw, gp->dt_bias, gp->a_log, gp->lower) : !gate) return KDA_ERR_INVALID_ARG;
    if (!aligned({qkv_proj, conv_w, conv_state, conv_snapshots, gate, state, snapshots, out_gate, o_norm, y, out}) ||
        !aligned({beta}, 4))
        return KDA_ERR_INVALID_ARG;
    if (batch < 1 || heads < 1 || T < 1 || heads > KDA_PREFILL_MAX_HEADS) return KDA_ERR_INVALID_ARG;
    if (n_snapshots < 0 || n_snapshots > T || (n_snapshots > 0 && (!snapshots || !conv_snapshots)))
        return KDA_ERR_INVALID_ARG;
    if (conv_kernel < 1) return KDA_ERR_INVALID_ARG;
    if (!(isfinite(norm_eps) && norm_eps >= KDA_GATED_RMSNORM_MIN_EPS)) return KDA_ERR_INVALID_ARG;
    if (!(isfinite(l2_eps) && l2_eps >= KDA_GATED_RMSNORM_MIN_EPS)) return KDA_ERR_INVALID_ARG;
    if (conv_kernel > KDA_FRONT_END_MAX_CONV_KERNEL) return KDA_ERR_UNSUPPORTED;
    const int64_t C = 3 * (int64_t)heads * KDA_HEAD_DIM;
    const int64_t x = mul({batch, T, C});
    const int64_t w = mul({C, conv_kernel});
    const int64_t cst = mul({batch, C, conv_kernel});
    const int64_t csn = mul({n_snapshots, batch, C, conv_kernel});
    const int64_t vec = mul({batch, T, heads, KDA_HEAD_DIM});
    const int64_t sca = mul({batch, T, heads});
    const int64_t st = mul({batch, heads, KDA_HEAD_DIM, KDA_HEAD_DIM});
    const int64_t sn = mul({n_snapshots, batch, heads, KDA_HEAD_DIM, KDA_HEAD_DIM});
    if (x < 0 || w < 0 || cst < 0 || csn < 0 || vec < 0 || sca < 0 || st < 0 || sn < 0) return KDA_ERR_INVALID_ARG;
    if ((int64_t)batch * heads > 0x7fffffffLL - 8) return KDA_ERR_INVALID_ARG;  // one workgroup per head
    if (!n_snapshots) snapshots = conv_snapshots = nullptr;
    const Range r[] = {{y, vec * 2},
                       {state, st * 4},
                       {out, vec * 4},
                       {snapshots, sn * 4},
                       {conv_state, cst * 4},
                       {conv_snapshots, csn * 4},
                       {qkv_proj, x * 2},
                       {conv_w, w * 2},
                       {gate, vec * 4},
                       {beta, sca * 4},
                       {out_gate, vec * 2},
                       {o_norm, KDA_HEAD_DIM * 2},
                       {gp ? gp->g_raw : nullptr, vec * 2},
                       {gp ? gp->dt_bias : nullptr, (int64_t)heads * KDA_HEAD_DIM * 4},
                       {gp ? gp->a_log : nullptr, (int64_t)heads * 4}};
    if (any_overlap(r, 15, 6)) return KDA_ERR_INVALID_ARG;
    const int rc = kda::launch_decode_fused(qkv_proj, conv_w, conv_state, conv_snapshots, gate, beta, gp, state, out,
                                            snapshots, n_snapshots, batch, heads, T, conv_kernel, out_gate, o_norm, y,
                                            norm_eps, l2_eps, static_cast<hipStream_t>(stream));
    return rc == 0 ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

KDA_API int kda_decode_front_end(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state, float* q, float* k,
                                 float* v, float* conv_snapshots, int n_snapshots, int batch, int heads, int T,
                                 int conv_kernel, float l2_eps, void* stream)
{
    if (!q || !k || !v) return KDA_ERR_INVALID_ARG;
    return front_end_checked(qkv, conv_w, conv_state, q, k, v, nullptr, conv_snapshots, n_snapshots, batch, heads, T,
                             conv_kernel, l2_eps, stream);
}

KDA_API int kda_decode_front_end_bf16(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state,
                                      uint16_t* conv_out, float* conv_snapshots, int n_snapshots, int batch,
                                      int heads, int T, int conv_kernel, float l2_eps, void* stream)
{
    if (!conv_out) return KDA_ERR_INVALID_ARG;
    return front_end_checked(qkv, conv_w, conv_state, nullptr, nullptr, nullptr, conv_out, conv_snapshots,
                             n_snapshots, batch, heads, T, conv_kernel, l2_eps, stream);
}

KDA_API int kda_prefill_front_end(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state, float* q, float* k,
                                  float* v, int batch, int heads, int T, int chunk, int conv_kernel, float l2_eps,
                                  void* stream)
{
    if (!qkv || !conv_w || !conv_state || !q || !k || !v) return KDA_ERR_INVALID_ARG;
    if (!aligned({qkv, conv_w, conv_state, q, k, v})) return KDA_ERR_INVALID_ARG;
    if (batch < 1 || heads < 1 || T < 1 || heads > KDA_PREFILL_MAX_HEADS) return KDA_ERR_INVALID_ARG;
    if (conv_kernel < 1) return KDA_ERR_INVALID_ARG;
    if (!(isfinite(l2_eps) && l2_eps >= KDA_GATED_RMSNORM_MIN_EPS)) return KDA_ERR_INVALID_ARG;
    if (!chunk_ok(chunk) || conv_kernel > KDA_FRONT_END_MAX_CONV_KERNEL) return KDA_ERR_UNSUPPORTED;
    const int64_t t_pad = ((int64_t)T + chunk - 1) / chunk * chunk;
    const int64_t C = 3 * (int64_t)heads * KDA_HEAD_DIM;
    const int64_t x = mul({batch, T, C});
    const int64_t w = mul({C, conv_kernel});
    const int64_t st = mul({batch, C, conv_kernel});
    const int64_t vec = mul({batch, t_pad, heads, KDA_HEAD_DIM});
    if (x < 0 || w < 0 || st < 0 || vec < 0 || t_pad > 0x7fffffffLL) return KDA_ERR_INVALID_ARG;
    // one wave per (sequence, 32-token strip, part, head) vector; one thread per (sequence, channel)
    if (mul({batch, (T + 31) / 32, 3, heads}) > 0x7fffffffLL || mul({batch, C}) > 0x7fffffffLL)
        return KDA_ERR_INVALID_ARG;
    const Range r[] = {{q, vec * 4}, {k, vec * 4}, {v, vec * 4}, {conv_state, st * 4}, {qkv, x * 2}, {conv_w, w * 2}};
    if (any_overlap(r, 6, 4)) return KDA_ERR_INVALID_ARG;
    const int rc = kda::launch_prefill_front_end(qkv, conv_w, conv_state, q, k, v, batch, heads, T, (int)t_pad,
                                                 conv_kernel, l2_eps, static_cast<hipStream_t>(stream));
    return rc == 0 ? KDA_OK : KDA_ERR_HIP;
}

namespace {

int prefill_fused_checked(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state, const float* gate,
                          const float* beta, const kda::GateParams* gp, float* state, float* out, int batch, int heads,
                          int T, int chunk, int conv_kernel, float l2_eps, void* workspace, size_t workspace_bytes,
                          void* stream)
{
    if (!qkv || !conv_w || !conv_state || !beta || !state || !out) return KDA_ERR_INVALID_ARG;
    if (gp ? !gate_inputs_ok(gp->g_raw, gp->dt_bias, gp->a_log, gp->lower) : !gate) return KDA_ERR_INVALID_ARG;
    if (!aligned({qkv, conv_w, conv_state, gate, state, out, workspace}) || !aligned({beta}, 4))
        return KDA_ERR_INVALID_ARG;
    if (batch < 1 || heads < 1 || T < 1 || heads > KDA_PREFILL_MAX_HEADS) return KDA_ERR_INVALID_ARG;
    if (conv_kernel < 1) return KDA_ERR_INVALID_ARG;
    if (!(isfinite(l2_eps) && l2_eps >= KDA_GATED_RMSNORM_MIN_EPS)) return KDA_ERR_INVALID_ARG;
    if (!chunk_ok(chunk) || conv_kernel != 4) return KDA_ERR_UNSUPPORTED;
    const int64_t need = prefill_ws_bytes(batch, heads, T, chunk);
    const int64_t t_pad = ((int64_t)T + chunk - 1) / chunk * chunk;
    const int64_t C = 3 * (int64_t)heads * KDA_HEAD_DIM;
    const int64_t x = mul({batch, T, C});
    const int64_t w = mul({C, conv_kernel});
    const int64_t cs = mul({batch, C, conv_kernel});
    const int64_t vec = mul({batch, t_pad, heads, KDA_HEAD_DIM});
    const int64_t sca = mul({batch, t_pad, heads});
    const int64_t st = mul({batch, heads, KDA_HEAD_DIM, KDA_HEAD_DIM});
    if (need < 0 || x < 0 || w < 0 || cs < 0 || vec < 0 || sca < 0 || st < 0 || t_pad > 0x7fffffffLL)
        return KDA_ERR_INVALID_ARG;
    if (mul({T, C, 2}) > 0x7fffffffLL) return KDA_ERR_INVALID_ARG;  // 32-bit byte offsets inside one sequence
    if ((int64_t)batch * heads > 0x7fffffffLL / 64 || mul({batch, C}) > 0x7fffffffLL) return KDA_ERR_INVALID_ARG;
    if ((int64_t)batch * heads * (t_pad / chunk) > (1LL << 30)) return KDA_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < (size_t)need) return KDA_ERR_WORKSPACE;
    const Range r[] = {{out, vec * 4},
                       {state, st * 4},
                       {conv_state, cs * 4},
                       {workspace, need},
                       {qkv, x * 2},
                       {conv_w, w * 2},
                       {gate, vec * 4},
                       {beta, sca * 4},
                       {gp ? gp->g_raw : nullptr, vec * 2},
                       {gp ? gp->dt_bias : nullptr, (int64_t)heads * KDA_HEAD_DIM * 4},
                       {gp ? gp->a_log : nullptr, (int64_t)heads * 4}};
    if (any_overlap(r, 11, 4)) return KDA_ERR_INVALID_ARG;
    const int rc = kda::launch_chunk_prefill_fused(qkv, conv_w, conv_state, gate, beta, gp, state, out, batch, heads,
                                                   T, (int)t_pad, chunk, l2_eps, static_cast<float*>(workspace),
                                                   static_cast<hipStream_t>(stream));
    return rc == 0 ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

KDA_API int kda_chunk_prefill_fused(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state, const float* gate,
                                    const float* beta, float* state, float* out, int batch, int heads, int T, int chunk,
                                    int conv_kernel, float l2_eps, void* workspace, size_t workspace_bytes,
                                    void* stream)
{
    return prefill_fused_checked(qkv, conv_w, conv_state, gate, beta, nullptr, state, out, batch, heads, T, chunk,
                                 conv_kernel, l2_eps, workspace, workspace_bytes, stream);
}

KDA_API int kda_chunk_prefill_fused_gated(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state,
                                          const uint16_t* g_raw, const float* beta_logit, const float* dt_bias,
                                          const float* a_log, float gate_lower_bound, float* state, float* out,
                                          int batch, int heads, int T, int chunk, int conv_kernel, float l2_eps,
                                          void* workspace, size_t workspace_bytes, void* stream)
{
    const kda::GateParams gp{reinterpret_cast<const unsigned short*>(g_raw), dt_bias, a_log, gate_lower_bound};
    return prefill_fused_checked(qkv, conv_w, conv_state, nullptr, beta_logit, &gp, state, out, batch, heads, T,
                                 chunk, conv_kernel, l2_eps, workspace, workspace_bytes, stream);
}

KDA_API int kda_prefill_front_end_varlen(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state, float* q,
                                         float* k, float* v, const int* cu_seqlens, int n_seqs, int heads,
                                         int total_tokens, int conv_kernel, float l2_eps, void* stream)
{
    if (!qkv || !conv_w || !conv_state || !q || !k || !v || !cu_seqlens) return KDA_ERR_INVALID_ARG;
    if (!aligned({qkv, conv_w, conv_state, q, k, v}) || !aligned({cu_seqlens}, 4)) return KDA_ERR_INVALID_ARG;
    if (n_seqs < 1 || n_seqs > KDA_VARLEN_MAX_SEQS || heads < 1 || heads > KDA_PREFILL_MAX_HEADS || total_tokens < 1)
        return KDA_ERR_INVALID_ARG;
    if (conv_kernel < 1) return KDA_ERR_INVALID_ARG;
    if (!(isfinite(l2_eps) && l2_eps >= KDA_GATED_RMSNORM_MIN_EPS)) return KDA_ERR_INVALID_ARG;
    if (conv_kernel > KDA_FRONT_END_MAX_CONV_KERNEL) return KDA_ERR_UNSUPPORTED;
    const int64_t C = 3 * (int64_t)heads * KDA_HEAD_DIM;
    const int64_t x = mul({total_tokens, C});
    const int64_t w = mul({C, conv_kernel});
    const int64_t st = mul({n_seqs, C, conv_kernel});
    const int64_t vec = mul({total_tokens, heads, KDA_HEAD_DIM});
    if (x < 0 || w < 0 || st < 0 || vec < 0) return KDA_ERR_INVALID_ARG;
    // one wave per (32-token strip, part, head) vector; one thread per (sequence, channel)
    if (mul({(total_tokens + 31) / 32, 3, heads}) > 0x7fffffffLL || mul({n_seqs, C}) > 0x7fffffffLL)
        return KDA_ERR_INVALID_ARG;
    const Range r[] = {{q, vec * 4},  {k, vec * 4},       {v, vec * 4}, {conv_state, st * 4},
                       {qkv, x * 2},  {conv_w, w * 2},    {cu_seqlens, ((int64_t)n_seqs + 1) * 4}};
    if (any_overlap(r, 7, 4)) return KDA_ERR_INVALID_ARG;
    const int rc = kda::launch_prefill_front_end_varlen(qkv, conv_w, conv_state, q, k, v, cu_seqlens, n_seqs, heads,
                                                        total_tokens, conv_kernel, l2_eps,
                                                        static_cast<hipStream_t>(stream));
    return rc == 0 ? KDA_OK : KDA_ERR_HIP;
}

KDA_API int kda_decode_fused_k(const uint16_t* qkv_proj, const uint16_t* conv_w, float* conv_state,
                               float* conv_snapshots, const float* gate, const float* beta, float* state,
                               float* snapshots, int n_snapshots, const uint16_t* out_gate, const uint16_t* o_norm,
                               float norm_eps, float l2_eps, uint16_t* y, float* out, int batch, int heads, int T,
                               int conv_kernel, void* stream)
{
    return decode_fused_checked(qkv_proj, conv_w, conv_state, conv_snapshots, gate, beta, nullptr, state, snapshots,
                                n_snapshots, out_gate, o_norm, norm_eps, l2_eps, y, out, batch, heads, T, conv_kernel,
                                stream);
}

KDA_API int kda_decode_fused_step(const uint16_t* qkv_proj, const uint16_t* conv_w, float* conv_state,
                                  const float* gate, const float* beta, float* state, const uint16_t* out_gate,
                                  const uint16_t* o_norm, float norm_eps, float l2_eps, uint16_t* y, float* out,
                                  int batch, int heads, int conv_kernel, void* stream)
{
    return kda_decode_fused_k(qkv_proj, conv_w, conv_state, nullptr, gate, beta, state, nullptr, 0, out_gate, o_norm,
                              norm_eps, l2_eps, y, out, batch, heads, 1, conv_kernel, stream);
}

KDA_API int kda_decode_fused_k_gated(const uint16_t* qkv_proj, const uint16_t* conv_w, float* conv_state,
                                     float* conv_snapshots, const uint16_t* g_raw, const float* beta_logit,
                                     const float* dt_bias, const float* a_log, float gate_lower_bound, float* state,
                                     float* snapshots, int n_snapshots, const uint16_t* out_gate,
                                     const uint16_t* o_norm, float norm_eps, float l2_eps, uint16_t* y, float* out,
                                     int batch, int heads, int T, int conv_kernel, void* stream)
{
    const kda::GateParams gp{reinterpret_cast<const unsigned short*>(g_raw), dt_bias, a_log, gate_lower_bound};
    return decode_fused_checked(qkv_proj, conv_w, conv_state, conv_snapshots, nullptr, beta_logit, &gp, state,
                                snapshots, n_snapshots, out_gate, o_norm, norm_eps, l2_eps, y, out, batch, heads, T,
                                conv_kernel, stream);
}

KDA_API int kda_decode_fused_step_gated(const uint16_t* qkv_proj, const uint16_t* conv_w, float* conv_state,
                                        const uint16_t* g_raw, const float* beta_logit, const float* dt_bias,
                                        const float* a_log, float gate_lower_bound, float* state,
                                        const uint16_t* out_gate, const uint16_t* o_norm, float norm_eps,
                                        float l2_eps, uint16_t* y, float* out, int batch, int heads, int conv_kernel,
                                        void* stream)
{
    return kda_decode_fused_k_gated(qkv_proj, conv_w, conv_state, nullptr, g_raw, beta_logit, dt_bias, a_log,
                                    gate_lower_bound, state, nullptr, 0, out_gate, o_norm, norm_eps, l2_eps, y, out,
                                    batch, heads, 1, conv_kernel, stream);
}
