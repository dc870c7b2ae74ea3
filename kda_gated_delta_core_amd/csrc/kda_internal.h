// Host-side declarations shared by the C ABI and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Floats of one (sequence, head, chunk) record of the prefill workspace.  The
// matrices the scan multiplies with are stored as 16x16 tiles in the order its
// MFMA lanes consume them ("A tiles": tile (a, b) holds rows 16a.., columns
// 16b..; lane l of a tile = row 16a + l%16, columns 16b + 4(l/16) + 0..3), the
// per-slice addends as accumulator tiles (tile (X, j), lane l, element e =
// row 16X + 4(l/16) + e, column 16j + l%16):
//   W      A tiles [C/16][8]            T diag(beta) (e^G o K)
//   U      accumulator tiles [C/16][8]  T diag(beta) V
//   P      A tiles [C/16][8]            e^G o Q - M W
//   R      accumulator tiles [C/16][8]  M U
//   Ktil^T A tiles [8][C/16]            (e^{G_last - G} o K)^T
//   gamma  [128]                        e^{G_last}
// with G the cumulative log-decay inside the chunk, T = (I + A)^-1 and M the
// lower-triangular decayed Q K^T of the chunk.
constexpr size_t chunk_record_floats(int C) { return 5 * (size_t)C * 128 + 128; }

// q, k, v FP32 [B][T][H][128]; or, when qkv is not null, q | k | v BF16 [B][T][3][H][128] from qkv.
// gp not null: the gate from kda_gate of gp->g_raw (gate unused), beta holding logits (FP32 q, k, v only)
struct GateParams;
int launch_recurrent(const float* q, const float* k, const float* v, const uint16_t* qkv, const float* gate,
                     const float* beta, float* state, float* out, float* snaps, int n_snap, int batch, int heads,
                     int T, hipStream_t stream, const GateParams* gp = nullptr);
long long recurrent_max_units();
// the BF16 decode with the gated RMSNorm of every output row fused in: y [B][T][H][128] BF16 from
// out_gate (same layout) and o_norm [128]; out (FP32 core rows) may be null
int launch_decode_fused(const uint16_t* qkv_proj, const uint16_t* conv_w, float* conv_state, float* conv_snaps,
                        const float* gate, const float* beta, const GateParams* gp, float* state, float* out,
                        float* snaps, int n_snap, int batch, int heads, int T, int conv_kernel,
                        const uint16_t* out_gate, const uint16_t* o_norm, uint16_t* y, float eps, float l2_eps,
                        hipStream_t stream);
int launch_recurrent_norm(const uint16_t* qkv, const float* gate, const float* beta, float* state, float* out,
                          float* snaps, int n_snap, int batch, int heads, int T, const uint16_t* out_gate,
                          const uint16_t* o_norm, uint16_t* y, float eps, hipStream_t stream);

int launch_chunk_prefill(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                         float* state, float* out, int batch, int heads, int T, int t_pad, int chunk,
                         float* workspace, hipStream_t stream);

// the prefill on BF16 q | k | v rows qkv [B][T_pad][3][H][128]; the rest as launch_chunk_prefill
int launch_chunk_prefill_bf16(const uint16_t* qkv, const float* gate, const float* beta, float* state, float* out,
                              int batch, int heads, int T, int t_pad, int chunk, float* workspace, hipStream_t stream);

// the prefill with kda_gate and the beta sigmoid inside the prepare: beta_logit [B][T_pad][H] logits,
// gp the gate inputs (g_raw [B][T_pad][H][128] BF16); the rest as launch_chunk_prefill
int launch_chunk_prefill_gated(const float* q, const float* k, const float* v, const float* beta_logit,
                               const GateParams& gp, float* state, float* out, int batch, int heads, int T, int t_pad,
                               int chunk, float* workspace, hipStream_t stream);

// the prefill with the front end fused into the prepare (conv_kernel 4): qkv BF16 [B][T][3][H][128],
// conv_w BF16 [3 H 128][4], conv state [B][3 H 128][4] (advanced by T inputs), gate, beta, state, out
// as launch_chunk_prefill
int launch_chunk_prefill_fused(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state, const float* gate,
                               const float* beta, const GateParams* gp, float* state, float* out, int batch, int heads,
                               int T, int t_pad, int chunk, float l2_eps, float* workspace, hipStream_t stream);

// varlen form of the fused prefill: qkv [total][3 H 128], conv state [n][3 H 128][4], the rest as
// launch_chunk_prefill_varlen
int launch_chunk_prefill_varlen_fused(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state,
                                      const float* gate, const float* beta, float* state, float* out,
                                      const int* cu_seqlens, int n_seqs, int heads, int total, int chunk,
                                      float l2_eps, float* workspace, size_t meta_offset_floats,
                                      long long max_records, hipStream_t stream);

// each sequence's conv state advanced by its inputs (qkv [total][3 H 128], offsets read clamped)
int launch_conv_state_advance_varlen(const uint16_t* qkv, float* conv_state, const int* cu_seqlens, int n_seqs,
                                     int heads, int total, int conv_kernel, hipStream_t stream);

// the conv state of every (sequence, channel) advanced by the T inputs of qkv [B][T][3 H 128]
int launch_conv_state_advance(const uint16_t* qkv, float* conv_state, int batch, int heads, int T, int conv_kernel,
                              hipStream_t stream);

// the transition form of the prefill: P, Q [B][H][128][128], the final state from S being P S + Q
int launch_chunk_prefill_transition(const float* q, const float* k, const float* v, const float* gate,
                                    const float* beta, float* trans_p, float* trans_q, int batch, int heads, int T,
                                    int t_pad, int chunk, float* workspace, hipStream_t stream);

// the scan half of the dense prefill, from the records of a preceding prepare in workspace
int launch_chunk_scan(const float* workspace, float* state, float* out, int batch, int heads, int T, int t_pad,
                      int chunk, hipStream_t stream);

// S <- P S + Q (Q may be null) for n states of 128 x 128, in place
int launch_transition_apply(const float* P, const float* Q, float* S, int n, hipStream_t stream);

int launch_chunk_prefill_varlen(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                                float* state, float* out, const int* cu_seqlens, int n_seqs, int heads, int total,
                                int chunk, float* workspace, size_t meta_offset_floats, long long max_records,
                                hipStream_t stream);

// the varlen prefill on BF16 q | k | v rows qkv [total][3][H][128]; the rest as launch_chunk_prefill_varlen
int launch_chunk_prefill_varlen_bf16(const uint16_t* qkv, const float* gate, const float* beta, float* state,
                                     float* out, const int* cu_seqlens, int n_seqs, int heads, int total, int chunk,
                                     float* workspace, size_t meta_offset_floats, long long max_records,
                                     hipStream_t stream);

// outputs FP32 q, k, v [B][T][H][128]; or, when conv_out is not null, BF16 [B][T][3][H][128] there
int launch_front_end(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state, float* q, float* k, float* v,
                     uint16_t* conv_out, float* snaps, int n_snap, int batch, int heads, int T, int conv_kernel,
                     float l2_eps, hipStream_t stream);

// prefill front end: q, k, v FP32 [B][t_pad][H][128], rows < T written; conv state advanced by T inputs
int launch_prefill_front_end(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state, float* q, float* k,
                             float* v, int batch, int heads, int T, int t_pad, int conv_kernel, float l2_eps,
                             hipStream_t stream);

// varlen prefill front end: qkv [total][conv_dim], conv state [n][conv_dim][K], q, k, v [total][H][128]
int launch_prefill_front_end_varlen(const uint16_t* qkv, const uint16_t* conv_w, float* conv_state, float* q,
                                    float* k, float* v, const int* cu_seqlens, int n_seqs, int heads, int total,
                                    int conv_kernel, float l2_eps, hipStream_t stream);

int launch_gated_rmsnorm(const float* core, const uint16_t* gate, const uint16_t* weight, uint16_t* out,
                         long long n_vec, float eps, hipStream_t stream);

}  // namespace kda
