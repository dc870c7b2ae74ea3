// Host-side declarations shared by the C ABI and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace kda {

// Floats of one (sequence, head, chunk) record of the prefill workspace.  The
// matrices the scan multiplies with are stored as 16x16 tiles in the order its
// MFMA lanes consume them ("A tiles": tile (a, b) holds rows 16a.., columns
// 16b..; lane l of a tile = row 16a + l%16, columns 16b + 4(l/16) + 0..3):
//   W      A tiles [C/16][8]    T diag(beta) (e^G o K)
//   U      [C/16][8][64][4]     T diag(beta) V as 16x16 accumulator tiles: row tile X,
//                               column block j, lane l, element e = U[16X + 4(l/16) + e][16j + l%16]
//   Qhat   A tiles [C/16][8]    e^G o Q
//   Ktil^T A tiles [8][C/16]    (e^{G_last - G} o K)^T
//   M      A tiles [C/16][C/16] lower-triangular (diagonal included) decayed Q K^T
//   gamma  [128]                e^{G_last}
constexpr size_t chunk_record_floats(int C) { return 4 * (size_t)C * 128 + (size_t)C * C + 128; }

int launch_recurrent(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                     float* state, float* out, float* snaps, int n_snap, int batch, int heads, int T,
                     hipStream_t stream);
long long recurrent_max_units();

int launch_chunk_prefill(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                         float* state, float* out, int batch, int heads, int T, int t_pad, int chunk,
                         float* workspace, hipStream_t stream);

}  // namespace kda
