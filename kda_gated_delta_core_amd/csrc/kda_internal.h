// Host-side declarations shared by the C ABI and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace kda {

// Floats of one (sequence, head, chunk) record of the prefill workspace:
//   W      [C][128]   T diag(beta) (e^G o K)
//   U      [C][128]   T diag(beta) V
//   Qhat   [C][128]   e^G o Q
//   Ktil^T [128][C]   (e^{G_last - G} o K)^T
//   M      [C][C]     lower-triangular (diagonal included) decayed Q K^T
//   gamma  [128]      e^{G_last}
constexpr size_t chunk_record_floats(int C) { return 4 * (size_t)C * 128 + (size_t)C * C + 128; }

int launch_recurrent(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                     float* state, float* out, float* snaps, int n_snap, int batch, int heads, int T,
                     hipStream_t stream);
long long recurrent_max_units();

int launch_chunk_prefill(const float* q, const float* k, const float* v, const float* gate, const float* beta,
                         float* state, float* out, int batch, int heads, int T, int t_pad, int chunk,
                         float* workspace, hipStream_t stream);

}  // namespace kda
