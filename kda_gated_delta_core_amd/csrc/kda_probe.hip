// Traffic-only probe (measurement tooling, not part of the KDA C ABI): the
// decode kernel's state access pattern with none of the recurrence's
// arithmetic.  Blocks map to (head, value slice) exactly as in the decode
// kernel (4 slices of 32 value columns per 128 x 128 head state, the slices of
// a head 8 blocks apart; thread = 4 adjacent columns x 4 key rows); each block
// reads its slice and writes it to n_out regions region_floats apart.  It
// gives the practical HBM rate of the decode patterns (1 read : 1 write in
// place; 1 read : 5 writes for a 4-row walk with snapshots), against which
// the decode kernels are read.
#include <hip/hip_runtime.h>

typedef float probe_f4 __attribute__((ext_vector_type(4)));

namespace {
constexpr int kSlices = 4;
constexpr int kColGroups = 128 / kSlices / 4;   // float4 column groups per slice
constexpr int kRowGroups = 256 / kColGroups;    // thread rows per block
constexpr int kRows = 128 / kRowGroups;         // key rows per thread
constexpr int kHeadF4 = 128 * 128 / 4;          // float4s per head state
}  // namespace

__global__ __launch_bounds__(256) void probe_state_traffic_kernel(const probe_f4* __restrict__ src,
                                                                  probe_f4* __restrict__ dst, int heads, int n_out,
                                                                  long long region_f4, int nontemporal)
{
    const int r = blockIdx.x % (8 * kSlices);
    const int slice = r / 8;
    const int head = blockIdx.x / (8 * kSlices) * 8 + r % 8;
    if (head >= heads) return;
    const int cg = threadIdx.x % kColGroups, rg = threadIdx.x / kColGroups;
    const size_t base = (size_t)head * kHeadF4 + slice * kColGroups + cg;
    probe_f4 v[kRows];
#pragma unroll
    for (int m = 0; m < kRows; ++m) {
        const probe_f4* p = src + base + (size_t)(rg + kRowGroups * m) * 32;
        v[m] = nontemporal ? __builtin_nontemporal_load(p) : *p;
    }
    for (int t = 0; t < n_out; ++t) {
#pragma unroll
        for (int m = 0; m < kRows; ++m) {
            probe_f4* p = dst + (size_t)t * region_f4 + base + (size_t)(rg + kRowGroups * m) * 32;
            if (nontemporal) __builtin_nontemporal_store(v[m], p);
            else *p = v[m];
        }
    }
}

// src: heads * 16384 floats; dst: (n_out - 1) * region_floats + heads * 16384
// floats (dst may equal src when n_out == 1: the in-place pattern).  Returns
// 0, or -1 on bad arguments or a launch error.
extern "C" __attribute__((visibility("default"))) int probe_state_traffic(const float* src, float* dst, int heads,
                                                                        int n_out, long long region_floats,
                                                                        int nontemporal, void* stream)
{
    if (!src || !dst || heads < 1 || heads > (1 << 24) || n_out < 1 || region_floats < (long long)heads * 16384 ||
        (region_floats & 3))
        return -1;
    const unsigned grid = ((unsigned)heads + 7u) / 8u * 8u * kSlices;
    hipLaunchKernelGGL(probe_state_traffic_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       (const probe_f4*)src, (probe_f4*)dst, heads, n_out, region_floats / 4, nontemporal);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}
