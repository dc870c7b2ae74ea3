// Traffic-only probe (measurement tooling, not part of the KDA C ABI): each
// workgroup reads one 32 KiB state slice, as the decode kernel's workgroups
// do, and writes it to n_out regions region_floats apart, with no arithmetic
// of the recurrence.  It gives the practical HBM rate of the decode access
// patterns (1 read : 1 write in place; 1 read : 5 writes for a 4-row walk
// with snapshots), against which the decode kernels are read.
#include <hip/hip_runtime.h>

typedef float probe_f4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void probe_state_traffic_kernel(const probe_f4* __restrict__ src,
                                                                  probe_f4* __restrict__ dst, int n_out,
                                                                  long long region_f4, int nontemporal)
{
    const probe_f4* s = src + (size_t)blockIdx.x * 2048;
    probe_f4 r[8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
        r[m] = nontemporal ? __builtin_nontemporal_load(s + threadIdx.x + 256 * m) : s[threadIdx.x + 256 * m];
    for (int t = 0; t < n_out; ++t) {
        probe_f4* d = dst + (size_t)t * region_f4 + (size_t)blockIdx.x * 2048;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            if (nontemporal) __builtin_nontemporal_store(r[m], d + threadIdx.x + 256 * m);
            else d[threadIdx.x + 256 * m] = r[m];
        }
    }
}

// src: units * 8192 floats; dst: (n_out - 1) * region_floats + units * 8192 floats
// (dst may equal src when n_out == 1: the in-place pattern).  Returns 0, or -1
// on bad arguments or a launch error.
extern "C" __attribute__((visibility("default"))) int probe_state_traffic(const float* src, float* dst, int units,
                                                                        int n_out, long long region_floats,
                                                                        int nontemporal, void* stream)
{
    if (!src || !dst || units < 1 || n_out < 1 || region_floats < (long long)units * 8192 || (region_floats & 3))
        return -1;
    hipLaunchKernelGGL(probe_state_traffic_kernel, dim3(units), dim3(256), 0, (hipStream_t)stream,
                       (const probe_f4*)src, (probe_f4*)dst, n_out, region_floats / 4, nontemporal);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}
