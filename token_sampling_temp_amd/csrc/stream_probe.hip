// Measurement probes used by the benchmark, not part of the verification
// library: the HBM read rate a plain kernel reaches on this GPU (the
// measured ceiling beside the 8 TB/s data-sheet peak), and the rate the
// Gumbel-max arithmetic reaches with no memory traffic at all (the measured
// ceiling of that arithmetic-bound kernel).
//
// Read stream:
// Each workgroup reads one contiguous region with non-temporal 16-byte loads,
// U loads in flight per thread, and folds the words with XOR so the loads
// cannot be removed; one word per workgroup is written to `sink`.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_gumbel.hpp"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4* __restrict__ buf, int64_t nvec,
                                                          int64_t per_wg, uint32_t* __restrict__ sink) {
    const int64_t lo = (int64_t)blockIdx.x * per_wg;
    int64_t hi = lo + per_wg;
    hi = hi < nvec ? hi : nvec;
    uint32_t acc = 0;
    int64_t i = lo + threadIdx.x;
    for (; i + (U - 1) * 256 < hi; i += U * 256) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * 256);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < hi; i += 256) {
        const u32x4 v = __builtin_nontemporal_load(buf + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    acc ^= __shfl_xor(acc, 1);
    acc ^= __shfl_xor(acc, 2);
    acc ^= __shfl_xor(acc, 4);
    acc ^= __shfl_xor(acc, 8);
    acc ^= __shfl_xor(acc, 16);
    acc ^= __shfl_xor(acc, 32);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + threadIdx.x / 64] = acc;
}

// Gumbel-max arithmetic alone: 1024-thread workgroups (as the sampling
// kernel) where every thread folds `groups` entry groups with the sampling
// kernel's own per-group function; the logits are made from the group index
// (four bit operations per group, as many as unpacking four bf16 logits), so
// nothing is loaded.  One word per wave goes to sink.
__global__ __launch_bounds__(1024) void gumbel_alu_kernel(int groups, int V, float invT, uint64_t seed,
                                                          uint64_t subseq, uint32_t* __restrict__ sink) {
    float best = -INFINITY;
    int bi = -1;
    const int g0 = (int)(blockIdx.x * 1024 + threadIdx.x);
    const int stride = (int)(gridDim.x * 1024);
    for (int k = 0; k < groups; ++k) {
        const int g = g0 + k * stride;
        const uint32_t bits = 0x3F800000u | (((uint32_t)g & 0xFFFFu) << 4);
        const float f[4] = {__uint_as_float(bits), __uint_as_float(bits | 1u), __uint_as_float(bits | 2u),
                            __uint_as_float(bits | 3u)};
        sv::gumbel_group(f, g, V, invT, seed, subseq, best, bi);
    }
    uint32_t acc = __float_as_uint(best) ^ (uint32_t)bi;
    acc ^= __shfl_xor(acc, 1);
    acc ^= __shfl_xor(acc, 2);
    acc ^= __shfl_xor(acc, 4);
    acc ^= __shfl_xor(acc, 8);
    acc ^= __shfl_xor(acc, 16);
    acc ^= __shfl_xor(acc, 32);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 16 + threadIdx.x / 64] = acc;
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16, 16-byte aligned) from `buf` with `grid`
// workgroups of 256 threads, each reading one contiguous region; `loads` (4,
// 8 or 16) 16-byte loads in flight per thread.  sink: device memory of
// 4 * grid words.  Returns 0 on success, 1 for bad arguments, 3 for a launch
// error.
int svprobe_read_stream(const void* buf, int64_t bytes, int grid, int loads, uint32_t* sink, void* stream) {
    if (!buf || !sink || bytes <= 0 || bytes % 16 != 0 || (uintptr_t)buf % 16 != 0 || grid < 1 || grid > 65536)
        return 1;
    const int64_t nvec = bytes / 16;
    const int64_t per_wg = (nvec + grid - 1) / grid;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const u32x4* b = static_cast<const u32x4*>(buf);
    if (loads == 4) hipLaunchKernelGGL(read_stream_kernel<4>, dim3(grid), dim3(256), 0, st, b, nvec, per_wg, sink);
    else if (loads == 8) hipLaunchKernelGGL(read_stream_kernel<8>, dim3(grid), dim3(256), 0, st, b, nvec, per_wg, sink);
    else if (loads == 16) hipLaunchKernelGGL(read_stream_kernel<16>, dim3(grid), dim3(256), 0, st, b, nvec, per_wg, sink);
    else return 1;
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

// Run the Gumbel-max arithmetic on `grid` workgroups of 1024 threads, each
// thread folding `groups` groups of 4 entries (grid * 1024 * groups * 4
// entries in all; V bounds the entry index as in the kernel and should exceed
// it).  sink: device memory of 16 * grid words.  Returns 0 on success, 1 for
// bad arguments, 3 for a launch error.
int svprobe_gumbel_alu(int groups, int grid, int V, uint32_t* sink, void* stream) {
    if (!sink || groups < 1 || grid < 1 || grid > 65536 || V < 1 ||
        (int64_t)grid * 1024 * groups > (int64_t)INT32_MAX / 4)
        return 1;
    hipLaunchKernelGGL(gumbel_alu_kernel, dim3(grid), dim3(1024), 0, static_cast<hipStream_t>(stream), groups, V,
                       1.25f, (uint64_t)0x243F6A8885A308D3ull, (uint64_t)7, sink);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
