// Draft distributions over a reduced draft vocabulary, placed in the target
// vocabulary ("TensorRT-LLM _torch/speculative/interface.py", one-model
// sampler: draft entry s goes to target index (s + d2t[s]) mod V of a
// zero-filled row; without a table, to index s).
//
// The placement is done as a gather so that every target row is written
// once, with coalesced 16-byte stores: an inverse table t2d [V] (draft entry
// of each target entry, -1 for none) is built once per table, by a fill
// kernel and a scatter kernel; the expansion then reads t2d (the same V
// entries for every row, so an L2 hit after the first rows) and gathers the
// draft row (Vd entries, read once per row).  HBM-bound: 4 V bytes written and
// 4 Vd read per row.
#include "sv_common.hpp"
#include "sv_launch.hpp"

namespace sv {

constexpr int kD2tBlock = 256;

// t2d[t] = t for t < Vd when there is no table (the draft vocabulary is the
// first Vd target entries), else -1; the scatter kernel then fills in the table.
__global__ __launch_bounds__(kD2tBlock) void d2t_fill_kernel(int32_t* __restrict__ t2d, int64_t V, int64_t Vd,
                                                             bool identity) {
    for (int64_t t = (int64_t)blockIdx.x * kD2tBlock + threadIdx.x; t < V; t += (int64_t)gridDim.x * kD2tBlock)
        t2d[t] = (identity && t < Vd) ? (int32_t)t : -1;
}

// t2d[(s + d2t[s]) mod V] = s, a floor modulus; the offsets are reduced first
// so nothing overflows.  A target shared by several draft entries keeps the
// highest-numbered one (an atomic maximum over the -1 fill), as an in-order
// scatter would leave it; the result does not depend on thread timing.
__global__ __launch_bounds__(kD2tBlock) void d2t_scatter_kernel(const int64_t* __restrict__ d2t, int64_t Vd, int64_t V,
                                                                int32_t* __restrict__ t2d) {
    for (int64_t s = (int64_t)blockIdx.x * kD2tBlock + threadIdx.x; s < Vd; s += (int64_t)gridDim.x * kD2tBlock) {
        int64_t t = (s % V + d2t[s] % V) % V;
        if (t < 0) t += V;
        __hip_atomic_fetch_max(&t2d[t], (int32_t)s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// One workgroup per row (grid-stride over rows): out[t] = q[t2d[t]], 0 where
// t2d[t] is outside [0, Vd).  Rows whose output and the table are 16-byte
// aligned (V a multiple of 4) take 4 entries at a time with 16-byte loads of
// the table and 16-byte stores; others go entry by entry.
__global__ __launch_bounds__(kD2tBlock) void d2t_expand_kernel(const float* __restrict__ q,
                                                               const int32_t* __restrict__ t2d, int64_t rows,
                                                               int64_t Vd, int64_t V, float* __restrict__ out) {
    const int tid = threadIdx.x;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        float* o = out + r * V;
        const float* qr = q + r * Vd;
        if ((V & 3) == 0 && (uintptr_t)o % 16 == 0 && (uintptr_t)t2d % 16 == 0) {
            const int4* tv = reinterpret_cast<const int4*>(t2d);
            float4* ov = reinterpret_cast<float4*>(o);
            const int64_t nv = V / 4;
            auto gather = [&](const int4 sv) {
                float4 v;
                v.x = (sv.x >= 0 && sv.x < Vd) ? qr[sv.x] : 0.0f;
                v.y = (sv.y >= 0 && sv.y < Vd) ? qr[sv.y] : 0.0f;
                v.z = (sv.z >= 0 && sv.z < Vd) ? qr[sv.z] : 0.0f;
                v.w = (sv.w >= 0 && sv.w < Vd) ? qr[sv.w] : 0.0f;
                return v;
            };
            // four table vectors per thread are loaded before any gather, so
            // the dependent loads of four vectors are in flight together
            constexpr int kU = 4;
            int64_t i = tid;
            for (; i + (kU - 1) * kD2tBlock < nv; i += kU * kD2tBlock) {
                int4 sv[kU];
#pragma unroll
                for (int u = 0; u < kU; ++u) sv[u] = tv[i + u * kD2tBlock];
                float4 v[kU];
#pragma unroll
                for (int u = 0; u < kU; ++u) v[u] = gather(sv[u]);
#pragma unroll
                for (int u = 0; u < kU; ++u) ov[i + u * kD2tBlock] = v[u];
            }
            for (; i < nv; i += kD2tBlock) ov[i] = gather(tv[i]);
        } else {
            for (int64_t t = tid; t < V; t += kD2tBlock) {
                const int32_t s = t2d[t];
                o[t] = (s >= 0 && s < Vd) ? qr[s] : 0.0f;
            }
        }
    }
}

hipError_t launch_d2t_inverse(const int64_t* d2t, int64_t Vd, int64_t V, int32_t* t2d, hipStream_t stream) {
    const int64_t gf = (V + kD2tBlock - 1) / kD2tBlock;
    hipLaunchKernelGGL(d2t_fill_kernel, dim3((unsigned)(gf < 8192 ? gf : 8192)), dim3(kD2tBlock), 0, stream, t2d, V,
                       Vd, d2t == nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !d2t) return e;
    const int64_t gs = (Vd + kD2tBlock - 1) / kD2tBlock;
    hipLaunchKernelGGL(d2t_scatter_kernel, dim3((unsigned)(gs < 8192 ? gs : 8192)), dim3(kD2tBlock), 0, stream, d2t,
                       Vd, V, t2d);
    return hipGetLastError();
}

hipError_t launch_d2t_expand(const float* draft_probs, const int32_t* t2d, int64_t rows, int64_t Vd, int64_t V,
                             float* out, hipStream_t stream) {
    const int64_t grid = rows < 8192 ? rows : 8192;
    hipLaunchKernelGGL(d2t_expand_kernel, dim3((unsigned)grid), dim3(kD2tBlock), 0, stream, draft_probs, t2d, rows,
                       Vd, V, out);
    return hipGetLastError();
}

}  // namespace sv
