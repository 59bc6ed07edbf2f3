// Draft distributions over a reduced draft vocabulary, placed in the target
// vocabulary ("TensorRT-LLM _torch/speculative/interface.py", one-model
// sampler: draft entry s goes to target index (s + d2t[s]) mod V of a
// zero-filled row; without a table, to index s).
//
// The placement is done as a gather so that every target row is written
// once, with coalesced 16-byte stores: an inverse table t2d [V] (draft entry
// of each target entry, -1 for none) is built once per table, by a fill
// kernel and a scatter kernel; the expansion keeps a tile of t2d in registers
// and, for each of its rows, gathers the draft entries the tile names (Vd
// entries per row in all) and stores the tile's columns.  HBM-bound: 4 V bytes
// written and 4 Vd read per row.
#include <algorithm>

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

// out[t] = q[t2d[t]], 0 where t2d[t] is outside [0, Vd).
//
// Aligned case (V a multiple of 4, 16-byte aligned output and table): the
// grid is (column tile, row group).  A workgroup loads its tile of the table
// once (kD2tVec 16-byte vectors per thread, kD2tTile entries) and keeps it in
// registers while it writes those columns of its rows, two rows at a time:
// per row only the draft gathers (issued together, their addresses already
// in registers) and 16-byte non-temporal stores.  Otherwise one workgroup
// per row goes entry by entry.
constexpr int kD2tVec = 4;
constexpr int64_t kD2tTile = (int64_t)kD2tBlock * 4 * kD2tVec;

__global__ __launch_bounds__(kD2tBlock) void d2t_expand_kernel(const float* __restrict__ q,
                                                               const int32_t* __restrict__ t2d, int64_t rows,
                                                               int64_t Vd, int64_t V, float* __restrict__ out,
                                                               int64_t rows_per_group) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    const int tid = threadIdx.x;
    const int64_t tile = blockIdx.x, r0 = (int64_t)blockIdx.y * rows_per_group;
    const int64_t r1 = min(rows, r0 + rows_per_group);
    const int64_t nv = V / 4;
    const int4* tv = reinterpret_cast<const int4*>(t2d);
    int4 sv[kD2tVec];
    bool in[kD2tVec];
#pragma unroll
    for (int u = 0; u < kD2tVec; ++u) {
        const int64_t i = tile * (kD2tTile / 4) + u * kD2tBlock + tid;
        in[u] = i < nv;
        sv[u] = in[u] ? tv[i] : make_int4(-1, -1, -1, -1);
    }
    auto gather = [&](const float* qr, const int4 x) {
        f4 v;
        v.x = (x.x >= 0 && x.x < Vd) ? qr[x.x] : 0.0f;
        v.y = (x.y >= 0 && x.y < Vd) ? qr[x.y] : 0.0f;
        v.z = (x.z >= 0 && x.z < Vd) ? qr[x.z] : 0.0f;
        v.w = (x.w >= 0 && x.w < Vd) ? qr[x.w] : 0.0f;
        return v;
    };
    auto put = [&](int64_t r, int u, const f4 v) {
        if (in[u])
            __builtin_nontemporal_store(
                v, reinterpret_cast<f4*>(out + r * V) + tile * (kD2tTile / 4) + u * kD2tBlock + tid);
    };
    int64_t r = r0;
    for (; r + 1 < r1; r += 2) {
        f4 a[kD2tVec], c[kD2tVec];
#pragma unroll
        for (int u = 0; u < kD2tVec; ++u) {
            a[u] = gather(q + r * Vd, sv[u]);
            c[u] = gather(q + (r + 1) * Vd, sv[u]);
        }
#pragma unroll
        for (int u = 0; u < kD2tVec; ++u) {
            put(r, u, a[u]);
            put(r + 1, u, c[u]);
        }
    }
    if (r < r1) {
#pragma unroll
        for (int u = 0; u < kD2tVec; ++u) put(r, u, gather(q + r * Vd, sv[u]));
    }
}

__global__ __launch_bounds__(kD2tBlock) void d2t_expand_rows_kernel(const float* __restrict__ q,
                                                                    const int32_t* __restrict__ t2d, int64_t rows,
                                                                    int64_t Vd, int64_t V, float* __restrict__ out) {
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        float* o = out + r * V;
        const float* qr = q + r * Vd;
        for (int64_t t = threadIdx.x; t < V; t += kD2tBlock) {
            const int32_t s = t2d[t];
            o[t] = (s >= 0 && s < Vd) ? qr[s] : 0.0f;
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
    if ((V & 3) == 0 && (uintptr_t)out % 16 == 0 && (uintptr_t)t2d % 16 == 0) {
        // about sixteen workgroups per CU: tiles x row groups (measured on
        // 1280 rows of 128256: 4 per CU 211 us, 8 184 us, 16 178 us, 32 208 us)
        const int64_t tiles = (V + kD2tTile - 1) / kD2tTile;
        const int64_t want = std::max<int64_t>(1, 16 * (int64_t)device_compute_units() / tiles);
        const int64_t groups = std::min<int64_t>(rows, std::min<int64_t>(want, 65535));
        const int64_t per = (rows + groups - 1) / groups;
        hipLaunchKernelGGL(d2t_expand_kernel, dim3((unsigned)tiles, (unsigned)((rows + per - 1) / per)),
                           dim3(kD2tBlock), 0, stream, draft_probs, t2d, rows, Vd, V, out, per);
    } else {
        const int64_t grid = rows < 8192 ? rows : 8192;
        hipLaunchKernelGGL(d2t_expand_rows_kernel, dim3((unsigned)grid), dim3(kD2tBlock), 0, stream, draft_probs,
                           t2d, rows, Vd, V, out);
    }
    return hipGetLastError();
}

}  // namespace sv
