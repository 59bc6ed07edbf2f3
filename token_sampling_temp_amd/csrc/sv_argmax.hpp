// Block-wide argmax of one row (lowest index among equal maxima).
#pragma once

#include "sv_common.hpp"

namespace sv {

template <int BLOCK>
struct ArgmaxShared {
    float red_f[BLOCK / kWave];
    int64_t red_i[BLOCK / kWave];
    uint64_t red_u[BLOCK / kWave];
    uint32_t red_m[BLOCK / kWave];
};

// Exact slow path: packed (order-preserving key, index) maximum.  Handles NaN
// (every NaN is the largest key; the first one wins).
template <int BLOCK, typename T>
__device__ int64_t row_argmax_exact(const T* row, int64_t V, ArgmaxShared<BLOCK>& sh) {
    uint64_t best = 0;
    bool any = false;
    row_foreach<BLOCK, false>(row, V, [&](float v, int64_t idx) {
        const uint64_t k = pack_key_index(float_key(v), idx);
        if (!any || k > best) best = k;
        any = true;
    });
    if (!any) best = 0;
    const uint64_t m = block_reduce<BLOCK>(best, OpMaxU64{}, (uint64_t)0, sh.red_u);
    return packed_index(m);
}

// Fast path: each thread keeps the maximum of its elements and the first
// 16-byte vector (or scalar) where that maximum appeared; the block maximum is
// reduced as a float (so -0 == +0), and the threads holding it re-read their
// one vector to locate the lowest index.  Rows containing a NaN (detected from
// the magnitude bits) take the exact path.
template <int BLOCK, bool NT, typename T>
__device__ int64_t row_argmax(const T* row, int64_t V, ArgmaxShared<BLOCK>& sh) {
    constexpr int E = RowSplit<T>::kEpv;
    const RowSplit<T> s(row, V);
    const int tid = threadIdx.x;
    float best = -INFINITY;
    int64_t bpos = -1;   // first element of the recorded vector/scalar
    int bw = 0;          // its width (E or 1)
    uint32_t mag = 0;

    if (tid < s.head) {
        const float v = load_elem(row + tid);
        mag = mag_acc_scalar(mag, v, T{});
        best = v;
        bpos = tid;
        bw = 1;
    }
    const T* body = row + s.head;
    auto vec_max = [](const float (&f)[E]) {
        float m = f[0];
#pragma unroll
        for (int e = 1; e < E; ++e) m = fmaxf(m, f[e]);
        return m;
    };
    int64_t i = tid;
    for (; i + 3 * BLOCK < s.nvec; i += 4 * BLOCK) {
        u32x4 a[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) a[u] = load_vec<NT>(body, i + u * BLOCK);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float f[E];
            unpack(a[u], f);
            mag = mag_acc(mag, a[u], T{});
            const float m = vec_max(f);
            if (bpos < 0 || m > best) {
                best = m;
                bpos = s.head + (i + u * BLOCK) * E;
                bw = E;
            }
        }
    }
    for (; i < s.nvec; i += BLOCK) {
        const u32x4 a = load_vec<NT>(body, i);
        float f[E];
        unpack(a, f);
        mag = mag_acc(mag, a, T{});
        const float m = vec_max(f);
        if (bpos < 0 || m > best) {
            best = m;
            bpos = s.head + i * E;
            bw = E;
        }
    }
    if (tid < s.tail) {
        const int64_t idx = s.head + s.nvec * E + tid;
        const float v = load_elem(row + idx);
        mag = mag_acc_scalar(mag, v, T{});
        if (bpos < 0 || v > best) {
            best = v;
            bpos = idx;
            bw = 1;
        }
    }

    const uint32_t nan_flag = mag_has_nan(mag, T{}) ? 1u : 0u;
    const uint32_t any_nan = block_reduce<BLOCK>(nan_flag, OpOrU32{}, 0u, sh.red_m);
    if (any_nan) return row_argmax_exact<BLOCK>(row, V, sh);

    const float M = block_reduce<BLOCK>(bpos >= 0 ? best : -INFINITY, OpMaxF{}, -INFINITY, sh.red_f);
    int64_t cand = INT64_MAX;
    if (bpos >= 0 && best == M) {
        if (bw == 1) {
            cand = bpos;
        } else {
            float f[E];
            unpack(load_vec<false>(row + bpos, 0), f);
#pragma unroll
            for (int e = E - 1; e >= 0; --e)
                if (f[e] == M) cand = bpos + e;
        }
    }
    return block_reduce<BLOCK>(cand, OpMinI64{}, (int64_t)INT64_MAX, sh.red_i);
}

}  // namespace sv
