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
// (every NaN is the largest key; the first one wins).  Only rows holding a
// NaN come here, so it reads one element at a time and keeps few registers
// (a call's register count is the largest of its callees').
template <int BLOCK, typename T>
__device__ __noinline__ uint64_t row_argmax_exact(const T* row, int64_t V, ArgmaxShared<BLOCK>& sh) {
    uint64_t best = 0;   // below every packed key of an element
    for (int64_t i = threadIdx.x; i < V; i += BLOCK) {
        const uint64_t k = pack_key_index(float_key(load_elem(row + i)), i);
        best = k > best ? k : best;
    }
    return block_reduce<BLOCK>(best, OpMaxU64{}, (uint64_t)0, sh.red_u);
}

// Fast path: each thread keeps the maximum of its elements and the index of
// its first occurrence (found inside the 16-byte vector when the vector's
// maximum beats the running one); one packed (value key, index) maximum over
// the block then gives the value and its lowest index, -0 and +0 tying
// through the key.  Rows containing a NaN (detected from the magnitude bits)
// take the exact path.
//
// Rows whose byte length fits a buffer descriptor stream through one with the
// next batch of kArgmaxBatch loads issued before the current one is folded
// (loads past the row's end read zeros and are never folded), so every
// thread keeps between one and two batches in flight; each vector is loaded
// once.
//
// With STOP, `stop` is polled once per batch and the row is no longer read
// once it signals (the caller's sign that the row's result is no longer
// needed; the returned index is then meaningless).  Waves leave the loop on
// their own, with no barrier, and all of them still take part in the block
// reduction.
constexpr int kArgmaxBatch = 4;

//
// row_argmax_packed returns the packed (value key, index) maximum itself
// (0 for an empty row), which combines across pieces of a row by a plain
// 64-bit maximum once the indices are made absolute; row_argmax returns the
// index.
template <int BLOCK, bool NT, typename T, bool STOP = false>
__device__ uint64_t row_argmax_packed(const T* row, int64_t V, ArgmaxShared<BLOCK>& sh, RowStop* stop = nullptr) {
    constexpr int E = RowSplit<T>::kEpv;
    constexpr int U = kArgmaxBatch;
    const RowSplit<T> s(row, V);
    const int tid = threadIdx.x;
    float best = -INFINITY;
    int64_t bidx = -1;   // index of the thread's first maximum
    uint32_t mag = 0;

    if (tid < s.head) {
        const float v = load_elem(row + tid);
        mag = mag_acc_scalar(mag, v, T{});
        best = v;
        bidx = tid;
    }
    const T* body = row + s.head;
    // vector k of the body: its maximum, and where it first occurs if it beats best
    auto fold = [&](const u32x4 a, int64_t k) {
        float f[E];
        unpack(a, f);
        mag = mag_acc(mag, a, T{});
        float m = f[0];
#pragma unroll
        for (int e = 1; e < E; ++e) m = fmaxf(m, f[e]);
        if (bidx < 0 || m > best) {
            int e0 = E - 1;
#pragma unroll
            for (int e = E - 2; e >= 0; --e)
                if (f[e] == m) e0 = e;
            best = m;
            bidx = s.head + k * E + e0;
        }
    };
    auto poll = [&]() {
        if constexpr (STOP) stop->poll();
    };
    auto stopped = [&]() {
        if constexpr (STOP) return stop->check();
        else return false;
    };
    poll();
    int64_t i = tid;
    const int64_t body_bytes = s.nvec * 16;
    if (body_bytes + (int64_t)2 * U * BLOCK * 16 < ((int64_t)1 << 32)) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(body, (uint32_t)body_bytes);
        constexpr int kAux = NT ? 2 : 0;
        auto ld = [&](int64_t k) -> u32x4 {
            return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)k * 16u, 0, kAux));
        };
        u32x4 cur[U];
        if (i + (U - 1) * BLOCK < s.nvec) {
#pragma unroll
            for (int u = 0; u < U; ++u) cur[u] = ld(i + u * BLOCK);
            for (;;) {
                const int64_t nx = i + U * BLOCK;
                // checked before the next batch goes out: one batch at most is
                // read after the signal shows
                if (stopped()) {
                    i = s.nvec;
                    break;
                }
                poll();
                u32x4 nxt[U];
#pragma unroll
                for (int u = 0; u < U; ++u) nxt[u] = ld(nx + u * BLOCK);
#pragma unroll
                for (int u = 0; u < U; ++u) fold(cur[u], i + u * BLOCK);
                i = nx;
                if (i + (U - 1) * BLOCK >= s.nvec) {
                    // the last batch, partly or wholly past the end
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        if (i + u * BLOCK < s.nvec) fold(nxt[u], i + u * BLOCK);
                    i = s.nvec;
                    break;
                }
#pragma unroll
                for (int u = 0; u < U; ++u) cur[u] = nxt[u];
            }
        }
    } else {
        for (; i + (U - 1) * BLOCK < s.nvec; i += U * BLOCK) {
            if (stopped()) {
                i = s.nvec;
                break;
            }
            u32x4 a[U];
#pragma unroll
            for (int u = 0; u < U; ++u) a[u] = load_vec<NT>(body, i + u * BLOCK);
            poll();
#pragma unroll
            for (int u = 0; u < U; ++u) fold(a[u], i + u * BLOCK);
        }
    }
    for (; i < s.nvec; i += BLOCK) fold(load_vec<NT>(body, i), i);
    if (tid < s.tail) {
        const int64_t idx = s.head + s.nvec * E + tid;
        const float v = load_elem(row + idx);
        mag = mag_acc_scalar(mag, v, T{});
        if (bidx < 0 || v > best) {
            best = v;
            bidx = idx;
        }
    }

    // a NaN anywhere makes the packed key all ones, which no number reaches
    const uint64_t key = mag_has_nan(mag, T{}) ? ~(uint64_t)0
                         : bidx < 0          ? (uint64_t)0
                                             : pack_key_index(float_key(best), bidx);
    const uint64_t m = block_reduce<BLOCK>(key, OpMaxU64{}, (uint64_t)0, sh.red_u);
    if (m == ~(uint64_t)0) return row_argmax_exact<BLOCK>(row, V, sh);
    return m;
}

template <int BLOCK, bool NT, typename T, bool STOP = false>
__device__ __forceinline__ int64_t row_argmax(const T* row, int64_t V, ArgmaxShared<BLOCK>& sh,
                                              RowStop* stop = nullptr) {
    return packed_index(row_argmax_packed<BLOCK, NT, T, STOP>(row, V, sh, stop));
}

}  // namespace sv
