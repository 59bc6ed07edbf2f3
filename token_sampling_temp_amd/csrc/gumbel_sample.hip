// Temperature-only target sampling by Gumbel-max, then strict chain
// acceptance.  Two forms: one workgroup per request walking rows j = 0..D in
// order and stopping after the first draft mismatch (no workspace), or, with a
// workspace, one workgroup per (request, row) with rows after a mismatch
// skipped through the request's stop word (sv_rowpar.hpp).  Every row is read
// when every row's sample is requested.
//
// Row j of request b: s_v = z_v / T + G_v, G_v = -ln(-ln u_v), u_v the uniform
// of Philox word v of stream (seed_b, offset_b + 32 j); the sample is the
// lowest-index maximum of s.  Thread work unit = 4 consecutive vocabulary
// entries = one Philox block.
//
// The scores are float: z / T as z * (1/T), and both logarithms from the
// hardware base-2 logarithm times ln 2 (a few ulp from correctly rounded
// values; only a near tie of the two best scores can tell them apart).
#include <algorithm>

#include "sv_argmax.hpp"
#include "sv_gumbel.hpp"
#include "sv_launch.hpp"
#include "sv_rowpar.hpp"

namespace sv {

constexpr int kGbBlock = 1024;

template <typename T>
__device__ __forceinline__ void load_group4(const T* row, int64_t v0, int64_t V, bool aligned, float (&f)[4]);

template <>
__device__ __forceinline__ void load_group4<float>(const float* row, int64_t v0, int64_t V, bool aligned,
                                                   float (&f)[4]) {
    if (aligned && v0 + 3 < V) {
        unpack(load_vec<true>(row + v0, 0), f);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = (v0 + e < V) ? row[v0 + e] : 0.0f;
    }
}

template <>
__device__ __forceinline__ void load_group4<uint16_t>(const uint16_t* row, int64_t v0, int64_t V, bool aligned,
                                                      float (&f)[4]) {
    if (aligned && v0 + 3 < V) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(row + v0));
        f[0] = __uint_as_float(w.x << 16);
        f[1] = __uint_as_float(w.x & 0xFFFF0000u);
        f[2] = __uint_as_float(w.y << 16);
        f[3] = __uint_as_float(w.y & 0xFFFF0000u);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = (v0 + e < V) ? bf16_to_float(row[v0 + e]) : 0.0f;
    }
}

// Rows that are 4 * sizeof(T)-byte aligned with V a multiple of 4: each
// thread keeps the loads of its next kPf groups in flight while it computes
// the Philox block and the scores of the current one (consume a slot, refill
// it), so the row's load latency hides behind the arithmetic.  Buffer loads
// with the row as the range read zeros past its end.  With STOP, `stop` is
// polled once per round of kPf groups and the row is no longer read once it
// signals (the result is then meaningless).
constexpr int kPf = 4;
template <int BLOCK, typename T, bool STOP>
__device__ __forceinline__ void row_gumbel_pipelined(const T* row, int Vi, float invT, uint64_t seed,
                                                     uint64_t subseq, float& best, int& bi, RowStop* stop,
                                                     int gbase) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    constexpr bool kF32 = sizeof(T) == 4;
    typedef typename std::conditional<kF32, u32x4, u32x2>::type Raw;
    const int ngroups = (Vi + 3) / 4;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(row, (uint32_t)((int64_t)Vi * (int64_t)sizeof(T)));
    constexpr int kAux = 2;   // non-temporal: the row is read once
    auto ld = [&](int g) -> Raw {
        const uint32_t off = (uint32_t)g * (uint32_t)(4 * sizeof(T));
        if constexpr (kF32) return __builtin_bit_cast(Raw, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kAux));
        else return __builtin_bit_cast(Raw, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kAux));
    };
    auto unpack4 = [&](const Raw r, float (&f)[4]) {
        if constexpr (kF32) {
            f[0] = __uint_as_float(r[0]);
            f[1] = __uint_as_float(r[1]);
            f[2] = __uint_as_float(r[2]);
            f[3] = __uint_as_float(r[3]);
        } else {
            f[0] = __uint_as_float(r[0] << 16);
            f[1] = __uint_as_float(r[0] & 0xFFFF0000u);
            f[2] = __uint_as_float(r[1] << 16);
            f[3] = __uint_as_float(r[1] & 0xFFFF0000u);
        }
    };
    const int tid = threadIdx.x;
    if constexpr (STOP) {
        stop->poll();
        if (stop->check()) return;
    }
    Raw slot[kPf];
#pragma unroll
    for (int j = 0; j < kPf; ++j) slot[j] = ld(tid + j * BLOCK);
    for (int g0 = tid; g0 < ngroups; g0 += kPf * BLOCK) {
        if constexpr (STOP) {
            if (stop->check()) break;
            stop->poll();
        }
#pragma unroll
        for (int j = 0; j < kPf; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            const int g = g0 + j * BLOCK;
            float f[4];
            unpack4(slot[j], f);
            slot[j] = ld(g + kPf * BLOCK);
            if (g < ngroups) gumbel_group(f, g, Vi, invT, seed, subseq, best, bi, gbase);
        }
    }
}

// The packed (score key, index) maximum of the row's scores, indices from
// the start of `row`; gbase: the Philox block of its first group (a piece
// of a longer row starting at entry 4 gbase).
template <int BLOCK, typename T, bool STOP = false>
__device__ uint64_t row_gumbel_packed(const T* row, int64_t V, float invT, uint64_t seed, uint64_t subseq,
                                      ArgmaxShared<BLOCK>& sh, RowStop* stop = nullptr, int gbase = 0) {
    const bool aligned = ((uintptr_t)row % (4 * sizeof(T))) == 0;
    const int Vi = (int)V;   // V < 2^31
    const int ngroups = (Vi + 3) / 4;
    // this thread's best score and its index; elements are visited in
    // increasing index order, so a strict comparison keeps the lowest index
    float best = -INFINITY;
    int bi = (int)threadIdx.x * 4 < Vi ? (int)threadIdx.x * 4 : -1;
    // whole groups only (V a multiple of 4), so no load straddles the row's end
    if (aligned && (Vi & 3) == 0 &&
        V * (int64_t)sizeof(T) + (int64_t)(kPf + 1) * BLOCK * 4 * (int64_t)sizeof(T) < ((int64_t)1 << 32)) {
        row_gumbel_pipelined<BLOCK, T, STOP>(row, Vi, invT, seed, subseq, best, bi, stop, gbase);
        const uint64_t key = bi < 0 ? 0 : pack_key_index(float_key(best), (int64_t)bi);
        return block_reduce<BLOCK>(key, OpMaxU64{}, (uint64_t)0, sh.red_u);
    }
    for (int g = threadIdx.x; g < ngroups; g += BLOCK) {
        const int v0 = g * 4;
        float f[4];
        load_group4<T>(row, v0, V, aligned, f);
        const uint4 w = philox_block_mad(seed, subseq, (uint64_t)(g + gbase));
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        if (v0 + 3 < Vi) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float sc = gumbel_score(f[e], invT, ws[e]);
                if (sc > best) {
                    best = sc;
                    bi = v0 + e;
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float sc = gumbel_score(f[e], invT, ws[e]);
                if (v0 + e < Vi && sc > best) {
                    best = sc;
                    bi = v0 + e;
                }
            }
        }
    }
    const uint64_t key = bi < 0 ? 0 : pack_key_index(float_key(best), (int64_t)bi);
    return block_reduce<BLOCK>(key, OpMaxU64{}, (uint64_t)0, sh.red_u);
}

template <int BLOCK, typename T, bool STOP = false>
__device__ __forceinline__ int64_t row_gumbel(const T* row, int64_t V, float invT, uint64_t seed, uint64_t subseq,
                                              ArgmaxShared<BLOCK>& sh, RowStop* stop = nullptr) {
    return packed_index(row_gumbel_packed<BLOCK, T, STOP>(row, V, invT, seed, subseq, sh, stop));
}

template <typename T>
__global__ __launch_bounds__(kGbBlock) void gumbel_sample_kernel(
    const T* __restrict__ logits, const float* __restrict__ temperature, const int32_t* __restrict__ draft_ids,
    const uint64_t* __restrict__ seed, const uint64_t* __restrict__ offset, int64_t B, int D, int64_t V,
    const int32_t* __restrict__ req_index, int32_t* __restrict__ accepted, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ sampled_out) {
    __shared__ ArgmaxShared<kGbBlock> sh;
    __shared__ int32_t s_y[kMaxDraft + 1];
    const int64_t b = req_index ? (int64_t)req_index[blockIdx.x] : (int64_t)blockIdx.x;
    if (b < 0 || b >= B) return;
    const int N = D + 1;
    const float Tm = temperature[b];
    const bool greedy = (double)Tm < kGreedyTemperature;
    const float invT = 1.0f / Tm;
    const uint64_t sd = seed[b], off = offset[b];
    const bool all_rows = sampled_out != nullptr;
    int L = -1;
    for (int j = 0; j < N; ++j) {
        const T* row = logits + ((int64_t)b * N + j) * V;
        const int64_t y = greedy ? row_argmax<kGbBlock, true>(row, V, sh)
                                 : row_gumbel<kGbBlock>(row, V, invT, sd, off + kRngSlotSpan * (uint64_t)j, sh);
        if (threadIdx.x == 0) s_y[j] = (int32_t)y;
        if (L < 0 && (j == D || draft_ids[(int64_t)b * D + j] != (int32_t)y)) {
            L = j;
            if (!all_rows) break;
        }
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < N) {
        const int64_t o = (int64_t)b * N + t;
        accepted[o] = t <= L ? s_y[t] : -1;
        if (sampled_out) sampled_out[o] = s_y[t];
    }
    if (t == 0) accept_len[b] = L;
}

// Row-parallel form: workgroup g takes row j = g / n_req of request slot
// g % n_req.
template <typename T>
__global__ __launch_bounds__(kGbBlock) void gumbel_rows_kernel(
    const T* __restrict__ logits, const float* __restrict__ temperature, const int32_t* __restrict__ draft_ids,
    const uint64_t* __restrict__ seed, const uint64_t* __restrict__ offset, int64_t B, int D, int64_t V,
    const int32_t* __restrict__ req_index, int64_t n_req, void* __restrict__ ws, int32_t* __restrict__ accepted,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ sampled_out) {
    __shared__ ArgmaxShared<kGbBlock> sh;
    __shared__ uint32_t s_stop;
    const int N = D + 1;
    const int j = (int)(blockIdx.x / (uint64_t)n_req);
    const int64_t slot = (int64_t)blockIdx.x - (int64_t)j * n_req;
    const int64_t b = req_index ? (int64_t)req_index[slot] : slot;
    if (b < 0 || b >= B) return;
    const RowPar rp(ws, slot);
    const float Tm = temperature[b];
    const int32_t xj = j < D ? draft_ids[b * D + j] : -1;
    // the request's last workgroup writes the outputs
    auto finish = [&](int L, int32_t yt) {
        const int t = threadIdx.x;
        if (t < N) {
            const int64_t o = b * N + t;
            accepted[o] = t <= L ? yt : -1;
            if (sampled_out) sampled_out[o] = yt;
        }
        if (t == 0) accept_len[b] = L;
    };
    // row 0 is always needed, and every row when all samples are asked for;
    // another row whose request already ended before it counts itself in and
    // leaves at once, else it stops as soon as an earlier row ends the chain
    const bool may_stop = !sampled_out && j > 0;
    if (threadIdx.x == 0)
        s_stop = may_stop && (__hip_atomic_load(rp.word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) &
                              (((uint64_t)1 << j) - 1)) != 0;
    __syncthreads();
    if (s_stop) {
        if (threadIdx.x >= kWave) return;
        int32_t yt = -1;
        const int L = rp.arrive(j, N, false, 0, yt);
        if (L >= 0) finish(L, yt);
        return;
    }
    RowStop stop(may_stop ? rp.word : nullptr, ((uint64_t)1 << j) - 1, &s_stop, true);
    const T* row = logits + ((int64_t)b * N + j) * V;
    const int64_t y = (double)Tm < kGreedyTemperature
                          ? row_argmax<kGbBlock, true, T, true>(row, V, sh, &stop)
                          : row_gumbel<kGbBlock, T, true>(row, V, 1.0f / Tm, seed[b],
                                                          offset[b] + kRngSlotSpan * (uint64_t)j, sh, &stop);
    if (threadIdx.x >= kWave) return;
    int32_t yt = -1;
    const int L = rp.arrive(j, N, j == D || xj != (int32_t)y, (int32_t)y, yt);
    if (L >= 0) finish(L, yt);
}

// Staged form (strict acceptance, samples of later rows not asked for).
// Drafts from another distribution rarely match a Gumbel sample, so most
// requests end at row 0; giving every (request, row) its own workgroup
// leaves a long tail of workgroups that start only to find their request
// ended.  Here workgroup g < n_req samples row 0 of request slot g; the
// request ends there (its outputs are written at once) or continues.  The
// other gridDim - n_req workgroups (helpers) wait for every request's row-0
// verdict, list the requests that continue, and share the rows 1..D of
// those requests cut into S pieces of seg entries (S chosen in the kernel
// from how many rows remain).  The pieces of a row meet in the workspace:
// each stores its packed (score key, absolute index) maximum with bit 31 set
// (an index below 2^31 keeps that bit in its field anyway, so 0 means not
// yet written) and counts itself in; the last combines them.  Each finished
// row joins the request's hand-off (sv_rowpar.hpp), row 0 having counted
// itself in first.
//
// Workspace: n_req hand-off lines, the request's state in bytes 120..123 of
// its line (0 not yet known, 1 continues, 2 done); then a 256-byte block whose
// first word counts finished helpers; then one 128-byte line per (request,
// row 1..D) for the pieces (a count, then S values from byte 8).  The last
// helper clears the states and its count; the hand-off and piece lines are
// cleared by their last users, so the workspace is zero at rest.
constexpr int64_t kGbStateOff = 120;
constexpr int64_t kGbPieceLine = 128;
constexpr int kGbPiecesMax = 15;

template <typename T>
__global__ __launch_bounds__(kGbBlock) void gumbel_staged_kernel(
    const T* __restrict__ logits, const float* __restrict__ temperature, const int32_t* __restrict__ draft_ids,
    const uint64_t* __restrict__ seed, const uint64_t* __restrict__ offset, int64_t B, int D, int64_t V,
    const int32_t* __restrict__ req_index, int64_t n_req, void* __restrict__ ws, int32_t* __restrict__ accepted,
    int32_t* __restrict__ accept_len) {
    __shared__ ArgmaxShared<kGbBlock> sh;
    __shared__ uint32_t s_stop;
    __shared__ uint32_t s_wsum[kGbBlock / kWave];
    __shared__ int32_t s_cont[kGbBlock];
    const int N = D + 1;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
    char* const wsb = static_cast<char*>(ws);
    auto state_of = [&](int64_t slot) { return reinterpret_cast<uint32_t*>(wsb + slot * kRowParLine + kGbStateOff); };
    // the outputs of request b (wave 0)
    auto finish = [&](int64_t b, int L, int32_t yt) {
        if (lane < N) accepted[b * N + lane] = lane <= L ? yt : -1;
        if (lane == 0) accept_len[b] = L;
    };
    if ((int64_t)blockIdx.x < n_req) {
        // ---- row 0 of request slot blockIdx.x
        const int64_t slot = blockIdx.x;
        const int64_t b = req_index ? (int64_t)req_index[slot] : slot;
        uint32_t* const st = state_of(slot);
        if (b < 0 || b >= B) {
            if (tid == 0) __hip_atomic_store(st, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        const float Tm = temperature[b];
        const T* row = logits + (int64_t)b * N * V;
        const int64_t y = (double)Tm < kGreedyTemperature
                              ? row_argmax<kGbBlock, true>(row, V, sh)
                              : row_gumbel<kGbBlock>(row, V, 1.0f / Tm, seed[b], offset[b], sh);
        if (tid >= kWave) return;
        if (draft_ids[b * D] != (int32_t)y) {   // the chain ends at row 0
            finish(b, 0, (int32_t)y);
            if (lane == 0) __hip_atomic_store(st, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        if (lane == 0) __hip_atomic_store(st, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const RowPar rp(ws, slot);
        int32_t yt = -1;
        const int L = rp.arrive(0, N, false, (int32_t)y, yt);
        if (L >= 0) finish(b, L, yt);
        return;
    }
    // ---- helpers.  Every row-0 workgroup was dispatched before this one and
    // waits on nothing, so each wait below ends; the bound only keeps a
    // broken invariant from hanging the device.
    const int64_t h = (int64_t)blockIdx.x - n_req, H = (int64_t)gridDim.x - n_req;
    uint32_t cont = 0;
    if (tid < n_req) {
        uint32_t v = 0;
        for (int spin = 0; spin < (1 << 22); ++spin) {
            v = __hip_atomic_load(state_of(tid), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (v) break;
            __builtin_amdgcn_s_sleep(2);
        }
        cont = v == 1u ? 1u : 0u;
    }
    // the continuing request slots, in slot order
    const uint32_t inc = wave_inclusive_sum(cont, lane);
    if (lane == kWave - 1) s_wsum[wid] = inc;
    __syncthreads();
    uint32_t pos = inc - cont, ncont = 0;
#pragma unroll
    for (int i = 0; i < kGbBlock / kWave; ++i) {
        const uint32_t t = s_wsum[i];
        if (i < wid) pos += t;
        ncont += t;
    }
    if (cont) s_cont[pos] = tid;
    __syncthreads();
    // pieces per row: about one piece per helper over all the rows to
    // evaluate, each of at least 4096 entries and a multiple of 64 (so a
    // piece keeps the row's alignment), at most kGbPiecesMax
    const int64_t nrows = (int64_t)ncont * D;
    int S = (int)max((int64_t)1, min((int64_t)kGbPiecesMax, min(nrows > 0 ? H / nrows : 1, V / 4096)));
    const int64_t seg = ((V + S - 1) / S + 63) / 64 * 64;
    S = (int)((V + seg - 1) / seg);
    // items in row order (every continuing request's row 1, then row 2, ...),
    // the pieces of a row together: when many requests continue, helpers
    // take the earlier rows first and a later row of a request whose chain
    // ended meanwhile stops early
    const int64_t per_row = (int64_t)ncont * S;
    const int64_t items = per_row * D;
    for (int64_t it = h; it < items; it += H) {
        const int j = 1 + (int)(it / per_row);
        const int64_t rem = it - (int64_t)(j - 1) * per_row;
        const int64_t k = rem / S;
        const int piece = (int)(rem - k * S);
        const int64_t slot = s_cont[k];
        const int64_t b = req_index ? (int64_t)req_index[slot] : slot;
        const RowPar rp(ws, slot);
        char* const line = wsb + n_req * kRowParLine + 256 + (slot * D + (j - 1)) * kGbPieceLine;
        uint32_t* const cnt = reinterpret_cast<uint32_t*>(line);
        uint64_t* const part = reinterpret_cast<uint64_t*>(line + 8);
        const float Tm = temperature[b];
        if (tid == 0) s_stop = 0;
        __syncthreads();
        // a piece of a row after one that ended the chain stops early
        RowStop stop(rp.word, ((uint64_t)1 << j) - 1, &s_stop, true);
        const int64_t off = (int64_t)piece * seg;
        const T* row = logits + ((int64_t)b * N + j) * V + off;
        const int64_t len = min(seg, V - off);
        const uint64_t m = (double)Tm < kGreedyTemperature
                               ? row_argmax_packed<kGbBlock, true, T, true>(row, len, sh, &stop)
                               : row_gumbel_packed<kGbBlock, T, true>(row, len, 1.0f / Tm, seed[b],
                                                                      offset[b] + kRngSlotSpan * (uint64_t)j, sh,
                                                                      &stop, (int)(off / 4));
        if (tid < kWave && S == 1) {
            // a whole row: no pieces to meet
            const int64_t y = packed_index(m);
            const int32_t xj = j < D ? draft_ids[b * D + j] : -1;
            int32_t yt = -1;
            const int L = rp.arrive(j, N, j == D || xj != (int32_t)y, (int32_t)y, yt);
            if (L >= 0) finish(b, L, yt);
        } else if (tid < kWave) {
            const uint64_t mine = (m & 0xFFFFFFFF00000000ull) |
                                  (uint64_t)((0xFFFFFFFFu - (uint32_t)(packed_index(m) + off)) | 0x80000000u);
            uint32_t prev = 0;
            if (lane == 0) {
                __hip_atomic_store(&part[piece], mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if ((uint32_t)__builtin_amdgcn_readfirstlane((int)prev) == (uint32_t)(S - 1)) {
                // the row's last piece: every piece stored its value before
                // its count, so each wait ends
                uint64_t v = 0;
                if (lane < S) {
                    for (int spin = 0; spin < (1 << 20); ++spin) {
                        v = __hip_atomic_load(&part[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        if (v) break;
                        __builtin_amdgcn_s_sleep(1);
                    }
                    __hip_atomic_store(&part[lane], (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                if (lane == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const int64_t y = packed_index(wave_allreduce(v, OpMaxU64{}));
                const int32_t xj = j < D ? draft_ids[b * D + j] : -1;
                int32_t yt = -1;
                const int L = rp.arrive(j, N, j == D || xj != (int32_t)y, (int32_t)y, yt);
                if (L >= 0) finish(b, L, yt);
            }
        }
        __syncthreads();   // the next item reuses the reduction's LDS and the stop flag
    }
    // ---- the last helper to finish sets the states and its count back to zero
    uint32_t* const done = reinterpret_cast<uint32_t*>(wsb + n_req * kRowParLine);
    if (tid == 0)
        s_stop = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(H - 1);
    __syncthreads();
    if (s_stop) {
        if (tid < n_req) __hip_atomic_store(state_of(tid), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (tid == 0) __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

int64_t gumbel_workspace_bytes(int64_t n_req, int D) {
    if (D <= 0 || n_req <= 0) return 0;
    return (n_req * kRowParLine + 256 + n_req * D * kGbPieceLine + 255) / 256 * 256;
}

hipError_t launch_gumbel_sample(const void* logits, int dtype, const float* temperature,
                                const int32_t* draft_ids, const uint64_t* seed, const uint64_t* offset,
                                int64_t B, int D, int64_t V, const int32_t* req_index, int64_t n_req,
                                int32_t* accepted, int32_t* accept_len, int32_t* sampled_out, void* workspace,
                                hipStream_t stream) {
    const dim3 block(kGbBlock);
    const int64_t cus = device_compute_units();
    // below two requests per CU, with a workspace: the staged form when only
    // the accepted tokens are asked for, else one workgroup per row
    if (workspace && gumbel_workspace_bytes(n_req, D) > 0 && n_req < 2 * cus && !sampled_out &&
        n_req <= kGbBlock) {
        const dim3 grid((unsigned)(n_req + cus));
        if (dtype == kDtypeBF16)
            hipLaunchKernelGGL(gumbel_staged_kernel<uint16_t>, grid, block, 0, stream,
                               static_cast<const uint16_t*>(logits), temperature, draft_ids, seed, offset, B, D, V,
                               req_index, n_req, workspace, accepted, accept_len);
        else
            hipLaunchKernelGGL(gumbel_staged_kernel<float>, grid, block, 0, stream, static_cast<const float*>(logits),
                               temperature, draft_ids, seed, offset, B, D, V, req_index, n_req, workspace, accepted,
                               accept_len);
        return hipGetLastError();
    }
    if (workspace && gumbel_workspace_bytes(n_req, D) > 0 && n_req < 2 * cus) {
        const dim3 grid((unsigned)(n_req * (D + 1)));
        if (dtype == kDtypeBF16)
            hipLaunchKernelGGL(gumbel_rows_kernel<uint16_t>, grid, block, 0, stream,
                               static_cast<const uint16_t*>(logits), temperature, draft_ids, seed, offset, B, D, V,
                               req_index, n_req, workspace, accepted, accept_len, sampled_out);
        else
            hipLaunchKernelGGL(gumbel_rows_kernel<float>, grid, block, 0, stream, static_cast<const float*>(logits),
                               temperature, draft_ids, seed, offset, B, D, V, req_index, n_req, workspace, accepted,
                               accept_len, sampled_out);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)n_req);
    if (dtype == kDtypeBF16)
        hipLaunchKernelGGL(gumbel_sample_kernel<uint16_t>, grid, block, 0, stream,
                           static_cast<const uint16_t*>(logits), temperature, draft_ids, seed, offset, B, D, V,
                           req_index, accepted, accept_len, sampled_out);
    else
        hipLaunchKernelGGL(gumbel_sample_kernel<float>, grid, block, 0, stream,
                           static_cast<const float*>(logits), temperature, draft_ids, seed, offset, B, D, V,
                           req_index, accepted, accept_len, sampled_out);
    return hipGetLastError();
}

}  // namespace sv
