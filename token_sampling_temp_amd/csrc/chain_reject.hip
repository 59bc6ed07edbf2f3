// Chain rejection sampling of a linear draft.
//
// Work split: each request's row is cut into C segments and every (request,
// segment) pair is one 256-thread workgroup; C is chosen so the grid holds
// about one workgroup per CU (a large batch gets one workgroup per request).
//
// 1. Probe (every workgroup of a request, redundantly; the lines are shared
//    in L2): lane i < D of wave 0 loads p_i(x_i), q_i(x_i), forms the Philox
//    uniform u_i while those loads are in flight and decides u_i * q < p
//    exactly in double; lane D takes the final uniform.  L = first rejected
//    position (D if none), from a ballot.
// 2. Segment pass: r_v = max(0, p_L[v] - q_L[v]) (or p_D[v] for the bonus) is
//    summed in double per 1024-entry chunk; waves stream their chunks with
//    several rounds of 16-byte loads in flight, one sum per chunk.
// 3. A workgroup that owns the whole row keeps its chunk sums in LDS.
//    Otherwise the sums are published and the last workgroup of the request
//    to finish (agent-scope acquire-release counter, reset afterwards)
//    collects them.  The locating workgroup prefix-sums the chunk sums in
//    order (one wave, four sums per lane), finds the chunk holding u_f * R,
//    re-reads it and scans its sub-tiles lane by lane.  Zero-mass entries are
//    never selected.  Sums use fixed reduction trees, so results are
//    reproducible run to run.
// 4. Degenerate rows (residual mass not positive) fall back to a draw from the
//    target row by the same workgroup, then to floor(u_f * V).
// Without draft distributions (target-only verify) each draft is a point mass
// at its id: the probe takes q(x) = 1 and the residual pass streams p_L alone,
// the rejected id weighing max(0, p - 1).
// Draft rows over a smaller draft vocabulary (read through the inverse table
// t2d) are copied whole into LDS when they fit (a separate instantiation with
// dynamic LDS); the residual pass then streams p_L and t2d and looks the draft
// entries up in LDS instead of gathering them from global memory.
#include <mutex>

#include "sv_draw.hpp"
#include "sv_launch.hpp"

#ifndef SV_CHAIN_TARGET_WGS
#define SV_CHAIN_TARGET_WGS 256    // one 256-thread workgroup per CU on 256 CUs
#endif
#ifndef SV_CHAIN_DEPTH
#define SV_CHAIN_DEPTH 3           // rounds of loads in flight per wave
#endif
#ifndef SV_CHAIN_DEPTH_ONE_ROW
#define SV_CHAIN_DEPTH_ONE_ROW 1   // the same for a row streamed alone beside two-row requests
#endif
#ifndef SV_CHAIN_DEPTH_ALL_ONE_ROW
#define SV_CHAIN_DEPTH_ALL_ONE_ROW 2   // when every request streams one row
#endif
#ifndef SV_CHAIN_NT
#define SV_CHAIN_NT 1              // stream rows with non-temporal loads
#endif

#ifndef SV_CHAIN_T2D_AUX
#define SV_CHAIN_T2D_AUX 0         // the inverse table: temporal loads (shared by every request)
#endif
#ifndef SV_CHAIN_STAGE_U
#define SV_CHAIN_STAGE_U 4         // loads in flight per thread while staging a draft row
#endif

namespace sv {

#ifndef SV_CHAIN_BLOCK
#define SV_CHAIN_BLOCK 256
#endif
constexpr int kChainBlock = SV_CHAIN_BLOCK;
constexpr int kChainWaves = kChainBlock / kWave;
constexpr int64_t kChunk = 1024;   // entries per wave-round; one partial sum each
constexpr int kFallbackChunks = 512;
// dynamic LDS for a staged draft row: the 160 KB of a gfx950 CU less the
// static ChainShared and a margin
constexpr int64_t kMaxStagedBytes = 150 * 1024;

struct ChainShared {
    alignas(16) double chunk[kFallbackChunks];
    uint32_t code;
    int L;
    int32_t xL;   // point-mass drafts: the rejected id (-1 if none or out of range)
    int last;
    int64_t y;
};

template <bool NT>
__device__ __forceinline__ void load4(const float* row, int64_t idx, int64_t V, bool aligned, float (&f)[4]) {
    if (aligned && idx + 3 < V) {
        unpack(load_vec<NT>(row + idx, 0), f);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = (idx + e < V) ? row[idx + e] : 0.0f;
    }
}

template <bool NT>
__device__ __forceinline__ void lane_r4(const float* pr, const float* qr, bool resid, int64_t V, bool aligned,
                                        int64_t idx, double (&r)[4]) {
    float pf[4], qf[4] = {0.f, 0.f, 0.f, 0.f};
    load4<NT>(pr, idx, V, aligned, pf);
    if (resid) load4<NT>(qr, idx, V, aligned, qf);
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = rval(pf[e], qf[e], resid);
}

// Lane's entries of NSUB consecutive sub-tiles (64 lanes x 4) starting at
// base: sub-tile k holds entries base + (k*64 + lane)*4 + e.  Unconditional
// 16-byte loads when the run is aligned and in bounds, masked loads otherwise.
template <int NSUB, bool NT>
__device__ __forceinline__ void load_run(const float* row, int64_t base, int64_t V, bool aligned,
                                         float (&f)[NSUB][4]) {
    const int lane = threadIdx.x & (kWave - 1);
    if (aligned && base + (int64_t)NSUB * kWave * 4 <= V) {
        const float* pp = row + base + lane * 4;
#pragma unroll
        for (int k = 0; k < NSUB; ++k) unpack(load_vec<NT>(pp + k * kWave * 4, 0), f[k]);
    } else {
#pragma unroll
        for (int k = 0; k < NSUB; ++k) load4<NT>(row, base + (k * kWave + lane) * 4, V, aligned, f[k]);
    }
}

// The draft row's entries of a run, laid out as load_run's.  Without t2d
// the row is indexed by target entry; with t2d (a draft row over a smaller
// draft vocabulary of Vd entries) target entry v holds qr[t2d[v]], 0 where
// t2d[v] is outside [0, Vd) or v >= V.  t2d is read with load_run's pattern
// (16-byte loads when aligned), then the draft entries are gathered.
template <int NSUB, bool NT>
__device__ __forceinline__ void load_q_run(const float* qr, const int32_t* t2d, int64_t Vd, int64_t base, int64_t V,
                                           bool aligned, float (&f)[NSUB][4]) {
    if (!t2d) {
        load_run<NSUB, NT>(qr, base, V, aligned, f);
        return;
    }
    const int lane = threadIdx.x & (kWave - 1);
    float tb[NSUB][4];
    load_run<NSUB, false>(reinterpret_cast<const float*>(t2d), base, V, aligned, tb);
#pragma unroll
    for (int k = 0; k < NSUB; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t idx = base + (k * kWave + lane) * 4 + e;
            const int32_t sidx = __float_as_int(tb[k][e]);
            f[k][e] = (idx < V && sidx >= 0 && (int64_t)sidx < Vd) ? qr[sidx] : 0.0f;
        }
}

// Search NSUB sub-tiles (64 lanes x 4 entries each; index order sub-tile,
// lane, entry) starting at `base` for min{ j : run + sum_{<=j} r > T } over
// positive entries.  Wave-uniform result; -1 if not found.  `lastpos`
// receives the last positive entry of the run (wave-uniform); `total`
// receives the run's mass.
template <int NSUB, bool LAZY_LAST = false>
__device__ int64_t wave_search(const float* pr, const float* qr, bool resid, int64_t V, bool aligned,
                               int64_t base, double run, double T, bool force_last, int64_t& lastpos,
                               double& total, int64_t xo = -1, const int32_t* t2d = nullptr, int64_t Vd = 0) {
    const int lane = threadIdx.x & (kWave - 1);
    float pf[NSUB][4], qf[NSUB][4];
    load_run<NSUB, false>(pr, base, V, aligned, pf);
    if (resid) {
        load_q_run<NSUB, false>(qr, t2d, Vd, base, V, aligned, qf);
    } else {
#pragma unroll
        for (int k = 0; k < NSUB; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) qf[k][e] = 0.0f;
    }
    // entry weight; with point-mass drafts the rejected id xo weighs max(0, p - 1)
    auto rv = [&](int k, int e) {
        const double r = rval(pf[k][e], qf[k][e], resid);
        return base + (k * kWave + lane) * 4 + e == xo ? fmax(0.0, (double)pf[k][e] - 1.0) : r;
    };
    auto last_positive = [&]() {
        int64_t mylast = -1;
#pragma unroll
        for (int k = 0; k < NSUB; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (rv(k, e) > 0.0) mylast = base + (k * kWave + lane) * 4 + e;
        return wave_allreduce(mylast, [](int64_t a, int64_t b) { return a > b ? a : b; });
    };
    // LAZY_LAST: the last positive entry is found only when it is the answer
    lastpos = LAZY_LAST ? -1 : last_positive();
    total = 0.0;
    if (force_last) {
        if (LAZY_LAST) lastpos = last_positive();
        return -1;
    }
#pragma unroll
    for (int k = 0; k < NSUB; ++k) {
        double r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = rv(k, e);
        const double s = ((r[0] + r[1]) + r[2]) + r[3];
        const double incl = wave_incl_scan(s);
        const double excl = wave_shift_up1(incl);
        const uint64_t hit = __ballot(run + incl > T && s > 0.0);
        if (hit) {
            const int ls = __ffsll((unsigned long long)hit) - 1;
            int64_t cand = -1;
            if (lane == ls) {
                const int64_t i0 = base + (k * kWave + lane) * 4;
                double xr = run + excl;
                int last_e = -1;
                for (int e = 0; e < 4; ++e) {
                    if (r[e] > 0.0) last_e = e;
                    xr += r[e];
                    if (r[e] > 0.0 && xr > T) {
                        cand = i0 + e;
                        break;
                    }
                }
                if (cand < 0) cand = i0 + last_e;
            }
            return read_lane(cand, ls);
        }
        const double tot = read_lane(incl, kWave - 1);
        run += tot;
        total += tot;
    }
    if (LAZY_LAST) lastpos = last_positive();
    return -1;
}

// One wave picks the chunk holding the draw when the row has at most 256
// chunk sums (in LDS): lane l reads chunks 4l..4l+3 with two 16-byte LDS
// reads and keeps them in registers for its walk.  Same contract as
// wave_pick (index and mass before it; force_last when rounding left
// T = uf * R beyond every positive chunk; -1 when R is not positive), with
// its own fixed association order.
__device__ int pick_chunk256(const double* sums, int n, double uf, double& R, double& base, int& force_last) {
    const int lane = threadIdx.x & (kWave - 1);
    double v[4];
    {
        const double2* s2 = reinterpret_cast<const double2*>(sums) + lane * 2;
        const double2 a = s2[0], c = s2[1];
        v[0] = a.x;
        v[1] = a.y;
        v[2] = c.x;
        v[3] = c.y;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (lane * 4 + k >= n) v[k] = 0.0;
    const double lt = ((v[0] + v[1]) + v[2]) + v[3];
    const double incl = wave_incl_scan(lt);
    const double ex = wave_shift_up1(incl);
    R = read_lane(incl, kWave - 1);
    base = 0.0;
    force_last = 0;
    if (!(R > 0.0)) return -1;
    const double T = uf * R;
    const uint64_t ball = __ballot(incl > T && lt > 0.0);
    int pick = -1, lastp = -1;
    if (ball) {
        const int ls = __ffsll((unsigned long long)ball) - 1;
        double run = ex, b = 0.0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (pick < 0 && v[k] > 0.0) {
                lastp = lane * 4 + k;
                if (run + v[k] > T) {
                    pick = lane * 4 + k;
                    b = run;
                }
            }
            run += v[k];
        }
        const int fl = pick < 0;
        if (fl) pick = lastp;
        pick = read_lane(pick, ls);
        base = read_lane(b, ls);
        force_last = read_lane(fl, ls);
        return pick;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (v[k] > 0.0) lastp = lane * 4 + k;
    force_last = 1;
    return wave_allreduce(lastp, [](int a, int c) { return a > c ? a : c; });
}

// Single-workgroup inverse-CDF draw over a whole row (only for the
// degenerate fallback).  Returns -1 when the row has no positive mass.
__device__ int64_t draw_row_single(const float* pr, int64_t V, double uf, ChainShared& sh) {
    constexpr int64_t kTile = kWave * 4 * 4;   // 4 sub-tiles
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
    const bool aligned = (uintptr_t)pr % 16 == 0;
    const int64_t ntiles = (V + kTile - 1) / kTile;
    const int64_t mult = (ntiles + kFallbackChunks - 1) / kFallbackChunks;
    const int nch = (int)((ntiles + mult - 1) / mult);
    __syncthreads();
    for (int c = wid; c < nch; c += kChainWaves) {
        double acc = 0.0;
        for (int64_t t = 0; t < mult; ++t) {
            const int64_t tb = ((int64_t)c * mult + t) * kTile;
            if (tb >= V) break;
            for (int k = 0; k < 4; ++k) {
                double r[4];
                lane_r4<false>(pr, nullptr, false, V, aligned, tb + (k * kWave + lane) * 4, r);
                acc += ((r[0] + r[1]) + r[2]) + r[3];
            }
        }
        acc = wave_allreduce(acc, OpSumD{});
        if (lane == 0) sh.chunk[c] = acc;
    }
    __syncthreads();
    if (wid == 0) {
        double R, base;
        int force_last;
        const int cstar = wave_pick(nch, [&](int i) { return sh.chunk[i]; }, R, uf, base, force_last);
        int64_t y = -1;
        if (cstar >= 0) {
            const double T = uf * R;
            double run = base;
            int64_t lastpos = -1;
            for (int64_t t = 0; t < mult && y < 0; ++t) {
                const int64_t tb = ((int64_t)cstar * mult + t) * kTile;
                if (tb >= V) break;
                int64_t lp;
                double tot;
                y = wave_search<4>(pr, nullptr, false, V, aligned, tb, run, T, force_last != 0, lp, tot);
                lastpos = max(lastpos, lp);
                run += tot;
            }
            if (y < 0) y = lastpos;
        }
        if (lane == 0) sh.y = y;
    }
    __syncthreads();
    return sh.y;
}

// Cross-workgroup hand-off of chunk sums, built on single-location
// coherence alone (no ordering between different words is assumed, so no
// L2 write-back or invalidate is needed; on gfx950 an agent-scope release
// costs a write-back of the L2).  A chunk sum is never negative, so its sign
// bit is free: each workgroup stores sum | 2^63 with a relaxed 64-bit atomic
// store, then counts itself in with a relaxed add on the request's counter.
// The workgroup whose add returns C - 1 reads every sum, waiting until bit
// 63 shows (a workgroup barrier puts every store of a workgroup before its
// add, so the stores have been issued and the wait ends; the bound only
// keeps a broken invariant from hanging the device), and once it holds a
// sum writes zero back.
constexpr uint64_t kSumWritten = 1ull << 63;

__device__ __forceinline__ void publish_sum(double* p, double v) {
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), (uint64_t)__double_as_longlong(v) | kSumWritten,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ double take_sum(const double* p) {
    uint64_t u = 0;
    for (int spin = 0; spin < (1 << 20); ++spin) {
        u = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (u & kSumWritten) break;
        __builtin_amdgcn_s_sleep(1);
    }
    return __longlong_as_double((long long)(u & ~kSumWritten));
}

__device__ __forceinline__ bool arrive_last(uint32_t* counter, int C) {
    return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(C - 1);
}

// Segment pass for rows that are 16-byte aligned with V a multiple of 4 (and
// V < 2^29, so every offset fits 32 bits).  Every round is a buffer load with
// the workgroup's segment of the row as the range, so chunks past the end of
// the segment (the row's ragged last chunk, rounds that pad R to a multiple
// of DEPTH) read as zeros without a separate tail loop; DEPTH rounds are in
// flight from the first round to the last (consume a slot, refill it).
// Returns, on lane r, the sum of round r's chunk of this wave.
//
// T2D: the draft row lies in LDS (qlds, Vd entries) and the second stream is
// the inverse table t2d (same offsets as the target row; read with temporal
// loads, since every request reads the same table): target entry v weighs
// max(0, p[v] - qlds[t2d[v]]), with q = 0 where t2d[v] is outside [0, Vd).
template <bool RESID, int DEPTH, bool ONEHOT = false, bool T2D = false>
__device__ __forceinline__ double stream_chunks_fast(const float* pr, const float* qr, int64_t V, int64_t chunk0,
                                                     int R, int64_t xo = -1, const int32_t* t2d = nullptr,
                                                     uint32_t Vd = 0, const float* qlds = nullptr) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    constexpr int kAux = SV_CHAIN_NT ? 2 : 0;   // non-temporal
    constexpr int kAuxQ = T2D ? SV_CHAIN_T2D_AUX : kAux;
    const int64_t s0 = chunk0 * kChunk;
    int64_t s1 = (chunk0 + (int64_t)R * kChainWaves) * kChunk;
    s1 = s1 < V ? s1 : V;
    const uint32_t nbytes = (uint32_t)((s1 - s0) * 4);
    const __amdgpu_buffer_rsrc_t rsp = make_rsrc(pr + s0, nbytes);
    const __amdgpu_buffer_rsrc_t rsq =
        T2D ? make_rsrc(t2d + s0, nbytes) : make_rsrc((RESID ? qr : pr) + s0, nbytes);
    const int64_t lane_off = (int64_t)wid * kChunk + lane * 4;   // floats
    const uint32_t vo = (uint32_t)(lane_off * 4);
    u32x4 pv[DEPTH][4], qv[DEPTH][4];
    auto ld = [&](int slot, int r) {
        const uint32_t so = (uint32_t)r * (uint32_t)(kChainWaves * kChunk * 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            pv[slot][k] =
                __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsp, vo + k * kWave * 16, so, kAux));
            if constexpr (RESID)
                qv[slot][k] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsq, vo + k * kWave * 16, so, kAuxQ));
        }
    };
    double mine = 0.0;
    auto sum = [&](const u32x4 (&p4)[4], const u32x4 (&q4)[4], int r) {
        double acc = 0.0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float pf[4], qf[4] = {0.f, 0.f, 0.f, 0.f};
            unpack(p4[k], pf);
            if constexpr (RESID && T2D) {
#pragma unroll
                for (int e = 0; e < 4; ++e) qf[e] = q4[k][e] < Vd ? qlds[q4[k][e]] : 0.0f;
            } else if constexpr (RESID) {
                unpack(q4[k], qf);
            }
            double rr[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) rr[e] = rval(pf[e], qf[e], RESID);
            if constexpr (ONEHOT) {
                // point-mass draft at xo: that entry weighs max(0, p - 1)
                const int64_t d = xo - ((chunk0 + (int64_t)r * kChainWaves) * kChunk + lane_off + k * kWave * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (d == e) rr[e] = fmax(0.0, (double)pf[e] - 1.0);
            }
            double s4 = 0.0;
#pragma unroll
            for (int e = 0; e < 4; ++e) s4 += rr[e];
            acc += s4;
        }
        acc = wave_allreduce(acc, OpSumD{});
        if (lane == r) mine = acc;
    };
    // rounds [R, Rp) are past the segment and read zeros; their sums land on
    // lanes that are never published (R <= 64)
    const int Rp = (R + DEPTH - 1) / DEPTH * DEPTH;
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) ld(j, j);
    int r0 = 0;
    for (; r0 + DEPTH < Rp; r0 += DEPTH) {
#pragma unroll
        for (int j = 0; j < DEPTH; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            sum(pv[j], qv[j], r0 + j);
            __builtin_amdgcn_sched_barrier(0);
            ld(j, r0 + j + DEPTH);
        }
    }
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) sum(pv[j], qv[j], r0 + j);
    return mine;
}

// Copy n floats from global memory to LDS, U loads in flight per thread:
// 16-byte loads when the source is 16-byte aligned and n a multiple of 4.
template <int U>
__device__ __forceinline__ void stage_row(const float* __restrict__ src, int64_t n, float* dst) {
    const int tid = threadIdx.x;
    if ((uintptr_t)src % 16 == 0 && (n & 3) == 0) {
        const int64_t n4 = n / 4;
        const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
        u32x4* d4 = reinterpret_cast<u32x4*>(dst);
        for (int64_t i0 = 0; i0 < n4; i0 += (int64_t)U * kChainBlock) {
            u32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = i0 + u * kChainBlock + tid;
                v[u] = i < n4 ? s4[i] : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = i0 + u * kChainBlock + tid;
                if (i < n4) d4[i] = v[u];
            }
        }
    } else {
        for (int64_t i0 = 0; i0 < n; i0 += (int64_t)U * kChainBlock) {
            float v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = i0 + u * kChainBlock + tid;
                v[u] = i < n ? src[i] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = i0 + u * kChainBlock + tid;
                if (i < n) dst[i] = v[u];
            }
        }
    }
}

// Draft mode: kNoDraft (D = 0), kDraftProbs (draft distributions given) or
// kPointDraft (no draft distributions: each draft is a point mass at its id,
// so q(x) = 1 and the residual is p with the rejected id weighing max(0, p - 1)).
// kStaged: a separate instantiation for draft rows over a draft vocabulary
// that fits LDS, so the other kernels' code is untouched by it.
constexpr int kNoDraft = 0, kDraftProbs = 1, kPointDraft = 2;
template <int kMode, bool kStaged = false>
__global__ __launch_bounds__(kChainBlock) void chain_reject_kernel(
    const float* __restrict__ q, const int32_t* __restrict__ x, const float* __restrict__ p,
    const uint64_t* __restrict__ seed, const uint64_t* __restrict__ offset, int64_t B, int D, int64_t V,
    const int32_t* __restrict__ qo_indptr, int64_t n_rows, const int32_t* __restrict__ t2d, int64_t Vd,
    const int32_t* __restrict__ req_index, int64_t n_req, int C, int R, int64_t per_xcd,
    int32_t* __restrict__ accepted, int32_t* __restrict__ accept_len, double* partial,
    uint32_t* __restrict__ counter, int64_t qcap) {
    __shared__ ChainShared sh;
    // a draft row over the draft vocabulary, staged when it fits (qcap entries
    // of dynamic LDS; 0 when the launch has none)
    extern __shared__ __attribute__((aligned(16))) float qlds[];
    // XCD-aware mapping: workgroups are dispatched round-robin over the 8 XCDs,
    // so consecutive virtual ids (one request's segments) share an XCD's L2.
    const int64_t vid = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (vid >= n_req * C) return;
    const int64_t slot = vid / C;
    const int c = (int)(vid - slot * C);
    const int64_t b = req_index ? (int64_t)req_index[slot] : slot;
    if (b < 0 || b >= B) return;   // every workgroup of this slot leaves: its counter is untouched
    const int N = D + 1;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;

    // Target rows of request b start at row `base`; it verifies d <= D drafts.
    // Ragged batches (qo_indptr given) pack each request's d + 1 rows; the
    // positions past d are one-hot at token 0 for target and draft alike and
    // so are never read: position d drafts token 0 as a point mass, every
    // later position accepts, and the emitted count is clamped to d + 1.
    int64_t base = b * N;
    int d = D;
    if (qo_indptr) {
        const int64_t lo = qo_indptr[b], n = (int64_t)qo_indptr[b + 1] - lo;
        if (!(n >= 1 && n <= N && lo >= 0 && lo + n <= n_rows)) {
            // invalid length or rows outside the packed array: marked, nothing read
            if (c == 0) {
                if (tid < N) accepted[b * N + tid] = -1;
                if (tid == 0) accept_len[b] = -1;
            }
            return;
        }
        base = lo;
        d = (int)(n - 1);
    }

    // ---- 1. probe (wave 0): lane i < D tests position i, lane D draws u_f.
    // The loads at the draft ids are issued before the Philox rounds, so the
    // rounds overlap their round trip; the first reject comes from a ballot.
    // Lane i keeps draft id i for the output (written by the same lanes).
    int32_t xkeep = 0;
    if (tid <= D) {
        uint32_t w;
        bool ok = false;
        if constexpr (kMode != kNoDraft) {
            // lanes 0 and 1 (both active: D >= 1) fetch seed and offset with
            // the id loads; lane D repeats lane D-1's loads (in bounds), so no
            // lane branches and the Philox rounds overlap the draft-probability
            // round trip
            const uint64_t so = ((tid & 1) ? offset : seed)[b];
            const int ic = tid < D ? tid : D - 1;
            // positions from d on draft token 0 as a point mass; only row d is read
            const int32_t xi = ic < d ? x[b * D + ic] : 0;
            xkeep = xi;
            const bool inr = tid < D && xi >= 0 && (int64_t)xi < V;
            const int64_t xc = inr ? (int64_t)xi : 0;
            const float a = p[(base + (ic < d ? ic : d)) * V + xc];
            float cq = 1.0f;
            if (kMode == kDraftProbs && ic < d) {
                if (t2d) {
                    // draft row over the draft vocabulary: the id's entry through t2d
                    const int32_t sx = inr ? t2d[xc] : -1;
                    cq = (sx >= 0 && (int64_t)sx < Vd) ? q[(b * D + ic) * Vd + sx] : 0.0f;
                } else {
                    cq = q[(b * D + ic) * V + xc];
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            w = philox_word(read_lane(so, 0), read_lane(so, 1), (uint64_t)tid);
            ok = (inr && (double)uniform_of(w) * (double)cq < (double)a) || (tid > d && tid < D);
            if constexpr (kMode == kPointDraft) {
                // the rejected id, read from its lane (lanes 0..D are all active here)
                const int32_t xsel = inr ? xi : -1;
                const uint64_t rj = __ballot(tid < D && !ok);
                const int Lr = rj ? __ffsll((unsigned long long)rj) - 1 : D;
                const int32_t xr = Lr < D ? read_lane(xsel, Lr) : -1;
                if (tid == 0) sh.xL = xr;
            }
        } else {
            w = philox_word(seed[b], offset[b], (uint64_t)tid);
        }
        if (tid == D) sh.code = uniform_code(w);
        const uint64_t rej = __ballot(tid < D && !ok);
        if (tid == 0) sh.L = rej ? __ffsll((unsigned long long)rej) - 1 : D;
    }
    __syncthreads();
    const int L = sh.L;
    if (L > d) {
        // a ragged request accepted token 0 at its own last position: its
        // emitted tokens are the d drafts and 0, with no row to stream
        if (c == 0) {
            if (tid < N) accepted[b * N + tid] = tid < d ? xkeep : (tid == d ? 0 : -1);
            if (tid == 0) accept_len[b] = d;
        }
        return;
    }
    // a residual row with draft probabilities streams q_L; with point-mass
    // drafts (and at a ragged request's own last position, token 0) it streams
    // p_L alone, the rejected id xo weighing max(0, p - 1)
    const bool resid = kMode == kDraftProbs && L < d;
    const bool point = (kMode == kPointDraft && L < d) || (L == d && d < D);
    const int64_t xo = point ? (L < d ? (int64_t)sh.xL : 0) : -1;
    const float* pr = p + (base + L) * V;
    // draft rows hold V entries, or Vd (read through t2d) for a smaller draft vocabulary
    const float* qr = resid ? q + (b * D + L) * (t2d ? Vd : V) : nullptr;
    const bool aligned = ((uintptr_t)pr % 16 == 0) &&
                         (!resid || (t2d ? (uintptr_t)t2d % 16 == 0 : (uintptr_t)qr % 16 == 0));
    const int64_t nchunks = (V + kChunk - 1) / kChunk;

    // ---- 2. segment pass.  Wave w owns chunks chunk0 + 4r + w, r < R (1024
    // entries each); two rounds of loads are in flight at any time.  Lane r
    // keeps round r's chunk sum.
    const int64_t chunk0 = (int64_t)c * R * kChainWaves;
    double mine = 0.0;
    const bool fast = aligned && (V & 3) == 0 && V < ((int64_t)1 << 29);
    const bool staged = kStaged && fast && resid && t2d && Vd <= qcap;
    if (staged) {
        // the draft row (read once) goes to LDS
        stage_row<SV_CHAIN_STAGE_U>(qr, Vd, qlds);
        __syncthreads();
    }
    if (staged) {
        mine = stream_chunks_fast<true, SV_CHAIN_DEPTH, false, true>(pr, nullptr, V, chunk0, R, -1, t2d,
                                                                      (uint32_t)Vd, qlds);
    } else if (fast && !(resid && t2d)) {
        // With draft distributions a batch mixes two-row (residual) and
        // one-row (bonus) requests, and the two-row ones set the kernel's end:
        // a one-row workgroup keeps fewer loads in flight, so it takes a
        // smaller share of HBM while both kinds stream and finishes closer to
        // the two-row ones (measured on the large-vocab batch: 36.3 -> 35.5 us
        // together with the pick and the lazy last-positive search).  Without
        // draft distributions every request streams one row: two rounds in
        // flight measured best there (24.7 us against 25.3 with three).
        constexpr int kOneRowDepth = kMode == kDraftProbs ? SV_CHAIN_DEPTH_ONE_ROW : SV_CHAIN_DEPTH_ALL_ONE_ROW;
        if (resid) mine = stream_chunks_fast<true, SV_CHAIN_DEPTH>(pr, qr, V, chunk0, R);
        else if (point) mine = stream_chunks_fast<false, kOneRowDepth, true>(pr, qr, V, chunk0, R, xo);
        else mine = stream_chunks_fast<false, kOneRowDepth>(pr, qr, V, chunk0, R);
    } else {
        float pa[4][4], qa[4][4], pb[4][4], qb[4][4];
        auto load_chunk = [&](int r, float (&pf)[4][4], float (&qf)[4][4]) {
            const int64_t ch = chunk0 + (int64_t)r * kChainWaves + wid;
            if (ch < nchunks) {
                load_run<4, SV_CHAIN_NT != 0>(pr, ch * kChunk, V, aligned, pf);
                if (resid) load_q_run<4, SV_CHAIN_NT != 0>(qr, t2d, Vd, ch * kChunk, V, aligned, qf);
            }
        };
        auto sum_chunk = [&](int r, const float (&pf)[4][4], const float (&qf)[4][4]) {
            const int64_t ch = chunk0 + (int64_t)r * kChainWaves + wid;
            double acc = 0.0;
            if (ch < nchunks) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    double s4 = 0.0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        double r = rval(pf[k][e], resid ? qf[k][e] : 0.0f, resid);
                        if (ch * kChunk + (k * kWave + lane) * 4 + e == xo) r = fmax(0.0, (double)pf[k][e] - 1.0);
                        s4 += r;
                    }
                    acc += s4;
                }
            }
            acc = wave_allreduce(acc, OpSumD{});
            if (lane == r) mine = acc;
        };
        load_chunk(0, pa, qa);
        for (int r = 0; r < R; r += 2) {
            if (r + 1 < R) load_chunk(r + 1, pb, qb);
            sum_chunk(r, pa, qa);
            if (r + 2 < R) load_chunk(r + 2, pa, qa);
            if (r + 1 < R) sum_chunk(r + 1, pb, qb);
        }
    }
    // One workgroup for the whole row: its chunk sums go straight to LDS.
    // Otherwise they are published and the request's last workgroup locates.
    const bool sums_in_lds = nchunks <= kFallbackChunks;
    const bool solo = C == 1 && sums_in_lds;
    {
        const int64_t ch = chunk0 + (int64_t)lane * kChainWaves + wid;
        if (lane < R && ch < nchunks) {
            if (solo) sh.chunk[ch] = mine;
            else publish_sum(&partial[slot * nchunks + ch], mine);
        }
    }
    __syncthreads();
    if (!solo) {
        if (tid == 0) sh.last = arrive_last(&counter[slot], C) ? 1 : 0;
        __syncthreads();
        if (!sh.last) return;
    }

    // ---- 3. locate (the request's last workgroup).  Published chunk sums are
    // first copied to LDS by every thread at once (one round trip), then wave
    // 0 picks the chunk and searches it.
    const double uf = (double)sh.code * 0x1p-24;
    const double* part = partial + slot * nchunks;
    if (sums_in_lds && !solo) {
        constexpr int kPer = (kFallbackChunks + kChainBlock - 1) / kChainBlock;
        double v[kPer];
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int64_t i = tid + (int64_t)k * kChainBlock;
            v[k] = i < nchunks ? take_sum(&part[i]) : 0.0;
        }
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int64_t i = tid + (int64_t)k * kChainBlock;
            if (i < nchunks) sh.chunk[i] = v[k];
        }
        __syncthreads();
    }
    if (wid == 0) {
        double R_tot, base;
        int force_last;
        const int cstar =
            nchunks <= 256 ? pick_chunk256(sh.chunk, (int)nchunks, uf, R_tot, base, force_last)
            : sums_in_lds  ? wave_pick((int)nchunks, [&](int i) { return sh.chunk[i]; }, R_tot, uf, base, force_last)
                           : wave_pick((int)nchunks, [&](int i) { return take_sum(&part[i]); }, R_tot, uf, base,
                                       force_last);
        int64_t y = -1;
        if (cstar >= 0) {
            int64_t lastpos;
            double tot;
            y = wave_search<4, true>(pr, qr, resid, V, aligned, (int64_t)cstar * kChunk, base, uf * R_tot,
                                     force_last != 0, lastpos, tot, xo, t2d, Vd);
            if (y < 0) y = lastpos;
        }
        if (lane == 0) sh.y = y;
    }
    __syncthreads();
    if (!solo) {
        // every workspace byte this call used goes back to zero (its counter
        // below), so the workspace can serve any later call whatever its
        // layout; each sum is held (its written bit seen) before it is
        // cleared, and the next kernel boundary orders these stores
        double* mine_part = partial + slot * nchunks;
        for (int64_t i = tid; i < nchunks; i += kChainBlock) {
            take_sum(&mine_part[i]);
            __hip_atomic_store(reinterpret_cast<uint64_t*>(&mine_part[i]), (uint64_t)0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    int64_t y = sh.y;
    if (y < 0 && (resid || point)) y = draw_row_single(pr, V, uf, sh);
    if (y < 0) y = (int64_t)(((uint64_t)sh.code * (uint64_t)V) >> 24);
    if (tid < N) {
        int32_t t;
        if (tid < L) t = xkeep;
        else t = (tid == L) ? (int32_t)y : -1;
        accepted[b * N + tid] = t;
    }
    if (tid == 0) {
        accept_len[b] = L;
        // ready for the next call on this workspace (the kernel boundary orders it)
        if (!solo) __hip_atomic_store(&counter[slot], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

int64_t chain_partials_per_request(int64_t V) { return (V + kChunk - 1) / kChunk; }

// Segments per request: enough workgroups to keep ~SV_CHAIN_TARGET_WGS
// resident, at most 64 rounds of 4096 entries per workgroup.
static void chain_split(int64_t n_req, int64_t V, int& C, int& R) {
    const int64_t nchunks = chain_partials_per_request(V);
    const int64_t max_c = (nchunks + kChainWaves - 1) / kChainWaves;
    int64_t c = (SV_CHAIN_TARGET_WGS + n_req - 1) / n_req;
    c = c < 1 ? 1 : (c > max_c ? max_c : c);
    int64_t r = (nchunks + kChainWaves * c - 1) / (kChainWaves * c);
    if (r > 64) r = 64;
    c = (nchunks + kChainWaves * r - 1) / (kChainWaves * r);
    C = (int)c;
    R = (int)r;
}

// Workspace layout: n_req 32-bit counters (padded to 256 bytes), then
// n_req * chain_partials_per_request(V) doubles.  Needed only when a
// request's row is split over several workgroups or its chunk sums exceed
// the LDS table.  Every call returns the bytes it used to zero.
static int64_t chain_counter_bytes(int64_t n_req) { return (n_req * 4 + 255) / 256 * 256; }

int64_t chain_workspace_bytes(int64_t n_req, int64_t V) {
    if (n_req <= 0) return 0;
    int C, R;
    chain_split(n_req, V, C, R);
    const int64_t nchunks = chain_partials_per_request(V);
    if (C == 1 && nchunks <= kFallbackChunks) return 0;
    return chain_counter_bytes(n_req) + n_req * nchunks * 8;
}

// ---------------------------------------------------------------------------
// Static scratch for callers that cannot allocate (specverify_chain_reject_noalloc):
// a file-scope device array with the layout of the caller workspace.  Each
// device holds its own copy at its own address, so host code never passes
// the array's name to a kernel: the address comes from hipGetSymbolAddress,
// once per device, and is kept.  The first call on a device also clears the
// array with a fill kernel on that call's stream; every later call finds the
// bytes it needs at zero because every call returns what it used to zero.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kChainStaticScratchBytes];

__global__ __launch_bounds__(256) void scratch_clear_kernel(u32x4* __restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = u32x4{0u, 0u, 0u, 0u};
}

namespace {
constexpr int kScratchDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};
}  // namespace

hipError_t chain_static_scratch(hipStream_t stream, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        constexpr int64_t n = kChainStaticScratchBytes / 16;
        hipLaunchKernelGGL(scratch_clear_kernel, dim3(256), dim3(256), 0, stream, static_cast<u32x4*>(ptr), n);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_chain_reject(const float* draft_probs, const int32_t* draft_ids, const float* target_probs,
                               const int32_t* qo_indptr, int64_t n_rows, const int32_t* t2d, int64_t Vd,
                               const uint64_t* seed,
                               const uint64_t* offset, int64_t B, int D, int64_t V, const int32_t* req_index,
                               int64_t n_req, int32_t* accepted, int32_t* accept_len, void* workspace,
                               hipStream_t stream) {
    int C, R;
    chain_split(n_req, V, C, R);
    uint32_t* counter = nullptr;
    double* partial = nullptr;
    if (chain_workspace_bytes(n_req, V) > 0) {
        if (!workspace) return hipErrorInvalidValue;
        counter = static_cast<uint32_t*>(workspace);
        partial = reinterpret_cast<double*>(static_cast<char*>(workspace) + chain_counter_bytes(n_req));
    }
    const int64_t total = n_req * C;
    const int64_t per_xcd = (total + 7) / 8;
    const int64_t grid = per_xcd * 8;
    if (grid > 2147483647LL) return hipErrorInvalidValue;
    auto* kernel = D == 0 ? chain_reject_kernel<kNoDraft>
                          : (draft_probs ? chain_reject_kernel<kDraftProbs> : chain_reject_kernel<kPointDraft>);
    // a draft row over a draft vocabulary small enough for LDS is staged there,
    // when each workgroup's segment spans at least Vd target entries (every
    // workgroup of a split row would stage the whole draft row)
    size_t lds = 0;
    if (D > 0 && draft_probs && t2d && Vd >= 1 && Vd * 4 <= kMaxStagedBytes &&
        (int64_t)R * kChainWaves * kChunk >= Vd) {
        kernel = chain_reject_kernel<kDraftProbs, true>;
        lds = (size_t)((Vd * 4 + 15) / 16 * 16);
        const hipError_t e =
            hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    const int64_t qcap = (int64_t)(lds / 4);
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kChainBlock), lds, stream, draft_probs, draft_ids,
                       target_probs, seed, offset, B, D, V, qo_indptr, n_rows, t2d, Vd, req_index, n_req, C, R,
                       per_xcd, accepted, accept_len, partial, counter, qcap);
    return hipGetLastError();
}

}  // namespace sv
