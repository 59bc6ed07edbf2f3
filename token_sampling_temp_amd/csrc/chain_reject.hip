// Chain rejection sampling of a linear draft.
//
// Work split: each request's row is cut into C segments and every (request,
// segment) pair is one 256-thread workgroup; C is chosen so the grid holds
// about five resident workgroups per CU, so a batch fills the chip whatever
// its accept pattern.
//
// 1. Probe (every workgroup of a request, redundantly; the lines are shared
//    in L2): thread i < D loads p_i(x_i), q_i(x_i) and the Philox uniform u_i
//    and decides u_i * q < p exactly in double; thread D takes the final
//    uniform.  L = first rejected position (D if none).
// 2. Segment pass: r_v = max(0, p_L[v] - q_L[v]) (or p_D[v] for the bonus) is
//    summed in double per 1024-entry chunk; waves stream their chunks with two
//    rounds of 16-byte loads in flight, and publish one sum per chunk.
// 3. The last workgroup of the request to finish (device-scope atomic counter,
//    reset afterwards; no cache-flushing fences) prefix-sums the chunk sums in
//    order, finds the chunk holding u_f * R, re-reads it and finishes with a
//    64-lane scan.  Zero-mass entries are never selected.  Sums use fixed
//    reduction trees, so results are reproducible run to run.
// 4. Degenerate rows (residual mass not positive) fall back to a draw from the
//    target row by the same workgroup, then to floor(u_f * V).
#include "sv_common.hpp"
#include "sv_launch.hpp"

#ifndef SV_CHAIN_TARGET_WGS
#define SV_CHAIN_TARGET_WGS 1024   // ~4 resident 256-thread workgroups per CU on 256 CUs
#endif
#ifndef SV_CHAIN_NT
#define SV_CHAIN_NT 1              // stream rows with non-temporal loads
#endif

namespace sv {

constexpr int kChainBlock = 256;
constexpr int kChainWaves = kChainBlock / kWave;
constexpr int64_t kChunk = 1024;   // entries per wave-round; one partial sum each
constexpr int kFallbackChunks = 512;

struct ChainShared {
    double chunk[kFallbackChunks];
    int acc[kMaxDraft];
    uint32_t code;
    int L;
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

__device__ __forceinline__ double rval(float pv, float qv, bool resid) {
    return resid ? fmax(0.0, (double)pv - (double)qv) : (double)pv;
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

// Inclusive 64-lane scan (Hillis-Steele, fixed association order).
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const T u = __shfl_up(v, off, kWave);
        if (lane >= off) v += u;
    }
    return v;
}

// Search NSUB sub-tiles (64 lanes x 4 entries each; index order sub-tile,
// lane, entry) starting at `base` for min{ j : run + sum_{<=j} r > T } over
// positive entries.  Wave-uniform result; -1 if not found.  `lastpos`
// receives the last positive entry of the run (wave-uniform); `total`
// receives the run's mass.
template <int NSUB>
__device__ int64_t wave_search(const float* pr, const float* qr, bool resid, int64_t V, bool aligned,
                               int64_t base, double run, double T, bool force_last, int64_t& lastpos,
                               double& total) {
    const int lane = threadIdx.x & (kWave - 1);
    float pf[NSUB][4], qf[NSUB][4];
    load_run<NSUB, false>(pr, base, V, aligned, pf);
    if (resid) {
        load_run<NSUB, false>(qr, base, V, aligned, qf);
    } else {
#pragma unroll
        for (int k = 0; k < NSUB; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) qf[k][e] = 0.0f;
    }
    int64_t mylast = -1;
#pragma unroll
    for (int k = 0; k < NSUB; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (rval(pf[k][e], qf[k][e], resid) > 0.0) mylast = base + (k * kWave + lane) * 4 + e;
    lastpos = wave_reduce(mylast, [](int64_t a, int64_t b) { return a > b ? a : b; });
    total = 0.0;
    if (force_last) return -1;
#pragma unroll
    for (int k = 0; k < NSUB; ++k) {
        double r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = rval(pf[k][e], qf[k][e], resid);
        const double s = ((r[0] + r[1]) + r[2]) + r[3];
        const double incl = wave_incl_scan(s);
        double excl = __shfl_up(incl, 1, kWave);
        if (lane == 0) excl = 0.0;
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
            return __shfl(cand, ls, kWave);
        }
        const double tot = __shfl(incl, kWave - 1, kWave);
        run += tot;
        total += tot;
    }
    return -1;
}

// Wave 0 of the block: given 'n' ordered non-negative masses m[0..n) (read
// through `get`), total R and target T = uf * R, find the first index whose
// running mass exceeds T (only positive entries qualify).  Returns the index
// and the mass before it; force_last is set when rounding left T beyond every
// positive entry (then the index is the last positive one).
template <typename Get>
__device__ int wave_pick(int n, Get get, double& R, double uf, double& base, int& force_last) {
    const int lane = threadIdx.x & (kWave - 1);
    const int g = (n + kWave - 1) / kWave;
    const int i0 = min(n, lane * g), i1 = min(n, i0 + g);
    double lt = 0.0;
    for (int i = i0; i < i1; ++i) lt += get(i);
    const double incl = wave_incl_scan(lt);
    R = __shfl(incl, kWave - 1, kWave);
    base = 0.0;
    force_last = 0;
    if (!(R > 0.0)) return -1;
    const double T = uf * R;
    const uint64_t ball = __ballot(incl > T && lt > 0.0);
    int pick = -1;
    if (ball) {
        const int ls = __ffsll((unsigned long long)ball) - 1;
        double ex = __shfl_up(incl, 1, kWave);
        if (lane == 0) ex = 0.0;
        if (lane == ls) {
            double run = ex;
            int lastp = -1;
            for (int i = i0; i < i1; ++i) {
                const double si = get(i);
                if (si > 0.0) {
                    lastp = i;
                    if (run + si > T) {
                        pick = i;
                        base = run;
                        break;
                    }
                }
                run += si;
            }
            if (pick < 0) {
                pick = lastp;
                force_last = 1;
            }
        }
        pick = __shfl(pick, ls, kWave);
        base = __shfl(base, ls, kWave);
        force_last = __shfl(force_last, ls, kWave);
    } else {
        int lp = -1;
        for (int i = i0; i < i1; ++i)
            if (get(i) > 0.0) lp = i;
        pick = wave_reduce(lp, [](int a, int b) { return a > b ? a : b; });
        force_last = 1;
    }
    return pick;
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
        acc = wave_reduce(acc, OpSumD{});
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

// Cross-workgroup hand-off without cache-maintenance fences: partial sums are
// published and read back with device-scope atomic read-modify-writes, which
// are performed at the memory-side coherence point.  The publishing lane
// consumes the RMW's return value before the workgroup barrier, so the value
// is globally performed before thread 0 increments the request's counter.
__device__ __forceinline__ void publish_partial(double* dst, double v) {
    const unsigned long long old = __hip_atomic_exchange(reinterpret_cast<unsigned long long*>(dst),
                                                         (unsigned long long)__double_as_longlong(v),
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" ::"v"(old));   // wait for the exchange to complete
}
__device__ __forceinline__ double read_partial(double* src) {
    const unsigned long long v = __hip_atomic_fetch_or(reinterpret_cast<unsigned long long*>(src), 0ull,
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return __longlong_as_double((long long)v);
}

// Segment pass for a workgroup whose chunks are all in bounds and 16-byte
// aligned: straight-line unconditional loads so that the next round's loads
// stay in flight while the current round is summed.  Returns, on lane r, the
// sum of round r's chunk of this wave.
template <bool RESID>
__device__ __forceinline__ double stream_chunks_fast(const float* pr, const float* qr, int64_t chunk0, int R) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    constexpr int64_t kStride = (int64_t)kChainWaves * kChunk;   // between a wave's consecutive chunks
    const float* pb0 = pr + (chunk0 + wid) * kChunk + lane * 4;
    const float* qb0 = RESID ? qr + (chunk0 + wid) * kChunk + lane * 4 : nullptr;
    u32x4 pa[4], qa[4], pbf[4], qbf[4];
    auto ld = [&](int r, u32x4 (&pv)[4], u32x4 (&qv)[4]) {
        const float* pp = pb0 + (int64_t)r * kStride;
#pragma unroll
        for (int k = 0; k < 4; ++k) pv[k] = load_vec<SV_CHAIN_NT != 0>(pp + k * kWave * 4, 0);
        if constexpr (RESID) {
            const float* qq = qb0 + (int64_t)r * kStride;
#pragma unroll
            for (int k = 0; k < 4; ++k) qv[k] = load_vec<SV_CHAIN_NT != 0>(qq + k * kWave * 4, 0);
        }
    };
    double mine = 0.0;
    auto sum = [&](int r, const u32x4 (&pv)[4], const u32x4 (&qv)[4]) {
        double acc = 0.0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float pf[4], qf[4] = {0.f, 0.f, 0.f, 0.f};
            unpack(pv[k], pf);
            if constexpr (RESID) unpack(qv[k], qf);
            double s4 = 0.0;
#pragma unroll
            for (int e = 0; e < 4; ++e) s4 += rval(pf[e], qf[e], RESID);
            acc += s4;
        }
        acc = wave_reduce(acc, OpSumD{});
        if (lane == r) mine = acc;
    };
    ld(0, pa, qa);
    int r = 0;
    for (; r + 1 < R; r += 2) {
        ld(r + 1, pbf, qbf);
        sum(r, pa, qa);
        if (r + 2 < R) ld(r + 2, pa, qa);
        sum(r + 1, pbf, qbf);
    }
    if (r < R) sum(r, pa, qa);
    return mine;
}

__global__ __launch_bounds__(kChainBlock) void chain_reject_kernel(
    const float* __restrict__ q, const int32_t* __restrict__ x, const float* __restrict__ p,
    const uint64_t* __restrict__ seed, const uint64_t* __restrict__ offset, int64_t B, int D, int64_t V,
    const int32_t* __restrict__ req_index, int64_t n_req, int C, int R, int64_t per_xcd,
    int32_t* __restrict__ accepted, int32_t* __restrict__ accept_len, double* __restrict__ partial,
    uint32_t* __restrict__ counter) {
    __shared__ ChainShared sh;
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

    // ---- 1. probe
    if (tid <= D) {
        const uint32_t w = philox_word(seed[b], offset[b], (uint64_t)tid);
        if (tid < D) {
            const int32_t xi = x[b * D + tid];
            bool ok = false;
            if (xi >= 0 && (int64_t)xi < V) {
                const float a = p[(b * N + tid) * V + xi];
                const float cq = q[(b * D + tid) * V + xi];
                ok = (double)uniform_of(w) * (double)cq < (double)a;
            }
            sh.acc[tid] = ok ? 1 : 0;
        } else {
            sh.code = uniform_code(w);
        }
    }
    __syncthreads();
    if (tid == 0) {
        int L = D;
        for (int i = 0; i < D; ++i)
            if (!sh.acc[i]) {
                L = i;
                break;
            }
        sh.L = L;
    }
    __syncthreads();
    const int L = sh.L;
    const bool resid = L < D;
    const float* pr = p + (b * N + L) * V;
    const float* qr = resid ? q + (b * D + L) * V : nullptr;
    const bool aligned = ((uintptr_t)pr % 16 == 0) && (!resid || (uintptr_t)qr % 16 == 0);
    const int64_t nchunks = (V + kChunk - 1) / kChunk;

    // ---- 2. segment pass.  Wave w owns chunks chunk0 + 4r + w, r < R (1024
    // entries each); two rounds of loads are in flight at any time.  Lane r
    // keeps round r's chunk sum.
    const int64_t chunk0 = (int64_t)c * R * kChainWaves;
    double mine = 0.0;
    if (aligned && (chunk0 + (int64_t)R * kChainWaves) * kChunk <= V) {
        if (resid) mine = stream_chunks_fast<true>(pr, qr, chunk0, R);
        else mine = stream_chunks_fast<false>(pr, qr, chunk0, R);
    } else {
        float pa[4][4], qa[4][4], pb[4][4], qb[4][4];
        auto load_chunk = [&](int r, float (&pf)[4][4], float (&qf)[4][4]) {
            const int64_t ch = chunk0 + (int64_t)r * kChainWaves + wid;
            if (ch < nchunks) {
                load_run<4, SV_CHAIN_NT != 0>(pr, ch * kChunk, V, aligned, pf);
                if (resid) load_run<4, SV_CHAIN_NT != 0>(qr, ch * kChunk, V, aligned, qf);
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
                    for (int e = 0; e < 4; ++e) s4 += rval(pf[k][e], resid ? qf[k][e] : 0.0f, resid);
                    acc += s4;
                }
            }
            acc = wave_reduce(acc, OpSumD{});
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
    {
        const int64_t ch = chunk0 + (int64_t)lane * kChainWaves + wid;
        if (lane < R && ch < nchunks) publish_partial(&partial[slot * nchunks + ch], mine);
    }
    __syncthreads();
    if (tid == 0)
        sh.last = (__hip_atomic_fetch_add(&counter[slot], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   (uint32_t)(C - 1)) ? 1 : 0;
    __syncthreads();
    if (!sh.last) return;

    // ---- 3. locate (the request's last workgroup; wave 0)
    const double uf = (double)sh.code * 0x1p-24;
    if (wid == 0) {
        double* part = partial + slot * nchunks;
        double R_tot, base;
        int force_last;
        const int cstar = wave_pick((int)nchunks, [&](int i) { return read_partial(&part[i]); }, R_tot, uf,
                                    base, force_last);
        int64_t y = -1;
        if (cstar >= 0) {
            int64_t lastpos;
            double tot;
            y = wave_search<4>(pr, qr, resid, V, aligned, (int64_t)cstar * kChunk, base, uf * R_tot,
                               force_last != 0, lastpos, tot);
            if (y < 0) y = lastpos;
        }
        if (lane == 0) sh.y = y;
    }
    __syncthreads();
    int64_t y = sh.y;
    if (y < 0 && resid) y = draw_row_single(pr, V, uf, sh);
    if (y < 0) y = (int64_t)(((uint64_t)sh.code * (uint64_t)V) >> 24);
    if (tid < N) {
        int32_t t;
        if (tid < L) t = x[b * D + tid];
        else t = (tid == L) ? (int32_t)y : -1;
        accepted[b * N + tid] = t;
    }
    if (tid == 0) {
        accept_len[b] = L;
        // ready for the next call on this workspace (kernel boundary orders it)
        __hip_atomic_store(&counter[slot], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

hipError_t launch_chain_reject(const float* draft_probs, const int32_t* draft_ids, const float* target_probs,
                               const uint64_t* seed, const uint64_t* offset, int64_t B, int D, int64_t V,
                               const int32_t* req_index, int64_t n_req, int32_t* accepted, int32_t* accept_len,
                               uint32_t* counter, double* partial, hipStream_t stream) {
    int C, R;
    chain_split(n_req, V, C, R);
    const int64_t total = n_req * C;
    const int64_t per_xcd = (total + 7) / 8;
    const int64_t grid = per_xcd * 8;
    if (grid > 2147483647LL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(chain_reject_kernel, dim3((unsigned)grid), dim3(kChainBlock), 0, stream, draft_probs,
                       draft_ids, target_probs, seed, offset, B, D, V, req_index, n_req, C, R, per_xcd, accepted,
                       accept_len, partial, counter);
    return hipGetLastError();
}

}  // namespace sv
