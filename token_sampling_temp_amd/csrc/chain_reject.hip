// Chain rejection sampling of a linear draft (one workgroup per request).
//
// 1. Probe: thread i < D loads p_i(x_i), q_i(x_i) and its Philox uniform u_i
//    and decides u_i * q < p exactly in double; thread D takes the final
//    uniform.  L = first rejected position (D if none).
// 2. Row pass: r_v = max(0, p_L[v] - q_L[v]) (or p_D[v] for the bonus) is
//    summed in double per 1024-element tile ("chunk"); chunk sums go to LDS.
// 3. Locate: wave 0 prefix-sums the chunk sums (fixed order), finds the chunk
//    holding u_f * R, re-reads that one tile and finds the token by a lane
//    scan.  Zero-mass entries are never selected.
#include "sv_common.hpp"
#include "sv_launch.hpp"

namespace sv {

constexpr int kChainBlock = 1024;
constexpr int kTile = 1024;        // 4 sub-tiles x 64 lanes x 4 floats
constexpr int kMaxChunks = 4096;   // LDS chunk-sum slots; chunks grow for huge V

struct ChainShared {
    double chunk[kMaxChunks];
    double red_d[kChainBlock / kWave];
    int acc[kMaxDraft];
    uint32_t code;
    int L;
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

// Lane's four r values of sub-tile k of tile starting at tb.
template <bool NT>
__device__ __forceinline__ void lane_r4(const float* pr, const float* qr, bool resid, int64_t V, bool aligned,
                                        int64_t idx, double (&r)[4]) {
    float pf[4], qf[4] = {0.f, 0.f, 0.f, 0.f};
    load4<NT>(pr, idx, V, aligned, pf);
    if (resid) load4<NT>(qr, idx, V, aligned, qf);
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = rval(pf[e], qf[e], resid);
}

// Inverse-CDF draw of one index from r (see file comment).  Returns -1 when
// the total mass is not positive.  Block-uniform result.
__device__ int64_t draw_row(const float* pr, const float* qr, bool resid, int64_t V, double uf, ChainShared& sh) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
    constexpr int W = kChainBlock / kWave;
    const bool aligned = ((uintptr_t)pr % 16 == 0) && (!resid || (uintptr_t)qr % 16 == 0);
    const int64_t ntiles = (V + kTile - 1) / kTile;
    const int mult = (int)((ntiles + kMaxChunks - 1) / kMaxChunks);
    const int nch = (int)((ntiles + mult - 1) / mult);

    // ---- pass 1: chunk sums
    for (int c = wid; c < nch; c += W) {
        double acc = 0.0;
        for (int t = 0; t < mult; ++t) {
            const int64_t tb = ((int64_t)c * mult + t) * kTile;
            if (tb >= V) break;
            double r[4][4];
#pragma unroll
            for (int k = 0; k < 4; ++k) lane_r4<true>(pr, qr, resid, V, aligned, tb + k * 256 + lane * 4, r[k]);
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc += r[k][e];
        }
        acc = wave_reduce(acc, OpSumD{});
        if (lane == 0) sh.chunk[c] = acc;
    }
    __syncthreads();

    // ---- locate (wave 0)
    if (wid == 0) {
        const int g = (nch + kWave - 1) / kWave;
        const int c0 = min(nch, lane * g), c1 = min(nch, c0 + g);
        double lt = 0.0;
        for (int c = c0; c < c1; ++c) lt += sh.chunk[c];
        double incl = lt;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const double v = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += v;
        }
        const double R = __shfl(incl, kWave - 1, kWave);
        int64_t y = -1;
        if (R > 0.0) {
            const double T = uf * R;
            // chunk holding T
            const uint64_t ball = __ballot(incl > T && lt > 0.0);
            int cstar = -1;
            double base = 0.0;
            int force_last = 0;   // rounding left T past every positive chunk: take the last positive entry
            if (ball) {
                const int ls = __ffsll((unsigned long long)ball) - 1;
                const double ex = __shfl(incl, ls > 0 ? ls - 1 : 0, kWave);
                if (lane == ls) {
                    double run = ls > 0 ? ex : 0.0;
                    int lastpos = -1;
                    for (int c = c0; c < c1; ++c) {
                        const double sc = sh.chunk[c];
                        if (sc > 0.0) {
                            lastpos = c;
                            if (run + sc > T) {
                                cstar = c;
                                base = run;
                                break;
                            }
                        }
                        run += sc;
                    }
                    if (cstar < 0) {
                        cstar = lastpos;
                        force_last = 1;
                    }
                }
                cstar = __shfl(cstar, ls, kWave);
                base = __shfl(base, ls, kWave);
                force_last = __shfl(force_last, ls, kWave);
            } else {
                int lp = -1;
                for (int c = c0; c < c1; ++c)
                    if (sh.chunk[c] > 0.0) lp = c;
                cstar = wave_reduce(lp, [](int a, int b) { return a > b ? a : b; });
                force_last = 1;
            }
            // ---- search inside chunk cstar (re-read, cached loads)
            double run = base;
            int64_t lastpos = -1;
            for (int t = 0; t < mult && y < 0; ++t) {
                const int64_t tb = ((int64_t)cstar * mult + t) * kTile;
                if (tb >= V) break;
                for (int k = 0; k < 4; ++k) {
                    const int64_t idx = tb + k * 256 + lane * 4;
                    double r[4];
                    lane_r4<false>(pr, qr, resid, V, aligned, idx, r);
                    const double s = ((r[0] + r[1]) + r[2]) + r[3];
                    int my_last = -1;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (r[e] > 0.0) my_last = e;
                    if (my_last >= 0) lastpos = max(lastpos, idx + my_last);
                    if (force_last) continue;
                    double sincl = s;
#pragma unroll
                    for (int off = 1; off < kWave; off <<= 1) {
                        const double v = __shfl_up(sincl, off, kWave);
                        if (lane >= off) sincl += v;
                    }
                    double sexcl = __shfl_up(sincl, 1, kWave);
                    if (lane == 0) sexcl = 0.0;
                    const uint64_t hit = __ballot(run + sincl > T && s > 0.0);
                    if (hit) {
                        const int ls = __ffsll((unsigned long long)hit) - 1;
                        int64_t cand = -1;
                        if (lane == ls) {
                            double x = run + sexcl;
                            for (int e = 0; e < 4; ++e) {
                                x += r[e];
                                if (r[e] > 0.0 && x > T) {
                                    cand = idx + e;
                                    break;
                                }
                            }
                            if (cand < 0) cand = idx + my_last;
                        }
                        y = __shfl(cand, ls, kWave);
                        break;
                    }
                    run += __shfl(sincl, kWave - 1, kWave);
                }
            }
            if (y < 0) {
                y = wave_reduce(lastpos, [](int64_t a, int64_t b) { return a > b ? a : b; });
            }
        }
        if (lane == 0) sh.y = y;
    }
    __syncthreads();
    const int64_t y = sh.y;
    __syncthreads();
    return y;
}

__global__ __launch_bounds__(kChainBlock) void chain_reject_kernel(
    const float* __restrict__ q, const int32_t* __restrict__ x, const float* __restrict__ p,
    const uint64_t* __restrict__ seed, const uint64_t* __restrict__ offset, int64_t B, int D, int64_t V,
    const int32_t* __restrict__ req_index, int32_t* __restrict__ accepted, int32_t* __restrict__ accept_len) {
    __shared__ ChainShared sh;
    const int64_t b = req_index ? (int64_t)req_index[blockIdx.x] : (int64_t)blockIdx.x;
    if (b < 0 || b >= B) return;
    const int N = D + 1;
    const int tid = threadIdx.x;
    if (tid <= D) {
        const uint32_t w = philox_word(seed[b], offset[b], (uint64_t)tid);
        if (tid < D) {
            const int32_t xi = x[(int64_t)b * D + tid];
            bool ok = false;
            if (xi >= 0 && (int64_t)xi < V) {
                const float a = p[((int64_t)b * N + tid) * V + xi];
                const float c = q[((int64_t)b * D + tid) * V + xi];
                ok = (double)uniform_of(w) * (double)c < (double)a;
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
    const uint32_t code = sh.code;
    const double uf = (double)code * 0x1p-24;
    const float* pr = p + ((int64_t)b * N + L) * V;
    const bool resid = L < D;
    const float* qr = resid ? q + ((int64_t)b * D + L) * V : nullptr;
    int64_t y = draw_row(pr, qr, resid, V, uf, sh);
    if (y < 0 && resid) y = draw_row(pr, nullptr, false, V, uf, sh);
    if (y < 0) y = (int64_t)(((uint64_t)code * (uint64_t)V) >> 24);
    if (tid < N) {
        int32_t t;
        if (tid < L) t = x[(int64_t)b * D + tid];
        else t = (tid == L) ? (int32_t)y : -1;
        accepted[(int64_t)b * N + tid] = t;
    }
    if (tid == 0) accept_len[b] = L;
}

hipError_t launch_chain_reject(const float* draft_probs, const int32_t* draft_ids, const float* target_probs,
                               const uint64_t* seed, const uint64_t* offset, int64_t B, int D, int64_t V,
                               const int32_t* req_index, int64_t n_req, int32_t* accepted,
                               int32_t* accept_len, hipStream_t stream) {
    hipLaunchKernelGGL(chain_reject_kernel, dim3((unsigned)n_req), dim3(kChainBlock), 0, stream, draft_probs,
                       draft_ids, target_probs, seed, offset, B, D, V, req_index, accepted, accept_len);
    return hipGetLastError();
}

}  // namespace sv
