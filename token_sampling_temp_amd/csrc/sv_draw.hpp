// Pieces of the inverse-CDF draw shared by the chain-rejection and fused
// verify kernels.
#pragma once

#include "sv_common.hpp"

namespace sv {

// Weight of an entry in the draw: the residual max(0, p - q) or, for the
// bonus draw, p itself (double, exact from float inputs).
__device__ __forceinline__ double rval(float pv, float qv, bool resid) {
    return resid ? fmax(0.0, (double)pv - (double)qv) : (double)pv;
}

// Inclusive 64-lane scan (DPP, fixed association order).
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
    return wave_inclusive_sum(v, (int)(threadIdx.x & (kWave - 1)));
}

// One wave: given 'n' ordered non-negative masses m[0..n) (read
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
    const double ex = wave_shift_up1(incl);
    R = read_lane(incl, kWave - 1);
    base = 0.0;
    force_last = 0;
    if (!(R > 0.0)) return -1;
    const double T = uf * R;
    const uint64_t ball = __ballot(incl > T && lt > 0.0);
    int pick = -1;
    if (ball) {
        const int ls = __ffsll((unsigned long long)ball) - 1;
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
        pick = read_lane(pick, ls);
        base = read_lane(base, ls);
        force_last = read_lane(force_last, ls);
    } else {
        int lp = -1;
        for (int i = i0; i < i1; ++i)
            if (get(i) > 0.0) lp = i;
        pick = wave_allreduce(lp, [](int a, int b) { return a > b ? a : b; });
        force_last = 1;
    }
    return pick;
}

}  // namespace sv
