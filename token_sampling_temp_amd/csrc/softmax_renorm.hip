// Temperature softmax with top-k then top-p renormalisation; one workgroup
// per (request, position) row.
//
// Selection works on order-preserving integer keys of the logits (16 bits for
// bf16, 32 for float), so the kept set never depends on how exp rounds:
//   * top-k: radix select (8-bit digits, LDS count histograms) of the k-th
//     largest key; every key >= it is kept (ties kept);
//   * top-p: radix select over the same digits with LDS histograms of the
//     kept weights w = exp((z - max) / T) in 64-bit fixed point (integer
//     atomics: order independent, so results are reproducible), finding the
//     largest key whose upper mass reaches top_p times the top-k mass.
// Then out = w / sum(kept w), zero elsewhere.  T < 1e-5 writes a one-hot at
// the lowest-index argmax.
#include "sv_argmax.hpp"
#include "sv_launch.hpp"

namespace sv {

constexpr int kSmBlock = 1024;
constexpr float kLog2e = 1.4426950408889634f;

struct SmShared {
    ArgmaxShared<kSmBlock> am;
    uint32_t hist_c[256];
    unsigned long long hist_m[256];
    double red_d[kSmBlock / kWave];
    uint64_t red_u[kSmBlock / kWave];
    float red_f[kSmBlock / kWave];
    uint32_t sel_digit;
    uint32_t sel_rem;
    uint64_t sel_above;
};

template <typename T>
struct KeyBits;
template <>
struct KeyBits<float> {
    static constexpr int kBits = 32;
};
template <>
struct KeyBits<uint16_t> {
    static constexpr int kBits = 16;
};

template <typename T>
__device__ __forceinline__ uint32_t logit_key(float v) {
    return float_key(v) >> (32 - KeyBits<T>::kBits);
}

// Wave 0 scans 256 digit bins from the top.  Count mode: first digit d with
// sum_{d' >= d} cnt >= rem.  Mass mode: first digit with above + sum mass >=
// target (falls back to the lowest non-empty digit).  Results go to sh.sel_*.
__device__ void select_digit_count(SmShared& sh, uint32_t rem) {
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t c[4], lsum = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        c[e] = sh.hist_c[255 - 4 * lane - e];
        lsum += c[e];
    }
    uint32_t incl = lsum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t v = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += v;
    }
    const uint32_t excl = incl - lsum;
    const uint64_t ball = __ballot(incl >= rem);
    const int ls = __ffsll((unsigned long long)ball) - 1;
    if (lane == ls) {
        uint32_t run = excl;
        for (int e = 0; e < 4; ++e) {
            if (run + c[e] >= rem) {
                sh.sel_digit = 255 - 4 * lane - e;
                sh.sel_rem = rem - run;
                break;
            }
            run += c[e];
        }
    }
}

__device__ void select_digit_mass(SmShared& sh, uint64_t above, double target) {
    const int lane = threadIdx.x & (kWave - 1);
    uint64_t m[4], lsum = 0;
    uint32_t c[4];
    uint32_t lowest = 0xFFFFFFFFu;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int d = 255 - 4 * lane - e;
        m[e] = sh.hist_m[d];
        c[e] = sh.hist_c[d];
        lsum += m[e];
        if (c[e]) lowest = (uint32_t)d;
    }
    uint64_t incl = lsum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint64_t v = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += v;
    }
    const uint64_t excl = incl - lsum;
    // first (highest) non-empty digit whose cumulative upper mass reaches the target
    int first_ok = -1;
    {
        uint64_t run = excl;
        for (int e = 0; e < 4; ++e) {
            run += m[e];
            if (first_ok < 0 && c[e] && (double)(above + run) >= target) first_ok = e;
        }
    }
    const uint64_t ball = __ballot(first_ok >= 0);
    if (ball) {
        const int ls = __ffsll((unsigned long long)ball) - 1;
        if (lane == ls) {
            uint64_t run = excl;
            for (int e = 0; e < first_ok; ++e) run += m[e];
            sh.sel_digit = 255 - 4 * lane - first_ok;
            sh.sel_above = above + run;
        }
    } else {
        // rounding left the target above the total: keep everything present
        const uint32_t lo = wave_reduce(lowest, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
        uint64_t part = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if ((uint32_t)(255 - 4 * lane - e) > lo) part += m[e];
        const uint64_t above_lo = wave_reduce(part, OpSumU64{});
        if (lane == 0) {
            sh.sel_digit = lo;
            sh.sel_above = above + above_lo;
        }
    }
}

template <typename T>
__device__ uint32_t radix_kth_key(const T* row, int64_t V, uint32_t k, SmShared& sh) {
    constexpr int KB = KeyBits<T>::kBits;
    uint32_t prefix = 0, rem = k;
    for (int shift = KB - 8; shift >= 0; shift -= 8) {
        for (int i = threadIdx.x; i < 256; i += kSmBlock) sh.hist_c[i] = 0;
        __syncthreads();
        const int hs = shift + 8;
        row_foreach<kSmBlock, false>(row, V, [&](float v, int64_t) {
            const uint32_t key = logit_key<T>(v);
            if (hs >= KB || (key >> hs) == prefix) atomicAdd(&sh.hist_c[(key >> shift) & 255u], 1u);
        });
        __syncthreads();
        if (threadIdx.x < kWave) select_digit_count(sh, rem);
        __syncthreads();
        prefix = (prefix << 8) | sh.sel_digit;
        rem = sh.sel_rem;
    }
    return prefix;
}

template <typename T>
__device__ uint32_t radix_mass_key(const T* row, int64_t V, uint32_t kmin, float m, float scale, int qshift,
                                   double target, SmShared& sh) {
    constexpr int KB = KeyBits<T>::kBits;
    const double qscale = ldexp(1.0, qshift);
    uint32_t prefix = 0;
    uint64_t above = 0;
    for (int shift = KB - 8; shift >= 0; shift -= 8) {
        for (int i = threadIdx.x; i < 256; i += kSmBlock) {
            sh.hist_c[i] = 0;
            sh.hist_m[i] = 0;
        }
        __syncthreads();
        const int hs = shift + 8;
        row_foreach<kSmBlock, false>(row, V, [&](float v, int64_t) {
            const uint32_t key = logit_key<T>(v);
            if (key >= kmin && (hs >= KB || (key >> hs) == prefix)) {
                const float w = exp2f((v - m) * scale);
                const unsigned long long wq = (unsigned long long)__double2ull_rn((double)w * qscale);
                const uint32_t d = (key >> shift) & 255u;
                atomicAdd(&sh.hist_c[d], 1u);
                if (wq) atomicAdd(&sh.hist_m[d], wq);
            }
        });
        __syncthreads();
        if (threadIdx.x < kWave) select_digit_mass(sh, above, target);
        __syncthreads();
        prefix = (prefix << 8) | sh.sel_digit;
        above = sh.sel_above;
    }
    return prefix;
}

template <typename T>
__global__ __launch_bounds__(kSmBlock) void softmax_renorm_kernel(
    const T* __restrict__ logits, int64_t B, int npos, int64_t V, const float* __restrict__ temperature,
    const int32_t* __restrict__ top_k, const float* __restrict__ top_p, const int32_t* __restrict__ req_index,
    float* __restrict__ out) {
    __shared__ SmShared sh;
    const int64_t b = req_index ? (int64_t)req_index[blockIdx.x] : (int64_t)blockIdx.x;
    if (b < 0 || b >= B) return;
    const int64_t r = (int64_t)b * npos + blockIdx.y;
    const T* row = logits + r * V;
    float* orow = out + r * V;
    const float Tm = temperature[b];
    const int tid = threadIdx.x;

    if ((double)Tm < kGreedyTemperature) {
        const int64_t y = row_argmax<kSmBlock, false>(row, V, sh.am);
        for (int64_t i = tid; i < V; i += kSmBlock) orow[i] = (i == y) ? 1.0f : 0.0f;
        return;
    }
    const int32_t k = top_k ? top_k[b] : 0;
    const float tp = top_p ? top_p[b] : 1.0f;

    float lm = -INFINITY;
    row_foreach<kSmBlock, false>(row, V, [&](float v, int64_t) { lm = fmaxf(lm, v); });
    const float m = block_reduce<kSmBlock>(lm, OpMaxF{}, -INFINITY, sh.red_f);
    const float scale = kLog2e / Tm;

    uint32_t kmin = 0;
    if (k > 0 && (int64_t)k < V) kmin = radix_kth_key<T>(row, V, (uint32_t)k, sh);

    if (tp < 1.0f) {
        const int lg = V > 1 ? 64 - __clzll((unsigned long long)(V - 1)) : 0;
        const int qshift = 62 - lg;
        const double qscale = ldexp(1.0, qshift);
        uint64_t part = 0;
        row_foreach<kSmBlock, false>(row, V, [&](float v, int64_t) {
            if (logit_key<T>(v) >= kmin)
                part += (uint64_t)__double2ull_rn((double)exp2f((v - m) * scale) * qscale);
        });
        const uint64_t s_fx = block_reduce<kSmBlock>(part, OpSumU64{}, (uint64_t)0, sh.red_u);
        const double target = (double)tp * (double)s_fx;
        kmin = radix_mass_key<T>(row, V, kmin, m, scale, qshift, target, sh);
    }

    double ps = 0.0;
    row_foreach<kSmBlock, false>(row, V, [&](float v, int64_t) {
        if (logit_key<T>(v) >= kmin) ps += (double)exp2f((v - m) * scale);
    });
    const double S = block_reduce<kSmBlock>(ps, OpSumD{}, 0.0, sh.red_d);
    const float inv = (float)(1.0 / S);
    for (int64_t i = tid; i < V; i += kSmBlock) {
        const float v = load_elem(row + i);
        orow[i] = logit_key<T>(v) >= kmin ? exp2f((v - m) * scale) * inv : 0.0f;
    }
}

hipError_t launch_softmax_renorm(const void* logits, int dtype, int64_t B, int64_t npos, int64_t V,
                                 const float* temperature, const int32_t* top_k, const float* top_p,
                                 const int32_t* req_index, int64_t n_req, float* probs_out,
                                 hipStream_t stream) {
    const dim3 grid((unsigned)n_req, (unsigned)npos), block(kSmBlock);
    if (dtype == kDtypeBF16)
        hipLaunchKernelGGL(softmax_renorm_kernel<uint16_t>, grid, block, 0, stream,
                           static_cast<const uint16_t*>(logits), B, (int)npos, V, temperature, top_k, top_p,
                           req_index, probs_out);
    else
        hipLaunchKernelGGL(softmax_renorm_kernel<float>, grid, block, 0, stream,
                           static_cast<const float*>(logits), B, (int)npos, V, temperature, top_k, top_p,
                           req_index, probs_out);
    return hipGetLastError();
}

}  // namespace sv
