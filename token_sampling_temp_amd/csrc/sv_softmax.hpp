// Row algorithms of the temperature softmax with top-k then top-p
// renormalisation, shared by the softmax kernels and the fused verify kernel.
//
// Selection works on order-preserving integer keys of the logits (16 bits for
// bf16, 32 for float), so the kept set never depends on how exp rounds:
//   * top-k: radix select (8-bit digits, LDS count histograms) of the k-th
//     largest key; every key >= it is kept (ties kept);
//   * top-p: radix select over the same digits with LDS histograms of the
//     kept weights w = exp((z - max) / T) in 64-bit fixed point (integer
//     atomics: order independent, so results are reproducible), finding the
//     largest key whose upper mass reaches top_p times the top-k mass.
// Then out = w / sum(kept w), zero elsewhere.
#pragma once

#include "sv_argmax.hpp"

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

// Statistics of one temperature row, streamed from global memory (every pass
// re-reads it): the maximum m, the scale log2(e) / T, the smallest kept key
// (top-k, then top-p) and inv = 1 / (sum of the kept weights).  An element v
// then has probability exp2f((v - m) * scale) * inv if its key is >= kmin,
// else 0.
struct StreamStats {
    float m, scale, inv;
    uint32_t kmin;
};

template <typename T>
__device__ __forceinline__ StreamStats streamed_stats(const T* __restrict__ row, int64_t V, float Tm, int32_t k,
                                                      float tp, SmShared& sh) {
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
    return StreamStats{m, scale, (float)(1.0 / S), kmin};
}

// Statistics of one row for single-step sampling's joint filter: top-k and
// the top-p nucleus both judge the unfiltered row (the nucleus from the mass
// of every key, so radix_mass_key runs over all keys), and min-p keeps
// (v - m) >= thr = T ln(min(min_p, 1)) compared in double (thr = -inf when
// min_p is not positive).  An element v then has probability
// exp2f((v - m) * scale) * inv if its key is >= kmin and it passes min-p.
struct JointStats {
    float m, scale, inv;
    uint32_t kmin;
    double thr;
};

template <typename T>
__device__ __forceinline__ JointStats streamed_stats_joint(const T* __restrict__ row, int64_t V, float Tm, int32_t k,
                                                           float tp, float mp, SmShared& sh) {
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
            part += (uint64_t)__double2ull_rn((double)exp2f((v - m) * scale) * qscale);
        });
        const uint64_t s_fx = block_reduce<kSmBlock>(part, OpSumU64{}, (uint64_t)0, sh.red_u);
        const uint32_t kp = radix_mass_key<T>(row, V, 0u, m, scale, qshift, (double)tp * (double)s_fx, sh);
        kmin = kmin > kp ? kmin : kp;
    }
    const double thr = mp > 0.0f ? (double)Tm * log(mp < 1.0f ? (double)mp : 1.0) : -INFINITY;

    double ps = 0.0;
    row_foreach<kSmBlock, false>(row, V, [&](float v, int64_t) {
        if (logit_key<T>(v) >= kmin && (double)v - (double)m >= thr) ps += (double)exp2f((v - m) * scale);
    });
    const double S = block_reduce<kSmBlock>(ps, OpSumD{}, 0.0, sh.red_d);
    return JointStats{m, scale, (float)(1.0 / S), kmin, thr};
}

// One row streamed from global memory (every pass re-reads it).
template <typename T>
__device__ __forceinline__ void softmax_row_streamed(const T* __restrict__ row, float* __restrict__ orow, int64_t V,
                                                     float Tm, int32_t k, float tp, SmShared& sh) {
    const int tid = threadIdx.x;

    if ((double)Tm < kGreedyTemperature) {
        const int64_t y = row_argmax<kSmBlock, false>(row, V, sh.am);
        for (int64_t i = tid; i < V; i += kSmBlock) orow[i] = (i == y) ? 1.0f : 0.0f;
        return;
    }
    const StreamStats st = streamed_stats<T>(row, V, Tm, k, tp, sh);
    for (int64_t i = tid; i < V; i += kSmBlock) {
        const float v = load_elem(row + i);
        orow[i] = logit_key<T>(v) >= st.kmin ? exp2f((v - st.m) * st.scale) * st.inv : 0.0f;
    }
}

// ============================================================================
// Register-resident variant for bf16 rows (V <= 1024 * 8 * NV): the row is
// read from HBM once into registers as 16-bit order-preserving keys (8*NV
// per thread, packed in pairs) and the output is written with 16-byte stores.
//
// Selection never touches the elements twice: while the row is arriving, each
// vector is turned into keys and counted into an LDS histogram of all 65536
// keys (16-bit counters), and every later step works on that histogram.  The
// weight of an element depends only on its key, so a key's count times its
// weight gives its mass.  Top-k: one wave sums digits (the key's upper 8 bits)
// down from the maximum's digit until the count reaches k, then finds the key
// inside that digit.  Top-p: the mass of all kept keys (a block-wide pass),
// then one wave walks digits down from the maximum's until the cumulative
// mass reaches top_p times it, and finds the key inside that digit (when the
// kept keys span at most kDirectSpan values, one wave does all of it over the
// span).  Masses are 64-bit fixed point, floor(w * 2^qs) built exactly from
// the float bits of w = exp2((z - m) * log2(e) / T), so every sum is an
// order-independent integer sum and the selected keys are the same as those
// of the streamed kernel's radix selection on the same masses.  The output
// pass reads each element's probability from a per-key table built in the
// same LDS once the histogram is no longer needed.
//
// The kernel is persistent: one workgroup per compute unit walks the rows, so
// the loads of a row are issued right behind the stores of the previous one.
// Threads of a row exchange data only through LDS, so its barriers order LDS
// alone: the stores of the previous row and the loads of this one stay in
// flight across them.
//
// A row in which one key occurs 65536 times or more overflows its 16-bit
// counter; the sum of all counters then falls short of the element count, and
// the row is redone by the streamed algorithm (as are one-hot rows).
// ============================================================================
constexpr int kRrBlock = 1024;
constexpr int kRrWaves = kRrBlock / kWave;
constexpr int kKeys = 65536;
constexpr int kHistWords = kKeys / 2;     // 16-bit counters, two per dword
constexpr int kLutMax = kHistWords - 1;   // probability-table entries (slot 0 holds 0)
constexpr int kDirectSpan = 4096;         // key spans selected by one wave

// Keep the scheduler from interleaving the per-vector work of a fully
// unrolled pass (which would keep every element's temporaries live at once).
#define SV_VEC_FENCE() __builtin_amdgcn_sched_barrier(0)

// Make the register-resident row opaque to the optimiser at the start of a
// pass, so values derived from it in one pass are recomputed instead of being
// kept live across passes.
template <int NV>
__device__ __forceinline__ void launder(u32x4 (&w)[NV]) {
#pragma unroll
    for (int v = 0; v < NV; ++v) asm volatile("" : "+v"(w[v]));
}

struct RrShared {
    union {
        uint32_t hist[kHistWords];   // key k: bits 16*(k&1).. of dword k>>1
        float lut[kHistWords];       // then: lut[0] = 0, lut[1 + k - kmin] = probability of key k
        SmShared sm;                 // or: the streamed algorithm's state
    } u;
    uint64_t red[kRrWaves];          // per-wave partials of a block reduction
    uint32_t sel_digit;              // selected key (top-k, top-p)
    uint64_t sel_above;              // a wave-0 result handed to the block
    uint64_t sel_mass;               // mass at or above the top-p key
    uint32_t probe_key;              // the key of one requested element (rr_stats with a probe index)
};

typedef short s16x2 __attribute__((ext_vector_type(2)));

// Keys of the two bf16 halves of a packed pair: a non-negative bit pattern h
// maps to h + 0x8000, a negative one to 0x10000 - h, so the keys order like
// the values and -0 and +0 share the key 0x8000.
__device__ __forceinline__ uint32_t keys_of_pair(uint32_t w) {
    const u16x2 h = __builtin_bit_cast(u16x2, w);
    const uint32_t neg = __builtin_bit_cast(uint32_t, (u16x2)(0) - h);
    const uint32_t msk = __builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2, w) >> (s16x2)(15));
    const uint32_t pos = w ^ 0x80008000u;
    return (msk & neg) | (~msk & pos);
}

// The value of key k (inverse of keys_of_pair).
__device__ __forceinline__ float key_to_float(uint32_t k) {
    const uint32_t h = (k & 0x8000u) ? (k ^ 0x8000u) : ((0x10000u - k) & 0xFFFFu);
    return __uint_as_float(h << 16);
}

// Largest key among the 8 keys of a register vector.
__device__ __forceinline__ uint32_t vec_max_key(const u32x4 w) {
    const uint32_t p = pk_max_u16(pk_max_u16(w.x, w.y), pk_max_u16(w.z, w.w));
    return max(p & 0xFFFFu, p >> 16);
}

// Visit the 8 keys of register vector v: f(key, i) with i = 0..7 in
// increasing element index.
template <typename F>
__device__ __forceinline__ void visit8(const u32x4 w, F&& f) {
    f(w.x & 0xFFFFu, 0);
    f(w.x >> 16, 1);
    f(w.y & 0xFFFFu, 2);
    f(w.y >> 16, 3);
    f(w.z & 0xFFFFu, 4);
    f(w.z >> 16, 5);
    f(w.w & 0xFFFFu, 6);
    f(w.w >> 16, 7);
}

// floor(w * 2^qs) for w in [0, 1] (w a float), exactly, from its bits.
__device__ __forceinline__ uint64_t fixed_mass(float w, int qs) {
    const uint32_t bits = __float_as_uint(w);
    const int e = (int)((bits >> 23) & 0xFFu);
    if (e == 0) return 0;   // zero or denormal (< 2^-126): below any resolution used here
    const uint64_t mt = (uint64_t)((bits & 0x7FFFFFu) | 0x800000u);
    const int sh = e - 127 - 23 + qs;
    if (sh >= 0) return mt << sh;
    if (sh <= -24) return 0;
    return mt >> (-sh);
}

// 2^x with the hardware instruction (results below 2^-126 may flush to zero,
// i.e. probabilities under 1e-38 may read as 0).  Every step uses this same
// function, so a weight is identical wherever it is recomputed.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t hist_count(const RrShared& sh, uint32_t k) {
    return (sh.u.hist[k >> 1] >> ((k & 1u) << 4)) & 0xFFFFu;
}

__device__ __forceinline__ void hist_add(RrShared& sh, uint32_t k) {
    __hip_atomic_fetch_add(&sh.u.hist[k >> 1], 1u << ((k & 1u) << 4), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Block-wide reduction of a 32- or 64-bit value (every thread receives it).
template <typename T, typename Op>
__device__ __forceinline__ T rr_block_reduce(RrShared& sh, int tid, T v, Op op) {
    v = wave_allreduce(v, op);
    lds_barrier();
    if ((tid & (kWave - 1)) == 0) {
        uint64_t u = 0;
        __builtin_memcpy(&u, &v, sizeof(T));
        sh.red[tid / kWave] = u;
    }
    lds_barrier();
    T r;
    __builtin_memcpy(&r, &sh.red[0], sizeof(T));
#pragma unroll
    for (int i = 1; i < kRrWaves; ++i) {
        T x;
        __builtin_memcpy(&x, &sh.red[i], sizeof(T));
        r = op(r, x);
    }
    return r;
}

struct OpAddU32 {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; }
};
struct OpMaxU32 {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; }
};

// Sum over the histogram of count * weight for keys >= kmin (double), wave
// w taking digits w, w+16, ... as above; returns this lane's share.
__device__ __forceinline__ double rr_kept_weight(const RrShared& sh, int tid, uint32_t kmin, float m, float scale) {
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const uint2* h2 = reinterpret_cast<const uint2*>(sh.u.hist);
    double ps = 0.0;
#pragma unroll 1
    for (int g = 0; g < 256 / kRrWaves; g += 4) {
        uint2 h[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) h[j] = h2[(wave + kRrWaves * (g + j)) * 64 + lane];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d = wave + kRrWaves * (g + j);
            if ((uint32_t)(d * 256 + 255) < kmin) continue;
            const uint32_t k0 = (uint32_t)(d * 256 + 4 * lane);
            const uint32_t c[4] = {h[j].x & 0xFFFFu, h[j].x >> 16, h[j].y & 0xFFFFu, h[j].y >> 16};
            if (!__any((c[0] | c[1] | c[2] | c[3]) != 0)) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (c[e] && k0 + e >= kmin)
                    ps += (double)c[e] * (double)fast_exp2((key_to_float(k0 + e) - m) * scale);
        }
    }
    return ps;
}

// Wave 0: the k-th largest key (1 <= k < number of elements) into
// sh.sel_digit.  Digits are summed from the maximum's digit downwards until
// their count reaches k; inside that digit, the largest key whose count of
// keys at or above it (within the digit, plus the digits above) reaches k.
__device__ __noinline__ void rr_kth_key(RrShared& sh, int lane, uint32_t mkey, uint32_t k) {
    const uint2* h2 = reinterpret_cast<const uint2*>(sh.u.hist);
    uint32_t rem = k;
    int d = (int)(mkey >> 8);
    uint32_t c[4];
    uint32_t own;
    for (;;) {
        const uint2 h = h2[d * 64 + lane];
        c[0] = h.x & 0xFFFFu;
        c[1] = h.x >> 16;
        c[2] = h.y & 0xFFFFu;
        c[3] = h.y >> 16;
        own = c[0] + c[1] + c[2] + c[3];
        const uint32_t tot = wave_allreduce(own, OpAddU32{});
        if (tot >= rem || d == 0) break;
        rem -= tot;
        --d;
    }
    const uint32_t incl = wave_inclusive_sum(own, lane);
    const uint32_t above = read_lane(incl, kWave - 1) - incl;   // keys of the higher lanes
    if (lane == 0) sh.sel_digit = 0;   // (not reached when the counts are consistent)
    if (above < rem && above + own >= rem) {
        uint32_t run = above;
        int e = 3;
        for (; e > 0; --e) {
            run += c[e];
            if (run >= rem) break;
        }
        sh.sel_digit = (uint32_t)(d * 256 + 4 * lane + e);
    }
}

// Wave 0, key span kmin..mkey of at most kDirectSpan keys: top-p on the
// fixed-point masses count * floor(w * 2^qs), taken in descending key order:
// the first non-empty key whose cumulative mass reaches top_p times the span's
// mass (the lowest non-empty key if rounding leaves the target above the
// total).  sh.sel_digit = that key, sh.sel_mass = the mass at or above it.
// Lane l owns the l-th block of ceil(span / 64) keys from the top.
__device__ __noinline__ void rr_topp_direct(RrShared& sh, int lane, uint32_t kmin, uint32_t mkey, float m,
                                            float scale, int qs, float tp) {
    const int span = (int)(mkey - kmin) + 1;
    const int kpl = (span + kWave - 1) / kWave;
    auto mass_of = [&](uint32_t key, uint32_t& cnt) -> uint64_t {
        cnt = hist_count(sh, key);
        return cnt ? (uint64_t)cnt * fixed_mass(fast_exp2((key_to_float(key) - m) * scale), qs) : 0;
    };
    uint64_t lm = 0;
    uint32_t lc = 0;
    for (int j = 0; j < kpl; ++j) {
        const int i = lane * kpl + j;
        if (i < span) {
            uint32_t cnt;
            lm += mass_of(mkey - (uint32_t)i, cnt);
            lc += cnt;
        }
    }
    const uint64_t incl = wave_inclusive_sum(lm, lane);
    const uint64_t total = read_lane(incl, kWave - 1);
    const double target = (double)tp * (double)total;
    const uint64_t ball = __ballot(lc > 0 && (double)incl >= target);
    if (ball) {
        const int ls = __ffsll((unsigned long long)ball) - 1;
        if (lane == ls) {
            uint64_t run = incl - lm;
            for (int j = 0; j < kpl; ++j) {
                const int i = lane * kpl + j;
                if (i >= span) break;
                uint32_t cnt;
                const uint64_t mk = mass_of(mkey - (uint32_t)i, cnt);
                if (cnt && (double)(run + mk) >= target) {
                    sh.sel_digit = mkey - (uint32_t)i;
                    sh.sel_mass = run + mk;
                    break;
                }
                run += mk;
            }
        }
    } else {
        // rounding left the target above the total: keep everything present
        int last = -1;
        for (int j = 0; j < kpl; ++j) {
            const int i = lane * kpl + j;
            if (i < span && hist_count(sh, mkey - (uint32_t)i)) last = i;
        }
        const int lo = wave_allreduce(last, [](int x, int y) { return x > y ? x : y; });
        if (lane == 0) {
            sh.sel_digit = mkey - (uint32_t)lo;
            sh.sel_mass = total;
        }
    }
}

// Wave 0: sum of count * w over the keys kmin..mkey (span at most
// kDirectSpan), in double; every lane returns the same value.
__device__ __noinline__ double rr_span_weight(const RrShared& sh, int lane, uint32_t kmin, uint32_t mkey, float m,
                                              float scale) {
    const int span = (int)(mkey - kmin) + 1;
    const int kpl = (span + kWave - 1) / kWave;
    double ps = 0.0;
    for (int j = 0; j < kpl; ++j) {
        const int i = lane * kpl + j;
        if (i < span) {
            const uint32_t key = mkey - (uint32_t)i;
            const uint32_t cnt = hist_count(sh, key);
            if (cnt) ps += (double)cnt * (double)fast_exp2((key_to_float(key) - m) * scale);
        }
    }
    return wave_allreduce(ps, OpSumD{});
}

// This thread's share of the fixed-point mass of the keys >= kmin (all
// threads; wave w reads digits w, w+16, ..., lane l keys 4l..4l+3 of each).
__device__ __noinline__ uint64_t rr_total_mass(const RrShared& sh, int tid, uint32_t kmin, float m, float scale,
                                                  int qs) {
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const uint2* h2 = reinterpret_cast<const uint2*>(sh.u.hist);
    uint64_t ms = 0;
#pragma unroll 1
    for (int g = 0; g < 256 / kRrWaves; g += 4) {
        uint2 h[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) h[j] = h2[(wave + kRrWaves * (g + j)) * 64 + lane];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d = wave + kRrWaves * (g + j);
            const uint32_t k0 = (uint32_t)(d * 256 + 4 * lane);
            const uint32_t c[4] = {h[j].x & 0xFFFFu, h[j].x >> 16, h[j].y & 0xFFFFu, h[j].y >> 16};
            if (!__any((c[0] | c[1] | c[2] | c[3]) != 0)) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (c[e] && k0 + e >= kmin)
                    ms += (uint64_t)c[e] * fixed_mass(fast_exp2((key_to_float(k0 + e) - m) * scale), qs);
        }
    }
    return ms;
}

// Wave 0, any key span: top-p given the total fixed-point mass of the keys
// >= kmin.  Digits are visited from the maximum's digit downwards; the first
// non-empty digit whose cumulative mass reaches top_p * total holds the
// threshold, which is the first non-empty key of that digit (from the top)
// whose cumulative mass reaches it.  If rounding leaves the target above the
// total, the threshold is the lowest non-empty key.  sh.sel_digit = the
// threshold key, sh.sel_mass = the mass at or above it.  The masses are the
// same expressions as in rr_total_mass.
__device__ __noinline__ void rr_topp_topdown(RrShared& sh, int lane, uint32_t kmin, uint32_t mkey, float m,
                                             float scale, int qs, float tp, uint64_t total) {
    const uint2* h2 = reinterpret_cast<const uint2*>(sh.u.hist);
    const double target = (double)tp * (double)total;
    uint64_t above = 0;
    int lowest = -1;   // lowest non-empty key seen
    for (int d = (int)(mkey >> 8); d >= (int)(kmin >> 8); --d) {
        const uint2 h = h2[d * 64 + lane];
        const uint32_t k0 = (uint32_t)(d * 256 + 4 * lane);
        uint32_t c[4] = {h.x & 0xFFFFu, h.x >> 16, h.y & 0xFFFFu, h.y >> 16};
        uint64_t mk[4];
        uint64_t lm = 0;
        uint32_t lc = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (k0 + e < kmin) c[e] = 0;
            mk[e] = c[e] ? (uint64_t)c[e] * fixed_mass(fast_exp2((key_to_float(k0 + e) - m) * scale), qs) : 0;
            lm += mk[e];
            lc += c[e];
        }
        const uint32_t dc = wave_allreduce(lc, OpAddU32{});
        if (dc == 0) continue;
        // keys of this digit in descending order: lane 63 first, e = 3 first
        const uint64_t incl = wave_inclusive_sum(lm, lane);
        const uint64_t dm = read_lane(incl, kWave - 1);
        const uint64_t higher = dm - incl;   // mass of the keys in higher lanes
        int lo = -1;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (c[e] && lo < 0) lo = (int)(k0 + e);
        lowest = wave_allreduce(lo < 0 ? 0x7FFFFFFF : lo, [](int x, int y) { return x < y ? x : y; });
        if ((double)(above + dm) >= target) {
            const uint64_t ball = __ballot(lc > 0 && (double)(above + higher + lm) >= target);
            const int ls = 63 - __builtin_clzll((unsigned long long)ball);   // highest lane = highest keys
            if (lane == ls) {
                uint64_t run = above + higher;
                for (int e = 3; e >= 0; --e) {
                    if (c[e] && (double)(run + mk[e]) >= target) {
                        sh.sel_digit = k0 + e;
                        sh.sel_mass = run + mk[e];
                        break;
                    }
                    run += mk[e];
                }
            }
            return;
        }
        above += dm;
    }
    // rounding left the target above the total: keep everything present
    if (lane == 0) {
        sh.sel_digit = (uint32_t)lowest;
        sh.sel_mass = total;
    }
}

// Statistics of one register-resident row: the maximum key's value m, the
// scale, the smallest kept key, inv = 1 / (sum of the kept weights), and
// whether LDS holds the per-key probability table lut[1 + key - kmin] (keys
// kmin..max; lut[0] = 0).  Without the table, key >= kmin has probability
// fast_exp2((key_to_float(key) - m) * scale) * inv.
struct RrStats {
    float m, scale, inv;
    uint32_t kmin;
    bool table;
};

// Loads one row that is 16-byte aligned with V a multiple of 8 (every
// 16-byte vector lies wholly inside or wholly past the end of the row; buffer
// loads return zeros past the end) into w as keys, then selects and builds
// the table.  Returns false if a histogram counter overflowed.
//
// JOINT (single-step sampling): top-k and the top-p nucleus both judge the
// unfiltered row (the nucleus walk runs over every key), and min-p (mp > 0)
// keeps the keys whose value v satisfies (v - m) >= T ln(min(mp, 1)) in
// double, the smallest such key found by binary search (keys order like their
// values); the kept key is the largest of the three thresholds.
//
// vmax (not NULL): receives the largest key of each of the thread's vectors,
// two 16-bit keys per word (vector v in bits 16 * (v & 1) of word v / 2), so
// that a caller can revisit only the vectors that hold kept keys.
// probe (>= 0): the key of element `probe` is left in sh.probe_key (by the
// thread that holds it, before the selection's barriers).
template <int NV>
__device__ __forceinline__ void rr_issue(const uint16_t* __restrict__ row, int64_t V, int tid, u32x4 (&w)[NV]) {
    const __amdgpu_buffer_rsrc_t rin = make_rsrc(row, (uint32_t)(V * 2));
#pragma unroll
    for (int v = 0; v < NV; ++v)
        w[v] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rin, tid * 16, v * kRrBlock * 16, 0));
}

template <int NV, bool JOINT = false, bool VMAX = false>
__device__ __forceinline__ bool rr_stats(RrShared& sh, const uint16_t* __restrict__ row, int64_t V, float Tm,
                                         int32_t k, float tp, int tid, u32x4 (&w)[NV], RrStats& st, float mp,
                                         uint32_t (&vmax)[(NV + 1) / 2], int64_t probe = -1) {
    const int vfull = (int)(V / (kRrBlock * 8));   // vectors in range for every thread
    auto ebase = [&](int v) { return (v * kRrBlock + tid) * 8; };
    // ---- issue the row's loads
    rr_issue<NV>(row, V, tid, w);
    // ---- clear the histogram (the previous row's table reads are done first)
    lds_barrier();
    {
        uint4* h4 = reinterpret_cast<uint4*>(sh.u.hist);
#pragma unroll
        for (int i = 0; i < kHistWords / 4 / kRrBlock; ++i) h4[i * kRrBlock + tid] = make_uint4(0, 0, 0, 0);
    }
    lds_barrier();

    // ---- as each vector arrives: keys, running maximum, histogram (vectors
    // past the end of the row become bf16 -inf, key 0x0080, below every
    // finite logit; their count is taken out of the histogram below)
    uint32_t lk = 0;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        u32x4 x = w[v];
        if (v >= vfull && ebase(v) >= V) x = u32x4{0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u};
        x.x = keys_of_pair(x.x);
        x.y = keys_of_pair(x.y);
        x.z = keys_of_pair(x.z);
        x.w = keys_of_pair(x.w);
        const uint32_t vk = vec_max_key(x);
        lk = max(lk, vk);
        if constexpr (VMAX) {
            if (v & 1) vmax[v >> 1] |= vk << 16;
            else vmax[v >> 1] = vk;
        }
        if (probe >= 0 && (probe >> 3) == (int64_t)(v * kRrBlock + tid)) {
            const int i = (int)(probe & 7);
            const uint32_t wd = i < 2 ? x.x : (i < 4 ? x.y : (i < 6 ? x.z : x.w));
            sh.probe_key = (wd >> (16 * (i & 1))) & 0xFFFFu;
        }
        visit8(x, [&](uint32_t key, int) { hist_add(sh, key); });
        w[v] = x;
        SV_VEC_FENCE();
    }
    const uint32_t mkey = rr_block_reduce(sh, tid, lk, OpMaxU32{});   // its barriers also end the histogram
    const float m = key_to_float(mkey);

    // ---- overflow check (possible only when the row's slots number 65536 or
    // more): the 16-bit counters must add up to the slot count
    if (NV * 8 * kRrBlock > 65535) {
        const uint4* h4 = reinterpret_cast<const uint4*>(sh.u.hist);
        uint32_t all = 0;
#pragma unroll
        for (int i = 0; i < kHistWords / 4 / kRrBlock; ++i) {
            const uint4 q = h4[i * kRrBlock + tid];
            all += (q.x & 0xFFFFu) + (q.x >> 16) + (q.y & 0xFFFFu) + (q.y >> 16) + (q.z & 0xFFFFu) + (q.z >> 16) +
                   (q.w & 0xFFFFu) + (q.w >> 16);
        }
        const uint32_t total = rr_block_reduce(sh, tid, all, OpAddU32{});
        if (total != (uint32_t)(NV * 8 * kRrBlock)) return false;
    }
    {
        const uint32_t npad = (uint32_t)((int64_t)NV * 8 * kRrBlock - V);
        if (tid == 0 && npad) sh.u.hist[0x80u >> 1] -= npad;   // key 0x0080 (bf16 -inf) sits in the low half
        lds_barrier();
    }

    const float scale = kLog2e / Tm;
    uint32_t kmin = 0;

    // ---- top-k: k-th largest key, all ties kept (wave 0 walks the digits
    // down from the maximum's)
    if (k > 0 && (int64_t)k < V) {
        if (tid < kWave) rr_kth_key(sh, tid, mkey, (uint32_t)k);
        lds_barrier();
        kmin = sh.sel_digit;
    }

    // ---- top-p over the kept keys; S = sum of the kept weights.  A key span
    // kmin..mkey of at most kDirectSpan keys is handled by wave 0 alone.
    const int lg = V > 1 ? 64 - __clzll((unsigned long long)(V - 1)) : 0;
    const int qs = 62 - lg;
    const bool direct = mkey - kmin < (uint32_t)kDirectSpan;
    double S;
    if constexpr (JOINT) {
        if (tp < 1.0f) {
            const uint64_t total = rr_block_reduce(sh, tid, rr_total_mass(sh, tid, 0u, m, scale, qs), OpSumU64{});
            if (tid < kWave) rr_topp_topdown(sh, tid, 0u, mkey, m, scale, qs, tp, total);
            lds_barrier();
            kmin = max(kmin, sh.sel_digit);
        }
        if (mp > 0.0f) {
            const double thr = (double)Tm * log(mp < 1.0f ? (double)mp : 1.0);
            uint32_t lo = 0, hi = mkey;   // the maximum's key always passes (thr <= 0)
            while (lo < hi) {
                const uint32_t mid = (lo + hi) >> 1;
                if ((double)key_to_float(mid) - (double)m >= thr) hi = mid;
                else lo = mid + 1;
            }
            kmin = max(kmin, lo);
        }
        if (mkey - kmin < (uint32_t)kDirectSpan) {
            if (tid < kWave) {
                const double ws = rr_span_weight(sh, tid, kmin, mkey, m, scale);
                if (tid == 0) sh.sel_above = __builtin_bit_cast(uint64_t, ws);
            }
            lds_barrier();
            S = __builtin_bit_cast(double, sh.sel_above);
        } else {
            S = rr_block_reduce(sh, tid, rr_kept_weight(sh, tid, kmin, m, scale), OpSumD{});
        }
    } else if (tp < 1.0f && direct) {
        if (tid < kWave) rr_topp_direct(sh, tid, kmin, mkey, m, scale, qs, tp);
        lds_barrier();
        kmin = sh.sel_digit;
        S = (double)sh.sel_mass * ldexp(1.0, -qs);
    } else if (tp < 1.0f) {
        const uint64_t total = rr_block_reduce(sh, tid, rr_total_mass(sh, tid, kmin, m, scale, qs), OpSumU64{});
        if (tid < kWave) rr_topp_topdown(sh, tid, kmin, mkey, m, scale, qs, tp, total);
        lds_barrier();
        kmin = sh.sel_digit;
        S = (double)sh.sel_mass * ldexp(1.0, -qs);
    } else if (direct) {
        if (tid < kWave) {
            const double ws = rr_span_weight(sh, tid, kmin, mkey, m, scale);
            if (tid == 0) sh.sel_above = __builtin_bit_cast(uint64_t, ws);
        }
        lds_barrier();
        S = __builtin_bit_cast(double, sh.sel_above);
    } else {
        S = rr_block_reduce(sh, tid, rr_kept_weight(sh, tid, kmin, m, scale), OpSumD{});
    }
    const float inv = (float)(1.0 / S);

    // ---- probability table over keys kmin..mkey (replaces the histogram)
    const uint32_t span = mkey - kmin;   // the table holds span + 1 keys
    const bool table = span < (uint32_t)kLutMax;
    lds_barrier();
    if (table) {
        for (uint32_t j = tid; j <= span; j += kRrBlock)
            sh.u.lut[1 + j] = fast_exp2((key_to_float(kmin + j) - m) * scale) * inv;
        if (tid == 0) sh.u.lut[0] = 0.0f;
        lds_barrier();
    }

    st = RrStats{m, scale, inv, kmin, table};
    return true;
}

template <int NV, bool JOINT = false>
__device__ __forceinline__ bool rr_stats(RrShared& sh, const uint16_t* __restrict__ row, int64_t V, float Tm,
                                         int32_t k, float tp, int tid, u32x4 (&w)[NV], RrStats& st,
                                         float mp = 0.0f) {
    uint32_t unused[(NV + 1) / 2];
    return rr_stats<NV, JOINT, false>(sh, row, V, Tm, k, tp, tid, w, st, mp, unused);
}

// One register-resident row (rr_stats), then the output written with 16-byte
// buffer stores (dropped past the end of the row).  Returns false, with
// nothing written, if a histogram counter overflowed.
template <int NV>
__device__ __forceinline__ bool rr_row(RrShared& sh, const uint16_t* __restrict__ row, float* __restrict__ orow,
                                       int64_t V, float Tm, int32_t k, float tp) {
    // the thread index is made opaque per row, so nothing derived from it is
    // hoisted out of the row loop and held in registers across rows
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    u32x4 w[NV];
    RrStats st;
    if (!rr_stats<NV>(sh, row, V, Tm, k, tp, tid, w, st)) return false;
    const __amdgpu_buffer_rsrc_t rout = make_rsrc(orow, (uint32_t)(V * 4));
    const uint32_t kmin = st.kmin;
    const float m = st.m, scale = st.scale, inv = st.inv;
    const bool table = st.table;

    // ---- write
    const int koff = 1 - (int)kmin;
    launder<NV>(w);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        float o[8];
        if (__any(vec_max_key(w[v]) >= kmin)) {
            if (table) {
                visit8(w[v], [&](uint32_t key, int i) { o[i] = sh.u.lut[max((int)key + koff, 0)]; });
            } else {
                visit8(w[v], [&](uint32_t key, int i) {
                    o[i] = (key >= kmin) ? fast_exp2((key_to_float(key) - m) * scale) * inv : 0.0f;
                });
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = 0.0f;
        }
        const u32x4 a = {__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])};
        const u32x4 c = {__float_as_uint(o[4]), __float_as_uint(o[5]), __float_as_uint(o[6]), __float_as_uint(o[7])};
        __builtin_amdgcn_raw_buffer_store_b128(a, rout, tid * 32, v * kRrBlock * 32, 0);
        __builtin_amdgcn_raw_buffer_store_b128(c, rout, tid * 32 + 16, v * kRrBlock * 32, 0);
        SV_VEC_FENCE();
    }
    return true;
}


}  // namespace sv
