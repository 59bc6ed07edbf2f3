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

// ============================================================================
// Register-resident variant for bf16 rows (V <= 1024 * 8 * NV): the row is
// read from HBM once into registers (8*NV bf16 per thread, packed in pairs),
// every selection pass runs over registers, and the output is written with
// 16-byte stores.  Radix histograms are privatised 16 ways in LDS (lane & 15
// picks the copy), so lanes of a wave that hit one digit rarely collide on one
// address.  Top-p masses are 64-bit fixed point built exactly from the float
// bits of w = exp2((z - m) * log2(e) / T) (floor to 2^-qs), so every sum is an
// order-independent integer sum.
// ============================================================================
constexpr int kRrBlock = 1024;
constexpr int kCopies = 16;

// Keep the scheduler from interleaving the per-vector work of a fully
// unrolled pass (which would keep every element's temporaries live at once).
#define SV_VEC_FENCE() __builtin_amdgcn_sched_barrier(0)

// Make the register-resident row opaque to the optimiser at the start of a
// pass, so values derived from it in one pass (unpacked halves, keys) are
// recomputed instead of being kept live across passes.
template <int NV>
__device__ __forceinline__ void launder(u32x4 (&w)[NV]) {
#pragma unroll
    for (int v = 0; v < NV; ++v) asm volatile("" : "+v"(w[v]));
}

struct RrShared {
    uint32_t hc[256 * kCopies];
    unsigned long long hm[256 * kCopies];
    uint32_t cc[256];              // copies folded per digit
    unsigned long long cm[256];
    float red_f[kRrBlock / kWave];
    double red_d[kRrBlock / kWave];
    int64_t red_i[kRrBlock / kWave];
    uint32_t sel_digit;
    uint32_t sel_rem;
    uint64_t sel_above;
    uint64_t sel_mass;
};

// Raw buffer descriptor (gfx9 family third dword) over num_bytes bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes, 0x00020000);
}

// 16-bit order-preserving key of a bf16 bit pattern; -0 and +0 share a key.
__device__ __forceinline__ uint32_t bf16_key(uint32_t h) {
    h = (h == 0x8000u) ? 0u : h;
    return (h & 0x8000u) ? (~h & 0xFFFFu) : (h | 0x8000u);
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

// Visit the 8 bf16 bit patterns of register vector v: f(h, i) with i = 0..7
// in increasing element index.
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

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) { return __uint_as_float(h << 16); }

// 2^x with the hardware instruction (results below 2^-126 may flush to zero,
// i.e. probabilities under 1e-38 may read as 0).  Every pass uses this same
// function, so a weight is identical wherever it is recomputed.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave 0: choose the digit from the privatised histograms (sum of the 16
// copies per bin).  Lane l owns digits 255-4l .. 252-4l (descending).
// Count mode (mass_mode false): first digit d from the top whose cumulative
// count reaches rem.  Mass mode: first non-empty digit whose cumulative mass
// (plus `above`) reaches target, else the lowest non-empty digit.  Written
// to keep few registers live (the caller holds the row in registers).
__device__ __forceinline__ uint32_t rr_bin_count(const RrShared& sh, int d) { return sh.cc[d]; }
__device__ __forceinline__ uint64_t rr_bin_mass(const RrShared& sh, int d) { return sh.cm[d]; }

// Threads 0..255 fold the 16 copies of their digit into cc / cm (caller syncs).
__device__ __forceinline__ void rr_fold(RrShared& sh, bool mass) {
    const int d = threadIdx.x;
    if (d < 256) {
        uint32_t c = 0;
        uint64_t m = 0;
#pragma unroll 2
        for (int k = 0; k < kCopies; ++k) {
            c += sh.hc[d * kCopies + ((k + d) & (kCopies - 1))];
            if (mass) m += sh.hm[d * kCopies + ((k + d) & (kCopies - 1))];
        }
        sh.cc[d] = c;
        if (mass) sh.cm[d] = m;
    }
}

__device__ void rr_select(RrShared& sh, bool mass_mode, uint32_t rem, uint64_t above, double target) {
    const int lane = threadIdx.x & (kWave - 1);
    const int d0 = 255 - 4 * lane;
    uint32_t lc = 0;
    uint64_t lm = 0;
    for (int e = 0; e < 4; ++e) {
        lc += rr_bin_count(sh, d0 - e);
        if (mass_mode) lm += rr_bin_mass(sh, d0 - e);
    }
    if (!mass_mode) {
        uint32_t incl = lc;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const uint32_t v = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += v;
        }
        const uint64_t ball = __ballot(incl >= rem);
        const int ls = __ffsll((unsigned long long)ball) - 1;
        if (lane == ls) {
            uint32_t run = incl - lc;
            for (int e = 0; e < 4; ++e) {
                const uint32_t c = rr_bin_count(sh, d0 - e);
                if (run + c >= rem) {
                    sh.sel_digit = (uint32_t)(d0 - e);
                    sh.sel_rem = rem - run;
                    break;
                }
                run += c;
            }
        }
        return;
    }
    uint64_t incl = lm;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint64_t v = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += v;
    }
    // a lane holds the answer iff it has a non-empty digit and its inclusive mass reaches the target
    const uint64_t ball = __ballot(lc > 0 && (double)(above + incl) >= target);
    if (ball) {
        const int ls = __ffsll((unsigned long long)ball) - 1;
        if (lane == ls) {
            uint64_t run = incl - lm;
            for (int e = 0; e < 4; ++e) {
                const uint32_t c = rr_bin_count(sh, d0 - e);
                const uint64_t m = rr_bin_mass(sh, d0 - e);
                if (c && (double)(above + run + m) >= target) {
                    sh.sel_digit = (uint32_t)(d0 - e);
                    sh.sel_above = above + run;
                    sh.sel_mass = m;
                    break;
                }
                run += m;
            }
        }
    } else {
        // rounding left the target above the total: keep everything present
        uint32_t lowest = 0xFFFFFFFFu;
        for (int e = 0; e < 4; ++e)
            if (rr_bin_count(sh, d0 - e)) lowest = (uint32_t)(d0 - e);
        const uint32_t lo = wave_reduce(lowest, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
        uint64_t part = 0, at = 0;
        for (int e = 0; e < 4; ++e) {
            const uint32_t d = (uint32_t)(d0 - e);
            if (d >= lo) {
                const uint64_t m = rr_bin_mass(sh, (int)d);
                if (d > lo) part += m;
                else at = m;
            }
        }
        const uint64_t above_lo = wave_reduce(part, OpSumU64{});
        const uint64_t at_lo = wave_reduce(at, OpSumU64{});
        if (lane == 0) {
            sh.sel_digit = lo;
            sh.sel_above = above + above_lo;
            sh.sel_mass = at_lo;
        }
    }
}

__device__ __forceinline__ void rr_clear(RrShared& sh, bool mass) {
    for (int i = threadIdx.x; i < 256 * kCopies; i += kRrBlock) {
        sh.hc[i] = 0;
        if (mass) sh.hm[i] = 0;
    }
}

template <int NV>
__global__ __launch_bounds__(kRrBlock) void softmax_renorm_rr_kernel(
    const uint16_t* __restrict__ logits, int64_t B, int npos, int64_t V, const float* __restrict__ temperature,
    const int32_t* __restrict__ top_k, const float* __restrict__ top_p, const int32_t* __restrict__ req_index,
    float* __restrict__ out) {
    __shared__ RrShared sh;
    const int64_t b = req_index ? (int64_t)req_index[blockIdx.x] : (int64_t)blockIdx.x;
    if (b < 0 || b >= B) return;
    const int64_t r = (int64_t)b * npos + blockIdx.y;
    const uint16_t* row = logits + r * V;
    float* orow = out + r * V;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const bool in_al = ((uintptr_t)row & 15u) == 0;
    const bool out_al = ((uintptr_t)orow & 15u) == 0;
    // Buffer descriptors over this row (range-checked by the hardware): one
    // per-thread VGPR offset, the per-vector offset is a scalar.
    const __amdgpu_buffer_rsrc_t rin = make_rsrc(row, (uint32_t)(V * 2));
    const __amdgpu_buffer_rsrc_t rout = make_rsrc(orow, (uint32_t)(V * 4));
    const int vfull = (int)(V / (kRrBlock * 8));   // vectors that are in range for every thread
    auto ebase = [&](int v) { return (v * kRrBlock + tid) * 8; };

    // ---- load the row once (padding = bf16 -inf, which never changes a result)
    u32x4 w[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        if (in_al && v < vfull) {
            w[v] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rin, tid * 16, v * kRrBlock * 16, 0));
        } else {
            const int e0 = ebase(v);
            uint32_t h[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) h[i] = (e0 + i < V) ? (uint32_t)row[e0 + i] : 0xFF80u;
            w[v].x = h[0] | (h[1] << 16);
            w[v].y = h[2] | (h[3] << 16);
            w[v].z = h[4] | (h[5] << 16);
            w[v].w = h[6] | (h[7] << 16);
        }
    }
    SV_VEC_FENCE();
    const float Tm = temperature[b];

    // ---- maximum
    float lm = -INFINITY;
launder<NV>(w);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        visit8(w[v], [&](uint32_t h, int) { lm = fmaxf(lm, bf16_bits_to_float(h)); });
        SV_VEC_FENCE();
    }
    const float m = block_reduce<kRrBlock>(lm, OpMaxF{}, -INFINITY, sh.red_f);

    auto store8 = [&](int v, const float (&o)[8]) {
        if (out_al && v < vfull) {
            const u32x4 a = {__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])};
            const u32x4 c = {__float_as_uint(o[4]), __float_as_uint(o[5]), __float_as_uint(o[6]), __float_as_uint(o[7])};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, a),
                                                   rout, tid * 32, v * kRrBlock * 32, 0);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, c),
                                                   rout, tid * 32 + 16, v * kRrBlock * 32, 0);
        } else {
            const int e0 = ebase(v);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (e0 + i < V) orow[e0 + i] = o[i];
        }
    };

    const bool greedy = (double)Tm < kGreedyTemperature;
    int y32 = -1;
    if (greedy) {
        // lowest index holding the maximum (branch-free 32-bit minimum)
        int cand = 0x7FFFFFFF;
        launder<NV>(w);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            visit8(w[v], [&](uint32_t h, int i) {
                const int idx = ebase(v) + i;
                cand = min(cand, (bf16_bits_to_float(h) == m && idx < V) ? idx : 0x7FFFFFFF);
            });
            SV_VEC_FENCE();
        }
        y32 = (int)block_reduce<kRrBlock>((int64_t)cand, OpMinI64{}, (int64_t)INT64_MAX, sh.red_i);
    }
    const float scale = kLog2e / Tm;
    uint32_t kmin = 0;
    float inv = 1.0f;
    if (!greedy) {
        const int32_t k = top_k ? top_k[b] : 0;
        const float tp = top_p ? top_p[b] : 1.0f;
        const int copy = lane & (kCopies - 1);

        // ---- top-k: k-th largest key (two 8-bit digits), all ties kept
        if (k > 0 && (int64_t)k < V) {
            uint32_t prefix = 0, rem = (uint32_t)k;
            for (int shift = 8; shift >= 0; shift -= 8) {
                rr_clear(sh, false);
                __syncthreads();
    launder<NV>(w);
    #pragma unroll
                for (int v = 0; v < NV; ++v) {
                    visit8(w[v], [&](uint32_t h, int) {
                        const uint32_t key = bf16_key(h);
                        if (shift == 8 || (key >> 8) == prefix)
                            atomicAdd(&sh.hc[((key >> shift) & 255u) * kCopies + copy], 1u);
                    });
                    SV_VEC_FENCE();
                }
                __syncthreads();
                rr_fold(sh, false);
                __syncthreads();
                if (tid < kWave) rr_select(sh, false, rem, 0, 0.0);
                __syncthreads();
                prefix = (prefix << 8) | sh.sel_digit;
                rem = sh.sel_rem;
            }
            kmin = prefix;
        }

        // ---- top-p over the kept keys; fixed-point masses
        const int lg = V > 1 ? 64 - __clzll((unsigned long long)(V - 1)) : 0;
        const int qs = 62 - lg;
        double S = 1.0;
        if (tp < 1.0f) {
            uint32_t prefix = 0;
            uint64_t above = 0, total = 0;
            double target = 0.0;
            for (int shift = 8; shift >= 0; shift -= 8) {
                rr_clear(sh, true);
                __syncthreads();
    launder<NV>(w);
    #pragma unroll
                for (int v = 0; v < NV; ++v) {
                    uint32_t any = 0;
                    visit8(w[v], [&](uint32_t h, int) { any |= (bf16_key(h) >= kmin) ? 1u : 0u; });
                    if (__any(any)) {
                        visit8(w[v], [&](uint32_t h, int) {
                            const uint32_t key = bf16_key(h);
                            if (key >= kmin && (shift == 8 || (key >> 8) == prefix)) {
                                const float wv = fast_exp2((bf16_bits_to_float(h) - m) * scale);
                                const uint32_t d = ((key >> shift) & 255u) * kCopies + copy;
                                atomicAdd(&sh.hc[d], 1u);
                                const uint64_t wq = fixed_mass(wv, qs);
                                if (wq) atomicAdd(&sh.hm[d], (unsigned long long)wq);
                            }
                        });
                    }
                    SV_VEC_FENCE();
                }
                __syncthreads();
                rr_fold(sh, true);
                __syncthreads();
                if (shift == 8) {
                    // the first level's histogram holds every kept key: its total is the top-k mass
                    uint64_t part = 0;
                    for (int i = tid; i < 256; i += kRrBlock) part += sh.cm[i];
                    total = block_reduce<kRrBlock>(part, OpSumU64{}, (uint64_t)0,
                                                   reinterpret_cast<uint64_t*>(sh.red_i));
                    target = (double)tp * (double)total;
                }
                if (tid < kWave) rr_select(sh, true, 0, above, target);
                __syncthreads();
                prefix = (prefix << 8) | sh.sel_digit;
                above = sh.sel_above;
                if (shift == 0) S = (double)(above + sh.sel_mass) * ldexp(1.0, -qs);
            }
            kmin = prefix;
        } else {
            double ps = 0.0;
    launder<NV>(w);
    #pragma unroll
            for (int v = 0; v < NV; ++v) {
                uint32_t any = 0;
                visit8(w[v], [&](uint32_t h, int) { any |= (bf16_key(h) >= kmin) ? 1u : 0u; });
                if (__any(any)) {
                    visit8(w[v], [&](uint32_t h, int) {
                        if (bf16_key(h) >= kmin) ps += (double)fast_exp2((bf16_bits_to_float(h) - m) * scale);
                    });
                }
                SV_VEC_FENCE();
            }
            S = block_reduce<kRrBlock>(ps, OpSumD{}, 0.0, sh.red_d);
        }
        inv = (float)(1.0 / S);
    }

    // ---- write
launder<NV>(w);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        float o[8];
        uint32_t any = 0;
        if (greedy) {
            const int e0 = ebase(v);
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = (e0 + i == y32) ? 1.0f : 0.0f;
        } else {
        visit8(w[v], [&](uint32_t h, int) { any |= (bf16_key(h) >= kmin) ? 1u : 0u; });
        if (__any(any)) {
            visit8(w[v], [&](uint32_t h, int i) {
                o[i] = (bf16_key(h) >= kmin) ? fast_exp2((bf16_bits_to_float(h) - m) * scale) * inv : 0.0f;
            });
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = 0.0f;
        }
        }
        store8(v, o);
        SV_VEC_FENCE();
    }
}

// Largest register-resident row: 1024 threads x 8 x 20 = 163840 bf16 entries.
constexpr int kRrMaxNV = 20;

template <int NV>
static void launch_rr(dim3 grid, hipStream_t stream, const uint16_t* logits, int64_t B, int npos, int64_t V,
                      const float* temperature, const int32_t* top_k, const float* top_p, const int32_t* req_index,
                      float* out) {
    hipLaunchKernelGGL(softmax_renorm_rr_kernel<NV>, grid, dim3(kRrBlock), 0, stream, logits, B, npos, V,
                       temperature, top_k, top_p, req_index, out);
}

hipError_t launch_softmax_renorm(const void* logits, int dtype, int64_t B, int64_t npos, int64_t V,
                                 const float* temperature, const int32_t* top_k, const float* top_p,
                                 const int32_t* req_index, int64_t n_req, float* probs_out,
                                 hipStream_t stream) {
    const dim3 grid((unsigned)n_req, (unsigned)npos), block(kSmBlock);
    if (dtype == kDtypeBF16 && V <= (int64_t)kRrBlock * 8 * kRrMaxNV) {
        const int64_t nv = (V + kRrBlock * 8 - 1) / (kRrBlock * 8);
        const uint16_t* lg = static_cast<const uint16_t*>(logits);
        const int np = (int)npos;
        if (nv <= 1) launch_rr<1>(grid, stream, lg, B, np, V, temperature, top_k, top_p, req_index, probs_out);
        else if (nv <= 2) launch_rr<2>(grid, stream, lg, B, np, V, temperature, top_k, top_p, req_index, probs_out);
        else if (nv <= 4) launch_rr<4>(grid, stream, lg, B, np, V, temperature, top_k, top_p, req_index, probs_out);
        else if (nv <= 8) launch_rr<8>(grid, stream, lg, B, np, V, temperature, top_k, top_p, req_index, probs_out);
        else if (nv <= 12) launch_rr<12>(grid, stream, lg, B, np, V, temperature, top_k, top_p, req_index, probs_out);
        else if (nv <= 16) launch_rr<16>(grid, stream, lg, B, np, V, temperature, top_k, top_p, req_index, probs_out);
        else launch_rr<20>(grid, stream, lg, B, np, V, temperature, top_k, top_p, req_index, probs_out);
        return hipGetLastError();
    }
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
