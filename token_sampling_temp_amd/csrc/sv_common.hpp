// Device helpers shared by the verification kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kWave = 64;
constexpr double kGreedyTemperature = 1e-5;
constexpr uint64_t kRngSlotSpan = 32;

// ----------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
// as 1, 2, 3", SC'11): ten rounds of the 4x32 bijection, key bumped by the
// Weyl constants between rounds.  Key = seed; counter = (block lo, block hi,
// subsequence lo, subsequence hi).
// ----------------------------------------------------------------------------
__device__ __forceinline__ uint4 philox_block(uint64_t seed, uint64_t subseq, uint64_t block) {
    uint32_t c0 = (uint32_t)block, c1 = (uint32_t)(block >> 32);
    uint32_t c2 = (uint32_t)subseq, c3 = (uint32_t)(subseq >> 32);
    uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
        const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
        const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
    }
    return make_uint4(c0, c1, c2, c3);
}

__device__ __forceinline__ uint32_t philox_word(uint64_t seed, uint64_t subseq, uint64_t t) {
    const uint4 b = philox_block(seed, subseq, t >> 2);
    const uint32_t l = (uint32_t)(t & 3);
    return l == 0 ? b.x : (l == 1 ? b.y : (l == 2 ? b.z : b.w));
}

// Odd code 2*(w>>9)+1 in [1, 2^24 - 1]; uniform = code * 2^-24 (exact in float).
__device__ __forceinline__ uint32_t uniform_code(uint32_t w) { return ((w >> 9) << 1) | 1u; }
__device__ __forceinline__ float uniform_of(uint32_t w) {
    return (float)uniform_code(w) * 0x1p-24f;
}

// ----------------------------------------------------------------------------
// Order-preserving 32-bit keys of float values: -0 and +0 map to one key,
// every NaN maps to the largest key.
// ----------------------------------------------------------------------------
__device__ __forceinline__ uint32_t float_key(float f) {
    uint32_t b = __float_as_uint(f);
    if ((b & 0x7FFFFFFFu) == 0u) b = 0u;
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0xFFFFFFFFu;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Packed (key, index) so that a 64-bit max picks the largest key and, among
// equal keys, the lowest index.
__device__ __forceinline__ uint64_t pack_key_index(uint32_t key, int64_t idx) {
    return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}
__device__ __forceinline__ int64_t packed_index(uint64_t packed) {
    return (int64_t)(0xFFFFFFFFu - (uint32_t)(packed & 0xFFFFFFFFull));
}

__device__ __forceinline__ float bf16_to_float(uint16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}

// ----------------------------------------------------------------------------
// Wave (64-lane) and block reductions.  The association order is fixed, so
// floating-point results are reproducible run to run.
// ----------------------------------------------------------------------------
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = op(v, __shfl_xor(v, off, kWave));
    return v;
}

// Raw buffer descriptor (gfx9 family third dword) over num_bytes bytes.  Loads
// through it return zeros, and stores are dropped, at offsets past the end.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes, 0x00020000);
}

// Early-stop signal for a workgroup reading one row.  For a row read at
// memory speed the caller's 64-bit word is polled by wave 0 alone, because a
// wave's vector loads complete in issue order and a poll that waits on a
// contended line would hold back every load issued after it; wave 0 raises a
// flag in LDS that the other waves read.  For a row bound by arithmetic
// (`every_wave`) each wave polls for itself and so stops without first
// spending a round of work.  A poll issued by poll() is consumed by the next
// check().  With a null word nothing stops.
struct RowStop {
    const uint64_t* word;
    uint64_t mask;    // stop once (*word & mask) != 0
    uint32_t* flag;   // LDS word, zero before the row starts
    bool every_wave;
    uint64_t seen;    // the polling wave's last value

    __device__ RowStop(const uint64_t* w, uint64_t m, uint32_t* f, bool every)
        : word(w), mask(m), flag(f), every_wave(every), seen(0) {}
    __device__ __forceinline__ bool polls() const { return every_wave || threadIdx.x < kWave; }
    __device__ __forceinline__ void poll() {
        if (word && polls()) seen = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __device__ __forceinline__ bool check() {
        if (!word) return false;
        if (polls()) {
            const bool f = __builtin_amdgcn_readfirstlane((int)((seen & mask) != 0));
            if (f && !every_wave) __hip_atomic_store(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            return f;
        }
        return __builtin_amdgcn_readfirstlane(
                   (int)__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) != 0;
    }
};

// Workgroup barrier that orders LDS only: it waits for this wave's LDS
// operations, not for its outstanding global loads and stores (a plain
// __syncthreads() waits for those too).  For code whose threads exchange
// data only through LDS.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ----------------------------------------------------------------------------
// Cross-lane steps on the DPP network (register to register, no LDS round
// trip).  Every lane of the wave must be active.  Control codes: quad_perm
// [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E, row_half_mirror = 0x141,
// row_mirror = 0x140, row_shr:n = 0x110 + n.
// ----------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
// Like dpp_u32, but a lane whose source lies outside its row reads 0.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_or0_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL, typename T>
__device__ __forceinline__ T dpp_move(T v) {
    static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
    if constexpr (sizeof(T) == 4) {
        return __builtin_bit_cast(T, dpp_u32<CTRL>(__builtin_bit_cast(uint32_t, v)));
    } else {
        const uint64_t u = __builtin_bit_cast(uint64_t, v);
        const uint64_t r = (uint64_t)dpp_u32<CTRL>((uint32_t)u) | ((uint64_t)dpp_u32<CTRL>((uint32_t)(u >> 32)) << 32);
        return __builtin_bit_cast(T, r);
    }
}
template <int CTRL, typename T>
__device__ __forceinline__ T dpp_move_or0(T v) {
    static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
    if constexpr (sizeof(T) == 4) {
        return __builtin_bit_cast(T, dpp_or0_u32<CTRL>(__builtin_bit_cast(uint32_t, v)));
    } else {
        const uint64_t u = __builtin_bit_cast(uint64_t, v);
        const uint64_t r =
            (uint64_t)dpp_or0_u32<CTRL>((uint32_t)u) | ((uint64_t)dpp_or0_u32<CTRL>((uint32_t)(u >> 32)) << 32);
        return __builtin_bit_cast(T, r);
    }
}
template <typename T>
__device__ __forceinline__ T read_lane(T v, int lane) {
    if constexpr (sizeof(T) == 4) {
        return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
    } else {
        const uint64_t u = __builtin_bit_cast(uint64_t, v);
        const uint64_t r = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane) |
                           ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane) << 32);
        return __builtin_bit_cast(T, r);
    }
}

// Reduction over the 64 lanes with a fixed association order (butterfly in
// each row of 16 lanes, then the four row results in lane order); the result
// is wave-uniform.
template <typename T, typename Op>
__device__ __forceinline__ T wave_allreduce(T v, Op op) {
    v = op(v, dpp_move<0xB1>(v));
    v = op(v, dpp_move<0x4E>(v));
    v = op(v, dpp_move<0x141>(v));
    v = op(v, dpp_move<0x140>(v));
    return op(op(read_lane(v, 0), read_lane(v, 16)), op(read_lane(v, 32), read_lane(v, 48)));
}

// Lane l receives lane l-1's value; lane 0 receives 0 (wave_shr:1).
template <typename T>
__device__ __forceinline__ T wave_shift_up1(T v) {
    return dpp_move_or0<0x138>(v);
}

// Inclusive prefix sum over lanes 0..63 (lane l receives v_0 + ... + v_l);
// `lane` is this thread's lane number.
template <typename T>
__device__ __forceinline__ T wave_inclusive_sum(T v, int lane) {
    v += dpp_move_or0<0x111>(v);
    v += dpp_move_or0<0x112>(v);
    v += dpp_move_or0<0x114>(v);
    v += dpp_move_or0<0x118>(v);
    const T r0 = read_lane(v, 15), r1 = read_lane(v, 31), r2 = read_lane(v, 47);
    T add = 0;
    if (lane >= 16) add += r0;
    if (lane >= 32) add += r1;
    if (lane >= 48) add += r2;
    return v + add;
}

struct OpMaxF {
    __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct OpSumD {
    __device__ double operator()(double a, double b) const { return a + b; }
};
struct OpMaxU64 {
    __device__ uint64_t operator()(uint64_t a, uint64_t b) const { return a > b ? a : b; }
};
struct OpMinI64 {
    __device__ int64_t operator()(int64_t a, int64_t b) const { return a < b ? a : b; }
};
struct OpSumU64 {
    __device__ uint64_t operator()(uint64_t a, uint64_t b) const { return a + b; }
};
struct OpOrU32 {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a | b; }
};

// red must hold BLOCK/64 elements of T.  Every thread receives the result.
template <int BLOCK, typename T, typename Op>
__device__ __forceinline__ T block_reduce(T v, Op op, T identity, T* red) {
    constexpr int W = BLOCK / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    v = wave_reduce(v, op);
    __syncthreads();
    if (lane == 0) red[wid] = v;
    __syncthreads();
    T r = identity;
#pragma unroll
    for (int i = 0; i < W; ++i) r = op(r, red[i]);
    return r;
}

// ----------------------------------------------------------------------------
// Row access.  A row of V elements of type T is split into a scalar head up to
// the first 16-byte boundary, a body of 16-byte vectors and a scalar tail.
// ----------------------------------------------------------------------------
template <typename T>
struct RowSplit {
    int head;        // scalar elements before the first aligned vector
    int64_t nvec;    // aligned 16-byte vectors
    int tail;        // scalar elements after the body
    static constexpr int kEpv = 16 / (int)sizeof(T);
    __device__ RowSplit(const T* row, int64_t V) {
        const uintptr_t a = (uintptr_t)row;
        int64_t h = (int64_t)(((16u - (a & 15u)) & 15u) / sizeof(T));
        if (h > V) h = V;
        head = (int)h;
        nvec = (V - h) / kEpv;
        tail = (int)(V - h - nvec * kEpv);
    }
};

__device__ __forceinline__ float load_elem(const float* p) { return *p; }
__device__ __forceinline__ float load_elem(const uint16_t* p) { return bf16_to_float(*p); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Unpack a 16-byte vector into floats.
__device__ __forceinline__ void unpack(const u32x4 v, float (&f)[4]) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ void unpack(const u32x4 v, float (&f)[8]) {
    f[0] = __uint_as_float(v.x << 16);
    f[1] = __uint_as_float(v.x & 0xFFFF0000u);
    f[2] = __uint_as_float(v.y << 16);
    f[3] = __uint_as_float(v.y & 0xFFFF0000u);
    f[4] = __uint_as_float(v.z << 16);
    f[5] = __uint_as_float(v.z & 0xFFFF0000u);
    f[6] = __uint_as_float(v.w << 16);
    f[7] = __uint_as_float(v.w & 0xFFFF0000u);
}

// 16-byte vector load; NT = non-temporal (data read once, keep it out of the caches).
template <bool NT, typename T>
__device__ __forceinline__ u32x4 load_vec(const T* base, int64_t i) {
    const u32x4* p = reinterpret_cast<const u32x4*>(base) + i;
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

// Largest "magnitude bits" seen, used to detect NaN in a row cheaply:
// a float row holds a NaN iff max(bits & 0x7FFFFFFF) > 0x7F800000; a bf16 row
// iff either 16-bit half of the packed max exceeds 0x7F80.
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    const u16x2 x = __builtin_bit_cast(u16x2, a);
    const u16x2 y = __builtin_bit_cast(u16x2, b);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}
__device__ __forceinline__ uint32_t mag_acc(uint32_t acc, const u32x4 v, float) {
    const uint32_t m = 0x7FFFFFFFu;
    acc = max(acc, max(v.x & m, v.y & m));
    return max(acc, max(v.z & m, v.w & m));
}
__device__ __forceinline__ uint32_t mag_acc(uint32_t acc, const u32x4 v, uint16_t) {
    const uint32_t m = 0x7FFF7FFFu;
    acc = pk_max_u16(acc, pk_max_u16(v.x & m, v.y & m));
    return pk_max_u16(acc, pk_max_u16(v.z & m, v.w & m));
}
__device__ __forceinline__ uint32_t mag_acc_scalar(uint32_t acc, float f, float) {
    return max(acc, __float_as_uint(f) & 0x7FFFFFFFu);
}
__device__ __forceinline__ uint32_t mag_acc_scalar(uint32_t acc, float f, uint16_t) {
    return pk_max_u16(acc, (__float_as_uint(f) >> 16) & 0x7FFFu);
}
__device__ __forceinline__ bool mag_has_nan(uint32_t acc, float) { return acc > 0x7F800000u; }
__device__ __forceinline__ bool mag_has_nan(uint32_t acc, uint16_t) {
    return (acc & 0xFFFFu) > 0x7F80u || (acc >> 16) > 0x7F80u;
}

// Visit every element of a row once, in a fixed thread-to-element mapping:
// f(value, index).  Each thread sees its elements in increasing index order.
template <int BLOCK, bool NT, typename T, typename F>
__device__ __forceinline__ void row_foreach(const T* row, int64_t V, F&& f) {
    constexpr int E = RowSplit<T>::kEpv;
    const RowSplit<T> s(row, V);
    const int tid = threadIdx.x;
    if (tid < s.head) f(load_elem(row + tid), (int64_t)tid);
    const T* body = row + s.head;
    int64_t i = tid;
    for (; i + BLOCK < s.nvec; i += 2 * BLOCK) {
        const u32x4 a = load_vec<NT>(body, i);
        const u32x4 b = load_vec<NT>(body, i + BLOCK);
        float fa[E], fb[E];
        unpack(a, fa);
        unpack(b, fb);
#pragma unroll
        for (int e = 0; e < E; ++e) f(fa[e], s.head + i * E + e);
#pragma unroll
        for (int e = 0; e < E; ++e) f(fb[e], s.head + (i + BLOCK) * E + e);
    }
    if (i < s.nvec) {
        const u32x4 a = load_vec<NT>(body, i);
        float fa[E];
        unpack(a, fa);
#pragma unroll
        for (int e = 0; e < E; ++e) f(fa[e], s.head + i * E + e);
    }
    if (tid < s.tail) {
        const int64_t idx = s.head + s.nvec * E + tid;
        f(load_elem(row + idx), idx);
    }
}

}  // namespace sv
