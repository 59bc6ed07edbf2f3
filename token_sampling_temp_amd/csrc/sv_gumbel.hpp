// Gumbel-max arithmetic of one vocabulary entry group (4 entries = one
// Philox4x32-10 block), shared by the sampling kernel and the arithmetic
// ceiling probe that measures what this instruction mix can reach.
#pragma once

#include "sv_common.hpp"

namespace sv {

constexpr float kLn2 = 0.6931471805599453f;

// Philox4x32-10 block `block` of stream (seed, subseq) with each 32x32-bit
// product formed once as a 64-bit value (one multiply instruction per
// product instead of separate low and high halves).
__device__ __forceinline__ uint4 philox_block_mad(uint64_t seed, uint64_t subseq, uint64_t block) {
    uint32_t c0 = (uint32_t)block, c1 = (uint32_t)(block >> 32);
    uint32_t c2 = (uint32_t)subseq, c3 = (uint32_t)(subseq >> 32);
    uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c0 = n0;
        c1 = (uint32_t)p1;
        c2 = n2;
        c3 = (uint32_t)p0;
    }
    return make_uint4(c0, c1, c2, c3);
}

// z / T + G for Philox word w: u = (2 (w >> 9) + 1) 2^-24, -ln u and
// -ln(-ln u) through the hardware log2.
__device__ __forceinline__ float gumbel_score(float z, float invT, uint32_t w) {
    const float u = uniform_of(w);
    const float nl = __builtin_amdgcn_logf(u) * -kLn2;   // -ln u > 0
    return fmaf(__builtin_amdgcn_logf(nl), -kLn2, z * invT);
}

// Scores of group g (entries 4g .. 4g+3, those below Vi) folded into the
// thread's (best, bi); entries arrive in increasing index order.  gbase: the
// Philox block of group 0 (a piece of a row that starts at entry 4 gbase).
__device__ __forceinline__ void gumbel_group(const float (&f)[4], int g, int Vi, float invT, uint64_t seed,
                                             uint64_t subseq, float& best, int& bi, int gbase = 0) {
    const int v0 = g * 4;
    const uint4 w = philox_block_mad(seed, subseq, (uint64_t)(g + gbase));
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float sc = gumbel_score(f[e], invT, ws[e]);
        if (v0 + e < Vi && sc > best) {
            best = sc;
            bi = v0 + e;
        }
    }
}

}  // namespace sv
