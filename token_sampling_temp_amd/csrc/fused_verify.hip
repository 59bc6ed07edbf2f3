// Fused verify: target probabilities from logits (temperature softmax, then
// top-k, then top-p renormalisation) and chain rejection of a linear draft in
// one launch, without writing the probabilities.
//
// One 1024-thread workgroup per request walks the target rows j = 0..D in
// order.  For row j it computes the row's statistics with the softmax kernels'
// own row algorithms (register-resident for bf16 rows that fit, streamed
// otherwise, the argmax for one-hot rows), evaluates p_j at the draft id x_j
// and stops at the first rejection, so only logit rows 0..L are read.  The
// residual max(0, p_L - q_L) (or the bonus row p_D) is then drawn by inverse
// CDF over ascending vocabulary index: double sums per 1024-entry chunk,
// prefix over the chunk sums, search inside the chosen chunk.  Probability
// values, chunk sums, their order and the search are those of softmax_renorm
// followed by chain_reject (with a 16-byte aligned probability buffer), so the
// two paths return the same tokens.
#include <type_traits>

#include "sv_draw.hpp"
#include "sv_launch.hpp"
#include "sv_rowpar.hpp"
#include "sv_softmax.hpp"

namespace sv {

constexpr int kFvBlock = 1024;
static_assert(kFvBlock == kRrBlock && kFvBlock == kSmBlock, "one block size for every row algorithm");
constexpr int kFvWaves = kFvBlock / kWave;
constexpr int64_t kFvChunk = 1024;   // entries per chunk sum
constexpr int kFvMaxChunks = 512;    // V <= 524288

constexpr int kCompactCap = kFvBlock;   // kept entries a compacted draw handles (one per thread)

struct FusedShared {
    RrShared rr;                  // histogram / probability table / streamed and argmax state
    double chunk[kFvMaxChunks];   // chunk sums of the drawn row
    // compacted draw: the kept entries of a register-resident row
    uint64_t clist[kCompactCap];  // (index << 16) | key, in arrival order
    uint32_t cidx[kCompactCap];   // indices, ascending
    float cp[kCompactCap];        // target probabilities, same order
    float cq[kCompactCap];        // draft probabilities at the same indices (residual draws)
    double wsum[kFvWaves];        // per-wave totals of the block scan
    int32_t whit[kFvWaves];       // per-wave counts, then first crossing / last positive entry
    int32_t xs[kMaxDraft];        // draft ids
    float qx[kMaxDraft];          // q_i(x_i), 0 for an id outside [0, V)
    uint32_t zx[kMaxDraft];       // bits of the logit z_i(x_i)
    uint32_t code[kMaxDraft + 1]; // uniform codes: accept tests 0..D-1, final draw D
    int acc;
    int64_t y;
};

// How one row's probabilities are evaluated.
enum : int { kProbOneHot = 0, kProbTable = 1, kProbRrExp = 2, kProbStreamed = 3 };
struct RowProb {
    int mode;
    float m, scale, inv;
    uint32_t kmin;
    int64_t y;                  // one-hot index
    double thr = -INFINITY;     // streamed rows: min-p threshold on v - m (single-step sampling)
};

__device__ __forceinline__ float raw_value(uint16_t h) { return bf16_to_float(h); }
__device__ __forceinline__ float raw_value(float f) { return f; }

// Probability of entry idx whose logit has the bits `raw`: the value the
// softmax kernels write for it under the same statistics.
template <typename T>
__device__ __forceinline__ float row_prob(const RowProb rp, const RrShared& sh, T raw, int64_t idx) {
    if (rp.mode == kProbOneHot) return idx == rp.y ? 1.0f : 0.0f;
    if constexpr (sizeof(T) == 2) {
        if (rp.mode == kProbTable || rp.mode == kProbRrExp) {
            const uint32_t key = keys_of_pair((uint32_t)raw) & 0xFFFFu;
            if (rp.mode == kProbTable) return sh.u.lut[max((int)key + 1 - (int)rp.kmin, 0)];
            return key >= rp.kmin ? fast_exp2((key_to_float(key) - rp.m) * rp.scale) * rp.inv : 0.0f;
        }
    }
    const float v = raw_value(raw);
    return (logit_key<T>(v) >= rp.kmin && (double)v - (double)rp.m >= rp.thr) ? exp2f((v - rp.m) * rp.scale) * rp.inv
                                                                               : 0.0f;
}

// Four consecutive logits starting at idx (a multiple of 4); entries past V
// read as 0 bits (their probability is forced to 0 by the caller).
template <typename T>
__device__ __forceinline__ void load_raw4(const T* row, int64_t idx, int64_t V, bool vec_ok, T (&r)[4]) {
    if (vec_ok && idx + 3 < V) {
        if constexpr (sizeof(T) == 2) {
            const uint2 u = *reinterpret_cast<const uint2*>(row + idx);
            r[0] = (uint16_t)(u.x & 0xFFFFu);
            r[1] = (uint16_t)(u.x >> 16);
            r[2] = (uint16_t)(u.y & 0xFFFFu);
            r[3] = (uint16_t)(u.y >> 16);
        } else {
            const float4 f = *reinterpret_cast<const float4*>(row + idx);
            r[0] = f.x;
            r[1] = f.y;
            r[2] = f.z;
            r[3] = f.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = idx + e < V ? row[idx + e] : T{};
    }
}

__device__ __forceinline__ void load_q4(const float* row, int64_t idx, int64_t V, bool vec_ok, float (&f)[4]) {
    if (vec_ok && idx + 3 < V) {
        unpack(load_vec<false>(row + idx, 0), f);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) f[e] = idx + e < V ? row[idx + e] : 0.0f;
    }
}

// Probability of a kept key under register-resident statistics: the value
// row_prob gives the logit with that key.
__device__ __forceinline__ float key_prob(const RowProb rp, const RrShared& sh, uint32_t key) {
    if (rp.mode == kProbTable) return sh.u.lut[max((int)key + 1 - (int)rp.kmin, 0)];
    return key >= rp.kmin ? fast_exp2((key_to_float(key) - rp.m) * rp.scale) * rp.inv : 0.0f;
}

// Inverse-CDF draw of one index from r_v = max(0, p_v - q_v) (resid) or p_v,
// p given by rp on the logit row zr.  Whole workgroup; returns -1 when the
// weights have no positive mass.  Chunk c of 1024 entries is summed by one
// wave as four sub-tiles of 64 lanes x 4 consecutive entries (lane sums of
// four, then the sub-tiles in order, then the 64 lanes), wave 0 picks the
// chunk holding u_f * R and scans it in index order.
template <typename T, bool RESID>
__device__ __forceinline__ int64_t fused_draw(FusedShared& sh, const RowProb rp, const T* __restrict__ zr,
                              const float* __restrict__ qr, int64_t V, double uf) {
    constexpr bool resid = RESID;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
    const bool zvec = (uintptr_t)zr % (4 * sizeof(T)) == 0;
    const bool qvec = !resid || (uintptr_t)qr % 16 == 0;
    const int nch = (int)((V + kFvChunk - 1) / kFvChunk);
    auto weights = [&](int64_t idx, double (&r)[4]) {
        T z[4];
        float qf[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        load_raw4<T>(zr, idx, V, zvec, z);
        if constexpr (RESID) load_q4(qr, idx, V, qvec, qf);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float pv = idx + e < V ? row_prob<T>(rp, sh.rr, z[e], idx + e) : 0.0f;
            r[e] = rval(pv, qf[e], resid);
        }
    };
    // acc = sum over sub-tiles k (in order) of the lane's sum of four
    auto publish = [&](double acc, int c) {
        acc = wave_allreduce(acc, OpSumD{});
        if (lane == 0) sh.chunk[c] = acc;
    };
    // chunks wholly inside the row, with aligned rows: unconditional vector
    // loads, two chunks of a wave in flight (wave w takes w, w + 16, ...)
    const int nfull = (int)(V / kFvChunk);
    int cdone = 0;   // chunks below this are summed
    if constexpr (!RESID && sizeof(T) == 2) {
        // bf16 rows without draft probabilities, 16-byte aligned: buffer loads
        // of 16 bytes (8 entries per lane, two per chunk), four chunks of a
        // wave in flight, every chunk including a partial last one; entries
        // past the row read zeros and are left out.  (Chunk sums are taken
        // over the same entries in another order than below; only their
        // rounding differs.)
        if ((uintptr_t)zr % 16 == 0) {
            constexpr int kDep = 4;
            const int nr = nch > wid ? (nch - wid + kFvWaves - 1) / kFvWaves : 0;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(zr, (uint32_t)(V * 2));
            u32x4 zb[kDep][2];
            auto ld = [&](int slot, int r) {
                const uint32_t base = (uint32_t)(wid + r * kFvWaves) * (uint32_t)(kFvChunk * 2) + (uint32_t)lane * 16u;
                zb[slot][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, base, 0, 0));
                zb[slot][1] =
                    __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, base + kFvChunk, 0, 0));
            };
            // register-resident statistics: one key conversion per pair of logits
            const bool by_key = rp.mode == kProbTable || rp.mode == kProbRrExp;
            // guard: the row's last, partial chunk (entries at or past V left
            // out); each call below passes a constant
            auto sum_chunk = [&](int slot, int c, bool guard) {
                double acc = 0.0;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t wd[4] = {zb[slot][h].x, zb[slot][h].y, zb[slot][h].z, zb[slot][h].w};
                    const int64_t i0 = (int64_t)c * kFvChunk + h * (kFvChunk / 2) + lane * 8;
                    double s8 = 0.0;
                    if (by_key) {
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            const uint32_t k2 = keys_of_pair(wd[d]);
                            if (!guard || i0 + 2 * d < V) s8 += (double)key_prob(rp, sh.rr, k2 & 0xFFFFu);
                            if (!guard || i0 + 2 * d + 1 < V) s8 += (double)key_prob(rp, sh.rr, k2 >> 16);
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (!guard || i0 + e < V)
                                s8 += (double)row_prob<T>(rp, sh.rr, (uint16_t)(wd[e >> 1] >> (16 * (e & 1))), i0 + e);
                    }
                    acc += s8;
                }
                publish(acc, c);
            };
            auto sum = [&](int slot, int r) {
                const int c = wid + r * kFvWaves;
                if (c < nfull) sum_chunk(slot, c, false);
                else sum_chunk(slot, c, true);
            };
#pragma unroll
            for (int j = 0; j < kDep; ++j) ld(j, j);
            for (int r0 = 0; r0 < nr; r0 += kDep) {
#pragma unroll
                for (int j = 0; j < kDep; ++j) {
                    if (r0 + j < nr) sum(j, r0 + j);
                    ld(j, r0 + j + kDep);
                }
            }
            cdone = nch;
        }
    }
    if (cdone == 0 && zvec && qvec) {
        typedef typename std::conditional<sizeof(T) == 2, uint2, float4>::type ZV;
        ZV zb[2][4];
        u32x4 qb[2][4];
        const int nr = nfull > wid ? (nfull - wid + kFvWaves - 1) / kFvWaves : 0;
        auto ld = [&](int slot, int r) {
            const int64_t base = (int64_t)(wid + r * kFvWaves) * kFvChunk + lane * 4;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                zb[slot][k] = *reinterpret_cast<const ZV*>(zr + base + k * kWave * 4);
                if constexpr (RESID) qb[slot][k] = load_vec<false>(qr + base + k * kWave * 4, 0);
            }
        };
        auto sum = [&](int slot, int r) {
            const int c = wid + r * kFvWaves;
            double acc = 0.0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                T z[4];
                if constexpr (sizeof(T) == 2) {
                    z[0] = (uint16_t)(zb[slot][k].x & 0xFFFFu);
                    z[1] = (uint16_t)(zb[slot][k].x >> 16);
                    z[2] = (uint16_t)(zb[slot][k].y & 0xFFFFu);
                    z[3] = (uint16_t)(zb[slot][k].y >> 16);
                } else {
                    z[0] = zb[slot][k].x;
                    z[1] = zb[slot][k].y;
                    z[2] = zb[slot][k].z;
                    z[3] = zb[slot][k].w;
                }
                float qf[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if constexpr (RESID) unpack(qb[slot][k], qf);
                const int64_t i0 = (int64_t)c * kFvChunk + (k * kWave + lane) * 4;
                double s4 = 0.0;
#pragma unroll
                for (int e = 0; e < 4; ++e) s4 += rval(row_prob<T>(rp, sh.rr, z[e], i0 + e), qf[e], resid);
                acc += s4;
            }
            publish(acc, c);
        };
        if (nr >= 4) {
            ld(0, 0);
            ld(1, 1);
            int r0 = 0;
            for (; r0 + 4 <= nr; r0 += 2) {
                __builtin_amdgcn_sched_barrier(0);
                sum(0, r0);
                __builtin_amdgcn_sched_barrier(0);
                ld(0, r0 + 2);
                __builtin_amdgcn_sched_barrier(0);
                sum(1, r0 + 1);
                __builtin_amdgcn_sched_barrier(0);
                ld(1, r0 + 3);
            }
            // rounds r0, r0 + 1 are in flight; at most one remains after them
            sum(0, r0);
            if (r0 + 2 < nr) ld(0, r0 + 2);
            sum(1, r0 + 1);
            if (r0 + 2 < nr) sum(0, r0 + 2);
        } else {
            for (int r = 0; r < nr; ++r) {
                ld(0, r);
                sum(0, r);
            }
        }
        cdone = nfull;
    }
    // the rest (a partial last chunk, or every chunk of an unaligned row)
    for (int c = cdone + wid; c < nch; c += kFvWaves) {
        double acc = 0.0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            double r[4];
            weights((int64_t)c * kFvChunk + (k * kWave + lane) * 4, r);
            double s4 = 0.0;
#pragma unroll
            for (int e = 0; e < 4; ++e) s4 += r[e];
            acc += s4;
        }
        publish(acc, c);
    }
    __syncthreads();
    if (wid == 0) {
        double R, base;
        int force_last;
        const int cstar = wave_pick(nch, [&](int i) { return sh.chunk[i]; }, R, uf, base, force_last);
        int64_t y = -1;
        if (cstar >= 0) {
            const int64_t cb = (int64_t)cstar * kFvChunk;
            double r[4][4];
#pragma unroll
            for (int k = 0; k < 4; ++k) weights(cb + (k * kWave + lane) * 4, r[k]);
            int64_t mylast = -1;
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (r[k][e] > 0.0) mylast = cb + (k * kWave + lane) * 4 + e;
            const int64_t lastpos = wave_allreduce(mylast, [](int64_t a, int64_t b) { return a > b ? a : b; });
            if (!force_last) {
                const double Tt = uf * R;
                double run = base;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    if (y >= 0) continue;   // wave-uniform
                    const double s = ((r[k][0] + r[k][1]) + r[k][2]) + r[k][3];
                    const double incl = wave_incl_scan(s);
                    const double excl = wave_shift_up1(incl);
                    const uint64_t hit = __ballot(run + incl > Tt && s > 0.0);
                    if (hit) {
                        const int ls = __ffsll((unsigned long long)hit) - 1;
                        int64_t cand = -1;
                        if (lane == ls) {
                            const int64_t i0 = cb + (k * kWave + lane) * 4;
                            double xr = run + excl;
                            int last_e = -1;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                if (cand >= 0) continue;
                                if (r[k][e] > 0.0) last_e = e;
                                xr += r[k][e];
                                if (r[k][e] > 0.0 && xr > Tt) cand = i0 + e;
                            }
                            if (cand < 0) cand = i0 + last_e;
                        }
                        y = read_lane(cand, ls);
                    } else {
                        run += read_lane(incl, kWave - 1);
                    }
                }
            }
            if (y < 0) y = lastpos;
        }
        if (lane == 0) sh.y = y;
    }
    __syncthreads();
    return sh.y;
}


struct CompactDraw {
    int64_t y;   // the drawn index, -1 when the weights have no positive mass
    bool used;   // false: nothing drawn (too many vectors or kept entries)
};

// The draw of compact_draw over n listed kept entries (sh.clist, any order):
// rank by index while the draft probabilities are gathered, one block-wide
// scan of the weights in index order, and the first crossing of u_f * R.
// Whole workgroup.
__device__ __forceinline__ CompactDraw draw_listed(FusedShared& sh, const RowProb rp, uint32_t n,
                                                   const float* __restrict__ qr, double uf, int tid) {
    const int lane = tid & (kWave - 1), wid = tid / kWave;
    // ---- rank by index; gather the draft probabilities meanwhile
    if ((uint32_t)tid < n) {
        const uint64_t e = sh.clist[tid];
        const uint32_t idx = (uint32_t)(e >> 16);
        const float qv = qr ? qr[idx] : 0.0f;   // waited for only after the ranking loop
        uint32_t rank = 0;
        const uint32_t n2 = n & ~1u;
        for (uint32_t j = 0; j < n2; j += 2) {
            const uint64_t a = sh.clist[j], c = sh.clist[j + 1];
            rank += (a < e ? 1u : 0u) + (c < e ? 1u : 0u);
        }
        if (n & 1u) rank += sh.clist[n - 1] < e ? 1u : 0u;
        sh.cidx[rank] = idx;
        sh.cp[rank] = key_prob(rp, sh.rr, (uint32_t)(e & 0xFFFFu));
        sh.cq[rank] = qv;
    }
    lds_barrier();
    // ---- block-wide inclusive scan of the weights in index order
    const bool in = (uint32_t)tid < n;
    const double r = in ? rval(sh.cp[tid], sh.cq[tid], qr != nullptr) : 0.0;
    const double winc = wave_inclusive_sum(r, lane);
    if (lane == kWave - 1) sh.wsum[wid] = winc;
    lds_barrier();
    double off = 0.0, R = 0.0;
#pragma unroll
    for (int i = 0; i < kFvWaves; ++i) {
        const double t = sh.wsum[i];
        if (i < wid) off += t;
        R += t;
    }
    if (!(R > 0.0)) return CompactDraw{-1, true};   // uniform
    const double T = uf * R;
    const double incl = off + winc;
    const uint64_t hit = __ballot(in && r > 0.0 && incl > T);
    const uint64_t posv = __ballot(in && r > 0.0);
    // per wave: the first crossing (>= 0), else -2 - its last positive entry,
    // else -1
    if (lane == 0) {
        sh.whit[wid] = hit    ? wid * kWave + (__ffsll((unsigned long long)hit) - 1)
                       : posv ? -2 - (wid * kWave + (63 - __clzll((unsigned long long)posv)))
                              : -1;
    }
    lds_barrier();
    int first = -1, last = -1;
#pragma unroll
    for (int i = 0; i < kFvWaves; ++i) {
        const int h = sh.whit[i];
        if (h >= 0 && first < 0) first = h;
        if (h <= -2) last = -2 - h;   // waves in order: the last one seen is the largest
    }
    // no crossing: rounding left T beyond every partial sum, so the draw is
    // the last positive entry
    const int t = first >= 0 ? first : last;
    return CompactDraw{t >= 0 ? (int64_t)sh.cidx[t] : -1, true};
}

// Inverse-CDF draw over the kept entries of a register-resident row: every
// weight outside the kept set (keys below kmin) is zero, for the bonus draw
// (p) and the residual (max(0, p - q)) alike, so only the kept entries are
// visited.  The statistics pass recorded each thread vector's largest key
// (vmax); the vectors whose largest key reaches kmin are listed, one thread
// per listed vector re-reads it (16 bytes) and appends its kept entries
// (index, key) to LDS, the entries are ranked by index (each counts the
// smaller indices, reading the list as LDS broadcasts), the draft
// probabilities are gathered at the kept indices only (issued before the
// ranking, so the gather overlaps it), and one block-wide scan in index
// order finds y = min{ j : sum_{v <= j} r_v > u_f * R }.  Whole workgroup.
// Nothing is drawn (used = false) when more than kCompactCap vectors or kept
// entries would be involved.
template <int NV>
__device__ __forceinline__ CompactDraw compact_draw(FusedShared& sh, const RowProb rp,
                                                    const uint16_t* __restrict__ row,
                                                    const uint32_t (&vmax)[(NV + 1) / 2], int64_t V,
                                                    const float* __restrict__ qr, double uf, int tid) {
    const int lane = tid & (kWave - 1), wid = tid / kWave;
    const uint32_t kmin = rp.kmin;
    // block-wide exclusive scan of per-thread counts through sh.whit
    auto block_offsets = [&](uint32_t c, uint32_t& total) {
        const uint32_t inc = wave_inclusive_sum(c, lane);
        lds_barrier();   // earlier readers of whit are done
        if (lane == kWave - 1) sh.whit[wid] = (int32_t)inc;
        lds_barrier();
        uint32_t off = inc - c;
        total = 0;
#pragma unroll
        for (int i = 0; i < kFvWaves; ++i) {
            const uint32_t t = (uint32_t)sh.whit[i];
            if (i < wid) off += t;
            total += t;
        }
        return off;
    };
    // ---- the vectors that hold kept keys
    uint32_t nvq = 0;
#pragma unroll
    for (int v = 0; v < NV; ++v) nvq += ((vmax[v >> 1] >> (16 * (v & 1))) & 0xFFFFu) >= kmin ? 1u : 0u;
    uint32_t Q;
    uint32_t vpos = block_offsets(nvq, Q);
    if (!(Q > 0 && Q <= (uint32_t)kCompactCap)) return CompactDraw{-1, false};   // uniform
#pragma unroll
    for (int v = 0; v < NV; ++v)
        if (((vmax[v >> 1] >> (16 * (v & 1))) & 0xFFFFu) >= kmin) sh.cidx[vpos++] = (uint32_t)(v * kRrBlock + tid);
    lds_barrier();
    // ---- one listed vector per thread: re-read, count and append its kept entries
    const __amdgpu_buffer_rsrc_t rin = make_rsrc(row, (uint32_t)(V * 2));
    uint32_t keys[4] = {0u, 0u, 0u, 0u}, cnt = 0, vid = 0;
    if ((uint32_t)tid < Q) {
        vid = sh.cidx[tid];
        const u32x4 x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rin, vid * 16, 0, 0));
        keys[0] = keys_of_pair(x.x);
        keys[1] = keys_of_pair(x.y);
        keys[2] = keys_of_pair(x.z);
        keys[3] = keys_of_pair(x.w);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t key = (keys[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
            cnt += (key >= kmin && (int64_t)vid * 8 + i < V) ? 1u : 0u;
        }
    }
    uint32_t n;
    uint32_t epos = block_offsets(cnt, n);
    if (!(n > 0 && n <= (uint32_t)kCompactCap)) return CompactDraw{-1, false};   // uniform
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t key = (keys[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
        const int64_t idx = (int64_t)vid * 8 + i;
        if (cnt && key >= kmin && idx < V) sh.clist[epos++] = ((uint64_t)idx << 16) | key;
    }
    lds_barrier();
    return draw_listed(sh, rp, n, qr, uf, tid);
}

// compact_draw for a row still held in registers (w: rr_stats' keys, NV
// vectors per thread): each thread scans only its vectors whose largest key
// (vmax) reaches kmin and appends their kept entries, so no vector is read
// again.
template <int NV>
__device__ __forceinline__ CompactDraw compact_draw_regs(FusedShared& sh, const RowProb rp, const u32x4 (&w)[NV],
                                                         const uint32_t (&vmax)[(NV + 1) / 2], int64_t V,
                                                         const float* __restrict__ qr, double uf, int tid) {
    const int lane = tid & (kWave - 1), wid = tid / kWave;
    const uint32_t kmin = rp.kmin;
    auto hot = [&](int v) { return ((vmax[v >> 1] >> (16 * (v & 1))) & 0xFFFFu) >= kmin; };
    auto key_at = [&](int v, int i) {
        const uint32_t wd = i < 2 ? w[v].x : (i < 4 ? w[v].y : (i < 6 ? w[v].z : w[v].w));
        return (wd >> (16 * (i & 1))) & 0xFFFFu;
    };
    // whole vectors lie inside the row or past its end (V is a multiple of 8)
    auto inside = [&](int v) { return (int64_t)(v * kRrBlock + tid) * 8 < V; };
    uint32_t cnt = 0;
#pragma unroll
    for (int v = 0; v < NV; ++v)
        if (hot(v) && inside(v)) {
#pragma unroll
            for (int i = 0; i < 8; ++i) cnt += key_at(v, i) >= kmin ? 1u : 0u;
        }
    // block-wide exclusive scan of the counts through sh.whit
    const uint32_t inc = wave_inclusive_sum(cnt, lane);
    lds_barrier();   // earlier readers of whit are done
    if (lane == kWave - 1) sh.whit[wid] = (int32_t)inc;
    lds_barrier();
    uint32_t epos = inc - cnt, n = 0;
#pragma unroll
    for (int i = 0; i < kFvWaves; ++i) {
        const uint32_t t = (uint32_t)sh.whit[i];
        if (i < wid) epos += t;
        n += t;
    }
    if (!(n > 0 && n <= (uint32_t)kCompactCap)) return CompactDraw{-1, false};   // uniform
#pragma unroll
    for (int v = 0; v < NV; ++v)
        if (hot(v) && inside(v)) {
            const uint32_t base = (uint32_t)(v * kRrBlock + tid) * 8u;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t key = key_at(v, i);
                if (key >= kmin) sh.clist[epos++] = ((uint64_t)(base + i) << 16) | key;
            }
        }
    lds_barrier();
    return draw_listed(sh, rp, n, qr, uf, tid);
}

// NV > 0: bf16 logits whose rows are 16-byte aligned with V a multiple of 8
// and V <= 8192 * NV take the register-resident statistics (as the softmax
// kernel does); NV = 0: streamed statistics for every temperature row.
template <typename T, int NV>
__global__ __launch_bounds__(kFvBlock) void verify_fused_kernel(
    const T* __restrict__ logits, const float* __restrict__ temperature, const int32_t* __restrict__ top_k,
    const float* __restrict__ top_p, const float* __restrict__ q, const int32_t* __restrict__ x,
    const uint64_t* __restrict__ seed, const uint64_t* __restrict__ offset, int64_t B, int D, int64_t V,
    const int32_t* __restrict__ req_index, int32_t* __restrict__ accepted, int32_t* __restrict__ accept_len) {
    __shared__ FusedShared sh;
    const int64_t b = req_index ? (int64_t)req_index[blockIdx.x] : (int64_t)blockIdx.x;
    if (b < 0 || b >= B) return;   // uniform over the workgroup
    const int N = D + 1;
    const int tid = threadIdx.x;
    const float Tm = temperature[b];
    const int32_t k = top_k ? top_k[b] : 0;
    const float tp = top_p ? top_p[b] : 1.0f;

    // draft ids, q at the ids and the uniform codes, read once
    if (tid <= D) {
        sh.code[tid] = uniform_code(philox_word(seed[b], offset[b], (uint64_t)tid));
        if (tid < D) {
            const int32_t xi = x[b * D + tid];
            sh.xs[tid] = xi;
            const bool inr = xi >= 0 && (int64_t)xi < V;
            sh.qx[tid] = inr ? q[(b * D + tid) * V + xi] : 0.0f;
            T zv{};
            if (inr) zv = logits[(b * N + tid) * V + xi];
            uint32_t bits = 0;
            __builtin_memcpy(&bits, &zv, sizeof(T));
            sh.zx[tid] = bits;
        }
    }
    __syncthreads();

    // ---- rows 0..L: statistics, then the accept test at the draft id.  The
    // row where the chain stops (a rejection, or the bonus row D) is drawn
    // from; a register-resident row with a small kept set is drawn right
    // here, from the keys still in registers.
    const double uf = (double)sh.code[D] * 0x1p-24;
    RowProb rp{kProbOneHot, 0.0f, 0.0f, 0.0f, 0u, 0};
    int L = D;
    bool drawn = false;
    int64_t y = -1;
    // accept test at position j (block-uniform result)
    auto accepted_at = [&](int j) {
        if (tid == 0) {
            const int32_t xj = sh.xs[j];
            bool ok = false;
            if (xj >= 0 && (int64_t)xj < V) {
                T zv;
                const uint32_t bits = sh.zx[j];
                __builtin_memcpy(&zv, &bits, sizeof(T));
                const float pv = row_prob<T>(rp, sh.rr, zv, xj);
                ok = (double)((float)sh.code[j] * 0x1p-24f) * (double)sh.qx[j] < (double)pv;
            }
            sh.acc = ok ? 1 : 0;
        }
        __syncthreads();
        return sh.acc != 0;
    };
    for (int j = 0; j <= D; ++j) {
        const T* row = logits + ((int64_t)b * N + j) * V;
        bool stop = false, done = false;
        // the thread index is made opaque per row, so nothing derived from it
        // is hoisted out of the row loop and held in registers across rows
        int rtid = threadIdx.x;
        asm volatile("" : "+v"(rtid));
        if ((double)Tm < kGreedyTemperature) {
            __syncthreads();   // the previous row's table may still be read
            rp.mode = kProbOneHot;
            rp.y = row_argmax<kFvBlock, false>(row, V, sh.rr.u.sm.am);
        } else {
            if constexpr (NV > 0) {
                u32x4 w[NV];
                uint32_t vmax[(NV + 1) / 2];
                RrStats st;
                const uint16_t* row16 = reinterpret_cast<const uint16_t*>(row);
                if (rr_stats<NV, false, true>(sh.rr, row16, V, Tm, k, tp, rtid, w, st, 0.0f, vmax)) {
                    rp = RowProb{st.table ? kProbTable : kProbRrExp, st.m, st.scale, st.inv, st.kmin, 0};
                    done = true;
                    stop = j == D || !accepted_at(j);
                    if (stop) {
                        // a small kept set is drawn by revisiting only the vectors that hold it
                        const float* qj = j < D ? q + ((int64_t)b * D + j) * V : nullptr;
                        CompactDraw cd = compact_draw<NV>(sh, rp, row16, vmax, V, qj, uf, rtid);
                        // an empty residual falls back to the target row
                        if (cd.used && cd.y < 0 && qj) cd = compact_draw<NV>(sh, rp, row16, vmax, V, nullptr, uf, rtid);
                        y = cd.y;
                        drawn = cd.used;
                    }
                }
            }
            if (!done) {
                __syncthreads();
                const StreamStats ss = streamed_stats<T>(row, V, Tm, k, tp, sh.rr.u.sm);
                rp = RowProb{kProbStreamed, ss.m, ss.scale, ss.inv, ss.kmin, 0};
            }
        }
        if (!done) stop = j == D || !accepted_at(j);
        if (stop) {
            L = j;
            break;
        }
    }

    // ---- otherwise draw from row L's residual (or the bonus row) by
    // re-reading it, then from the target row, then floor(u_f * V)
    const bool resid = L < D;
    const T* zr = logits + ((int64_t)b * N + L) * V;
    const float* qr = resid ? q + ((int64_t)b * D + L) * V : nullptr;
    if (!drawn) {
        y = resid ? fused_draw<T, true>(sh, rp, zr, qr, V, uf) : fused_draw<T, false>(sh, rp, zr, nullptr, V, uf);
        if (y < 0 && resid) y = fused_draw<T, false>(sh, rp, zr, nullptr, V, uf);
    }
    if (y < 0) y = (int64_t)(((uint64_t)sh.code[D] * (uint64_t)V) >> 24);
    if (tid < N) {
        int32_t t;
        if (tid < L) t = sh.xs[tid];
        else t = (tid == L) ? (int32_t)y : -1;
        accepted[b * N + tid] = t;
    }
    if (tid == 0) accept_len[b] = L;
}

// Fused verify, one workgroup per row (request, j), rows dispatched in row
// order (every request's row 0 first): a request's rows are evaluated side
// by side instead of one after another.  When the rows outnumber the CUs
// (skip_ended), a row whose request already has an ended row before it is
// only counted in (its result cannot be used).  Each workgroup
// computes row j's statistics and accept test exactly as verify_fused_kernel
// does; a row that rejects (or the bonus row D) also draws its token, as it
// would if the chain stopped there.  Rows meet through the request's line of
// the workspace (sv_rowpar.hpp): each stores its drawn token and counts
// itself in, flagging the chain's end if it rejected or is row D; the last
// workgroup takes L = the first flagged row and writes x_0..x_{L-1}, the
// token row L drew, then -1.  Rows after L may be read although the serial
// kernel would stop before them; the results are bit-identical to it.  A
// request listed twice has a line per listing and gets the same outputs
// twice.
template <typename T, int NV>
__global__ __launch_bounds__(kFvBlock) void verify_fused_rows_kernel(
    const T* __restrict__ logits, const float* __restrict__ temperature, const int32_t* __restrict__ top_k,
    const float* __restrict__ top_p, const float* __restrict__ q, const int32_t* __restrict__ x,
    const uint64_t* __restrict__ seed, const uint64_t* __restrict__ offset, int64_t B, int D, int64_t V,
    const int32_t* __restrict__ req_index, int64_t n_req, int32_t* __restrict__ accepted,
    int32_t* __restrict__ accept_len, void* __restrict__ ws, int skip_ended) {
    __shared__ FusedShared sh;
    const int N = D + 1;
    // row-major: every request's row 0 is dispatched before any row 1
    const int j = (int)(blockIdx.x / (uint64_t)n_req);
    const int64_t slot = (int64_t)blockIdx.x - (int64_t)j * n_req;
    const int64_t b = req_index ? (int64_t)req_index[slot] : slot;
    if (b < 0 || b >= B) return;   // uniform over the workgroup
    const int tid = threadIdx.x;
    const RowPar rpar(ws, slot);
    if (skip_ended && j > 0) {
        // a row after one that already ended the chain is not needed: count it in and leave
        if (tid == 0) {
            const uint64_t w = __hip_atomic_load(rpar.word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sh.acc = (w & (((uint64_t)1 << j) - 1)) != 0 ? 1 : 0;
        }
        __syncthreads();
        if (sh.acc) {
            if (tid >= kWave) return;
            int32_t yt = -1;
            const int L = rpar.arrive(j, N, false, 0, yt);
            if (L < 0) return;
            const int32_t yl = read_lane(yt, L);
            if (tid < N) accepted[b * N + tid] = tid < L ? x[b * D + tid] : (tid == L ? yl : -1);
            if (tid == 0) accept_len[b] = L;
            return;
        }
    }
    const float Tm = temperature[b];
    const int32_t k = top_k ? top_k[b] : 0;
    const float tp = top_p ? top_p[b] : 1.0f;
    const T* row = logits + ((int64_t)b * N + j) * V;
    const float* qj = j < D ? q + ((int64_t)b * D + j) * V : nullptr;

    // The draft id is one uniform load; q at it is loaded by thread 0 now and
    // waited for only at the accept test, so neither holds up the row's loads.
    // A register-resident row takes the logit at the id from the thread that
    // holds it (rr_stats' probe); other rows read it at the test.  The
    // uniforms are formed at the test and the draw.
    const int32_t xj = j < D ? x[b * D + j] : -1;
    const bool xin = xj >= 0 && (int64_t)xj < V;
    float qx = 0.0f;
    if (tid == 0 && xin) qx = qj[xj];
    RowProb rp{kProbOneHot, 0.0f, 0.0f, 0.0f, 0u, 0};
    bool probed = false;   // sh.rr.probe_key holds the key of the logit at xj
    auto accepted_here = [&]() {   // the serial kernel's test at position j
        if (tid == 0) {
            bool ok = false;
            if (xin) {
                float pv;
                if constexpr (sizeof(T) == 2) {
                    if (probed) pv = key_prob(rp, sh.rr, sh.rr.probe_key);
                    else pv = row_prob<T>(rp, sh.rr, row[xj], xj);
                } else {
                    pv = row_prob<T>(rp, sh.rr, row[xj], xj);
                }
                const uint32_t cj = uniform_code(philox_word(seed[b], offset[b], (uint64_t)j));
                ok = (double)((float)cj * 0x1p-24f) * (double)qx < (double)pv;
            }
            sh.acc = ok ? 1 : 0;
        }
        __syncthreads();
        return sh.acc != 0;
    };
    // the draw's uniform, formed only by rows that draw
    auto draw_uniform = [&]() {
        return (double)uniform_code(philox_word(seed[b], offset[b], (uint64_t)D)) * 0x1p-24;
    };
    bool done = false, drawn = false, acc = false;
    int64_t y = -1;
    if ((double)Tm < kGreedyTemperature) {
        rp.mode = kProbOneHot;
        rp.y = row_argmax<kFvBlock, false>(row, V, sh.rr.u.sm.am);
    } else {
        if constexpr (NV > 0) {
            u32x4 w[NV];
            uint32_t vmax[(NV + 1) / 2];
            RrStats st;
            const uint16_t* row16 = reinterpret_cast<const uint16_t*>(row);
            if (rr_stats<NV, false, true>(sh.rr, row16, V, Tm, k, tp, tid, w, st, 0.0f, vmax, xin ? xj : -1)) {
                rp = RowProb{st.table ? kProbTable : kProbRrExp, st.m, st.scale, st.inv, st.kmin, 0};
                done = true;
                probed = true;
                acc = j < D && accepted_here();
                if (!acc) {
                    const double uf = draw_uniform();
                    // a short row keeps its keys in registers for the draw;
                    // a long one revisits the vectors that hold kept keys
                    CompactDraw cd;
                    if constexpr (NV <= 4) {
                        cd = compact_draw_regs<NV>(sh, rp, w, vmax, V, qj, uf, tid);
                        if (cd.used && cd.y < 0 && qj)
                            cd = compact_draw_regs<NV>(sh, rp, w, vmax, V, nullptr, uf, tid);
                    } else {
                        cd = compact_draw<NV>(sh, rp, row16, vmax, V, qj, uf, tid);
                        if (cd.used && cd.y < 0 && qj) cd = compact_draw<NV>(sh, rp, row16, vmax, V, nullptr, uf, tid);
                    }
                    y = cd.y;
                    drawn = cd.used;
                }
            }
        }
        if (!done) {
            __syncthreads();
            const StreamStats ss = streamed_stats<T>(row, V, Tm, k, tp, sh.rr.u.sm);
            rp = RowProb{kProbStreamed, ss.m, ss.scale, ss.inv, ss.kmin, 0};
        }
    }
    if (!done) acc = j < D && accepted_here();
    if (!acc && !drawn) {
        const double uf = draw_uniform();
        y = qj ? fused_draw<T, true>(sh, rp, row, qj, V, uf) : fused_draw<T, false>(sh, rp, row, nullptr, V, uf);
        if (y < 0 && qj) y = fused_draw<T, false>(sh, rp, row, nullptr, V, uf);
    }
    if (!acc && y < 0) y = (int64_t)(((uint64_t)(draw_uniform() * 0x1p24) * (uint64_t)V) >> 24);
    // the hand-off of sv_rowpar.hpp: a row ends the chain when its draft is
    // rejected (or it is the bonus row); the request's last workgroup gets
    // L = the first such row and the token row L drew
    if (tid >= kWave) return;
    int32_t yt = -1;
    const int L = rpar.arrive(j, N, j == D || !acc, (int32_t)(acc ? 0 : y), yt);
    if (L < 0) return;
    // tokens x_0..x_{L-1}, the token drawn on row L, then -1
    const int32_t yl = read_lane(yt, L);
    if (tid < N) accepted[b * N + tid] = tid < L ? x[b * D + tid] : (tid == L ? yl : -1);
    if (tid == 0) accept_len[b] = L;
}

// Single-step sampling ("tokenspeed sampling/backends/flashinfer.py",
// sample: softmax(logits, T), then top_k_top_p_sampling_from_probs with the
// joint filter order, per-request seed and offset; min-p as TensorRT-LLM's
// fused sampler takes it).  One 1024-thread workgroup per request: a row
// below the greedy temperature takes its argmax; otherwise the joint
// statistics (register-resident for bf16 rows that fit, streamed otherwise)
// and the verify's draw on row 0 with the uniform of word 0 of the request's
// stream (the bonus draw of a verify without drafts).
template <typename T, int NV>
__global__ __launch_bounds__(kFvBlock) void sample_kernel(
    const T* __restrict__ logits, const float* __restrict__ temperature, const int32_t* __restrict__ top_k,
    const float* __restrict__ top_p, const float* __restrict__ min_p, const uint64_t* __restrict__ seed,
    const uint64_t* __restrict__ offset, int64_t B, int64_t V, const int32_t* __restrict__ req_index,
    int32_t* __restrict__ tokens) {
    __shared__ FusedShared sh;
    const int64_t b = req_index ? (int64_t)req_index[blockIdx.x] : (int64_t)blockIdx.x;
    if (b < 0 || b >= B) return;   // uniform over the workgroup
    const int tid = threadIdx.x;
    const T* row = logits + b * V;
    const float Tm = temperature[b];
    if ((double)Tm < kGreedyTemperature) {
        const int64_t y = row_argmax<kFvBlock, false>(row, V, sh.rr.u.sm.am);
        if (tid == 0) tokens[b] = (int32_t)y;
        return;
    }
    if (tid == 0) sh.code[0] = uniform_code(philox_word(seed[b], offset[b], 0));
    const int32_t k = top_k ? top_k[b] : 0;
    const float tp = top_p ? top_p[b] : 1.0f;
    const float mp = min_p ? min_p[b] : 0.0f;
    RowProb rp{kProbStreamed, 0.0f, 0.0f, 0.0f, 0u, 0};
    bool done = false, drawn = false;
    int64_t y = -1;
    if constexpr (NV > 0) {
        u32x4 w[NV];
        uint32_t vmax[(NV + 1) / 2];
        RrStats st;
        const uint16_t* row16 = reinterpret_cast<const uint16_t*>(row);
        if (rr_stats<NV, true, true>(sh.rr, row16, V, Tm, k, tp, tid, w, st, mp, vmax)) {
            rp = RowProb{st.table ? kProbTable : kProbRrExp, st.m, st.scale, st.inv, st.kmin, 0};
            done = true;
            // a small kept set is drawn by revisiting only the vectors that hold it
            const CompactDraw cd = compact_draw<NV>(sh, rp, row16, vmax, V, nullptr, (double)sh.code[0] * 0x1p-24, tid);
            y = cd.y;
            drawn = cd.used;
        }
    }
    if (!done) {
        __syncthreads();
        const JointStats js = streamed_stats_joint<T>(row, V, Tm, k, tp, mp, sh.rr.u.sm);
        rp = RowProb{kProbStreamed, js.m, js.scale, js.inv, js.kmin, 0};
        rp.thr = js.thr;
    }
    __syncthreads();
    const double uf = (double)sh.code[0] * 0x1p-24;
    if (!drawn) y = fused_draw<T, false>(sh, rp, row, nullptr, V, uf);
    if (y < 0) y = (int64_t)(((uint64_t)sh.code[0] * (uint64_t)V) >> 24);
    if (tid == 0) tokens[b] = (int32_t)y;
}

hipError_t launch_sample(const void* logits, int dtype, const float* temperature, const int32_t* top_k,
                         const float* top_p, const float* min_p, const uint64_t* seed, const uint64_t* offset,
                         int64_t B, int64_t V, const int32_t* req_index, int64_t n_req, int32_t* tokens,
                         hipStream_t stream) {
    if (V > (int64_t)kFvMaxChunks * kFvChunk) return hipErrorInvalidValue;
    if (dtype == kDtypeBF16) {
        const uint16_t* lg = static_cast<const uint16_t*>(logits);
        const int64_t nv = (V + kRrBlock * 8 - 1) / (kRrBlock * 8);
        // the register-resident path needs every row 16-byte aligned
        const bool rr = (V & 7) == 0 && (uintptr_t)lg % 16 == 0 && nv <= 20;
#define SV_SK(NVV)                                                                                                   \
    hipLaunchKernelGGL((sample_kernel<uint16_t, NVV>), dim3((unsigned)n_req), dim3(kFvBlock), 0, stream, lg,         \
                       temperature, top_k, top_p, min_p, seed, offset, B, V, req_index, tokens)
        if (!rr) SV_SK(0);
        else if (nv <= 1) SV_SK(1);
        else if (nv <= 2) SV_SK(2);
        else if (nv <= 4) SV_SK(4);
        else if (nv <= 8) SV_SK(8);
        else if (nv <= 12) SV_SK(12);
        else if (nv <= 16) SV_SK(16);
        else SV_SK(20);
#undef SV_SK
    } else {
        hipLaunchKernelGGL((sample_kernel<float, 0>), dim3((unsigned)n_req), dim3(kFvBlock), 0, stream,
                           static_cast<const float*>(logits), temperature, top_k, top_p, min_p, seed, offset, B, V,
                           req_index, tokens);
    }
    return hipGetLastError();
}

int64_t verify_fused_max_vocab() { return (int64_t)kFvMaxChunks * kFvChunk; }

int64_t verify_fused_workspace_bytes(int64_t n_req, int D) {
    return (D > 0 && n_req > 0) ? rowpar_workspace_bytes(n_req) : 0;
}

template <typename T, int NV>
static void launch_fv(const T* logits, const float* temperature, const int32_t* top_k, const float* top_p,
                      const float* q, const int32_t* x, const uint64_t* seed, const uint64_t* offset, int64_t B,
                      int D, int64_t V, const int32_t* req_index, int64_t n_req, int32_t* accepted,
                      int32_t* accept_len, void* workspace, hipStream_t stream) {
    // with the workspace: one workgroup per row; rows that cannot all run at
    // once skip the rows after one that ended the chain
    const int64_t rows = n_req * (D + 1);
    if (workspace && verify_fused_workspace_bytes(n_req, D) > 0) {
        const int skip = rows > device_compute_units() ? 1 : 0;
        hipLaunchKernelGGL((verify_fused_rows_kernel<T, NV>), dim3((unsigned)rows), dim3(kFvBlock), 0, stream,
                           logits, temperature, top_k, top_p, q, x, seed, offset, B, D, V, req_index, n_req,
                           accepted, accept_len, workspace, skip);
        return;
    }
    hipLaunchKernelGGL((verify_fused_kernel<T, NV>), dim3((unsigned)n_req), dim3(kFvBlock), 0, stream, logits,
                       temperature, top_k, top_p, q, x, seed, offset, B, D, V, req_index, accepted, accept_len);
}

hipError_t launch_verify_fused(const void* logits, int dtype, const float* temperature, const int32_t* top_k,
                               const float* top_p, const float* draft_probs, const int32_t* draft_ids,
                               const uint64_t* seed, const uint64_t* offset, int64_t B, int D, int64_t V,
                               const int32_t* req_index, int64_t n_req, int32_t* accepted, int32_t* accept_len,
                               void* workspace, hipStream_t stream) {
    if (V > verify_fused_max_vocab()) return hipErrorInvalidValue;
    if (dtype == kDtypeBF16) {
        const uint16_t* lg = static_cast<const uint16_t*>(logits);
        const int64_t nv = (V + kRrBlock * 8 - 1) / (kRrBlock * 8);
        // the register-resident path needs every row 16-byte aligned
        const bool rr = (V & 7) == 0 && (uintptr_t)lg % 16 == 0 && nv <= 20;
#define SV_FV(NVV) \
    launch_fv<uint16_t, NVV>(lg, temperature, top_k, top_p, draft_probs, draft_ids, seed, offset, B, D, V, req_index, \
                             n_req, accepted, accept_len, workspace, stream)
        if (!rr) SV_FV(0);
        else if (nv <= 1) SV_FV(1);
        else if (nv <= 2) SV_FV(2);
        else if (nv <= 4) SV_FV(4);
        else if (nv <= 8) SV_FV(8);
        else if (nv <= 12) SV_FV(12);
        else if (nv <= 16) SV_FV(16);
        else SV_FV(20);
#undef SV_FV
    } else {
        launch_fv<float, 0>(static_cast<const float*>(logits), temperature, top_k, top_p, draft_probs, draft_ids,
                            seed, offset, B, D, V, req_index, n_req, accepted, accept_len, workspace, stream);
    }
    return hipGetLastError();
}

}  // namespace sv
