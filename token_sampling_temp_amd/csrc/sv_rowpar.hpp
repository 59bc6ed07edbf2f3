// Row-parallel strict acceptance: one workgroup per (request, row) instead of
// one workgroup walking a request's rows in order.
//
// Strict acceptance ("TensorRT-LLM _torch/speculative/interface.py",
// _sample_and_accept_draft_tokens_base) needs the target tokens y_0..y_L only,
// where L is the first row whose draft id differs from y (or D).  The grid is
// row-major (workgroup g handles row g / n_req of request slot g % n_req), so
// the dispatcher starts every request's row 0 before any row 1, and so on.
//
// Each request slot owns one 128-byte line of the caller's workspace:
//   word   uint64  bits 0..N-1: rows that ended the chain (draft id rejected,
//                  or the bonus row D); bits 32..63: rows finished
//   ys[j]  uint32  row j's token with bit 31 set once written (0: not yet)
// A row that streams its logits polls `word` and stops as soon as a lower
// row's bit is set (its result can no longer be used).  When done, the row
// stores its token (any value if it stopped) and adds (1 << 32) plus its own
// bit if it ended the chain, in one atomic add that returns the previous
// word; the add that brings the count to N identifies the request's last
// workgroup, which reads L = the lowest set bit, collects ys[0..L] and writes
// the outputs.
//
// The hand-off needs no ordering between different words: the last
// workgroup waits on each ys[t] until bit 31 shows (every row stores its
// token before its add, so the store is already issued and the wait ends),
// and whatever a skipped or stopped row stored lies after L and is unused.
// Having read every token, the last workgroup clears its line, so the
// workspace is zero at rest and the next call, of any batch size, finds it
// so.
#pragma once

#include "sv_common.hpp"

namespace sv {

constexpr int64_t kRowParLine = 128;

// Bytes of the row-parallel workspace for n_req requests.
inline int64_t rowpar_workspace_bytes(int64_t n_req) { return (n_req * kRowParLine + 255) / 256 * 256; }

constexpr uint32_t kTokenWritten = 0x80000000u;

struct RowPar {
    uint64_t* word;
    uint32_t* ys;

    __device__ RowPar(void* ws, int64_t slot) {
        word = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + slot * kRowParLine);
        ys = reinterpret_cast<uint32_t*>(word + 1);
    }

    // Called by every lane of wave 0 once row j's token y is known (the same
    // value in every lane; anything if the row stopped early).  ends: row j
    // ends the chain.  Returns L in the request's last workgroup, with
    // yt = y_lane for lanes below N, and -1 elsewhere.
    __device__ __forceinline__ int arrive(int j, int N, bool ends, int32_t y, int32_t& yt) const {
        const int lane = threadIdx.x & (kWave - 1);
        uint64_t prev = 0;
        const uint64_t mine = ends ? (uint64_t)1 << j : 0;
        if (lane == 0) {
            __hip_atomic_store(&ys[j], kTokenWritten | (uint32_t)y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            prev = __hip_atomic_fetch_add(word, ((uint64_t)1 << 32) | mine, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
        }
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)prev);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(prev >> 32));
        if (hi != (uint32_t)(N - 1)) return -1;
        const uint32_t ended = lo | (uint32_t)mine;
        // every row's add follows its own store, so each wait below ends; the
        // bound only keeps a broken invariant from hanging the device
        uint32_t v = kTokenWritten;
        if (lane < N) {
            for (int spin = 0; spin < (1 << 20); ++spin) {
                v = __hip_atomic_load(&ys[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (v & kTokenWritten) break;
                __builtin_amdgcn_s_sleep(1);
            }
            __hip_atomic_store(&ys[lane], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (lane == 0) __hip_atomic_store(word, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        yt = (int32_t)(v & ~kTokenWritten);
        return ended ? __builtin_ctz(ended) : N - 1;
    }
};

}  // namespace sv
