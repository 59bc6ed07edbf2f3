// Host-side launchers of the verification kernels (called by the C ABI layer
// after argument validation).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace sv {

// Compute units of the current device, cached per device (256, the MI355X
// count, when the runtime cannot tell).
inline int device_compute_units() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

constexpr int kDtypeF32 = 0;
constexpr int kDtypeBF16 = 1;
constexpr int kMaxDraft = 16;

hipError_t launch_greedy_verify(const void* logits, int dtype, const int32_t* draft_ids, int64_t B, int D,
                                int64_t V, const int32_t* req_index, int64_t n_req, int32_t* accepted,
                                int32_t* accept_len, int32_t* predict, int32_t* accept_index,
                                int32_t* argmax_out, void* workspace, hipStream_t stream);
// Bytes of the row-parallel workspace greedy verify takes (0: none used).
int64_t greedy_workspace_bytes(int64_t n_req, int D);

// Chain rejection's workspace in bytes for n_req requests over V entries (0:
// none).  It holds n_req 32-bit counters, zero before and after every call
// (the kernel resets the ones it used), then the partial sums.
int64_t chain_partials_per_request(int64_t V);
int64_t chain_workspace_bytes(int64_t n_req, int64_t V);
// The library's static scratch for chain rejection without a caller workspace
// (same layout, at most kChainStaticScratchBytes): this device's address,
// resolved and cleared (a fill kernel on `stream`) on the first call per device.
constexpr int64_t kChainStaticScratchBytes = 4 << 20;
hipError_t chain_static_scratch(hipStream_t stream, void** out);
// qo_indptr NULL: dense target rows [B, D+1, V]; else packed rows [n_rows, V],
// request b owning rows [qo_indptr[b], qo_indptr[b+1]).  t2d NULL: draft rows
// [B, D, V]; else [B, D, Vd] over a smaller draft vocabulary, target entry v
// reading draft entry t2d[v].
hipError_t launch_chain_reject(const float* draft_probs, const int32_t* draft_ids, const float* target_probs,
                               const int32_t* qo_indptr, int64_t n_rows, const int32_t* t2d, int64_t Vd,
                               const uint64_t* seed,
                               const uint64_t* offset, int64_t B, int D, int64_t V, const int32_t* req_index,
                               int64_t n_req, int32_t* accepted, int32_t* accept_len, void* workspace,
                               hipStream_t stream);

// Draft -> target vocabulary placement.  launch_d2t_inverse builds t2d [V]
// (draft entry of each target entry, -1 for none) from the offset table
// d2t [Vd] (NULL: the first Vd target entries); launch_d2t_expand writes
// out [rows, V] with out[t] = draft_probs[t2d[t]] (0 where t2d[t] < 0).
hipError_t launch_d2t_inverse(const int64_t* d2t, int64_t Vd, int64_t V, int32_t* t2d, hipStream_t stream);
hipError_t launch_d2t_expand(const float* draft_probs, const int32_t* t2d, int64_t rows, int64_t Vd, int64_t V,
                             float* out, hipStream_t stream);

// Single-step sampling of one token per request from logits [B, V]
// (V <= verify_fused_max_vocab()).
hipError_t launch_sample(const void* logits, int dtype, const float* temperature, const int32_t* top_k,
                         const float* top_p, const float* min_p, const uint64_t* seed, const uint64_t* offset,
                         int64_t B, int64_t V, const int32_t* req_index, int64_t n_req, int32_t* tokens,
                         hipStream_t stream);

hipError_t launch_softmax_renorm(const void* logits, int dtype, int64_t B, int64_t npos, int64_t V,
                                 const float* temperature, const int32_t* top_k, const float* top_p,
                                 const int32_t* req_index, int64_t n_req, float* probs_out,
                                 hipStream_t stream);

hipError_t launch_gumbel_sample(const void* logits, int dtype, const float* temperature,
                                const int32_t* draft_ids, const uint64_t* seed, const uint64_t* offset,
                                int64_t B, int D, int64_t V, const int32_t* req_index, int64_t n_req,
                                int32_t* accepted, int32_t* accept_len, int32_t* sampled_out, void* workspace,
                                hipStream_t stream);
// Bytes of the row-parallel workspace Gumbel sampling takes (0: none used).
int64_t gumbel_workspace_bytes(int64_t n_req, int D);

// Fused target rows + chain rejection (V <= verify_fused_max_vocab()).  With
// a workspace of verify_fused_workspace_bytes(n_req, D) bytes (one line per
// request, zero between calls) every (request, row) gets a workgroup;
// without one, a request's rows are evaluated in order.
int64_t verify_fused_max_vocab();
int64_t verify_fused_workspace_bytes(int64_t n_req, int D);
hipError_t launch_verify_fused(const void* logits, int dtype, const float* temperature, const int32_t* top_k,
                               const float* top_p, const float* draft_probs, const int32_t* draft_ids,
                               const uint64_t* seed, const uint64_t* offset, int64_t B, int D, int64_t V,
                               const int32_t* req_index, int64_t n_req, int32_t* accepted, int32_t* accept_len,
                               void* workspace, hipStream_t stream);

}  // namespace sv
