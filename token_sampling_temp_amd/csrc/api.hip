// C ABI of the verification library: host-side validation, device check and
// kernel launch on the caller's stream.  Validation happens before any HIP
// call, so argument errors are reported without touching a device.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "specverify.h"
#include "sv_launch.hpp"

static_assert(SPECVERIFY_STATIC_SCRATCH_BYTES == sv::kChainStaticScratchBytes,
              "the header's static scratch size must match the library's");

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

constexpr int64_t kMaxV = 2147483647LL;
constexpr int kMaxDevices = 256;
std::atomic<int> g_device_ok[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other

int check_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SPECVERIFY_HIP_ERROR, "hipGetDevice: %s", hipGetErrorString(e));
    int state = (dev >= 0 && dev < kMaxDevices) ? g_device_ok[dev].load(std::memory_order_relaxed) : 0;
    if (state == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess)
            return fail(SPECVERIFY_HIP_ERROR, "hipGetDeviceProperties: %s", hipGetErrorString(e));
        state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        if (dev >= 0 && dev < kMaxDevices) g_device_ok[dev].store(state, std::memory_order_relaxed);
        if (state == 2)
            return fail(SPECVERIFY_UNSUPPORTED, "device %d is %s; this library is built for gfx950", dev,
                        prop.gcnArchName);
    }
    if (state == 2) return fail(SPECVERIFY_UNSUPPORTED, "device %d is not gfx950", dev);
    return SPECVERIFY_OK;
}

// Sizes shared by every entry point.  Returns OK or INVALID_ARGUMENT.
int check_sizes(const char* fn, int64_t B, int64_t npos, int64_t V, const int32_t* req_index, int64_t n_req,
                int64_t elem_bytes) {
    if (B < 0) return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: B=%lld must be >= 0", fn, (long long)B);
    if (V < 1 || V > kMaxV)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: V=%lld must be in [1, 2^31)", fn, (long long)V);
    if (n_req < 0 || n_req > B)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: n_req=%lld must be in [0, B=%lld]", fn, (long long)n_req,
                    (long long)B);
    if (!req_index && n_req != B)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: n_req=%lld must equal B=%lld when req_index is NULL", fn,
                    (long long)n_req, (long long)B);
    if (n_req > 2147483647LL)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: n_req=%lld exceeds the grid limit", fn, (long long)n_req);
    // B * npos * V * elem_bytes must fit comfortably in 63 bits
    const long double bytes = (long double)B * (long double)npos * (long double)V * (long double)elem_bytes;
    if (bytes > 4.0e18L) return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: tensor size overflows", fn);
    return SPECVERIFY_OK;
}

int check_draft(const char* fn, int64_t D) {
    if (D < 0 || D > SPECVERIFY_MAX_DRAFT)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: D=%lld must be in [0, %d]", fn, (long long)D,
                    SPECVERIFY_MAX_DRAFT);
    return SPECVERIFY_OK;
}

int check_dtype(const char* fn, int dtype) {
    if (dtype != SPECVERIFY_F32 && dtype != SPECVERIFY_BF16)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: dtype=%d must be SPECVERIFY_F32 or SPECVERIFY_BF16", fn,
                    dtype);
    return SPECVERIFY_OK;
}

#define SV_REQUIRE(ptr, name)                                                                             \
    do {                                                                                                  \
        if (!(ptr)) return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: %s must not be NULL", fn, name);       \
    } while (0)

#define SV_TRY(expr)                  \
    do {                              \
        const int _s = (expr);        \
        if (_s != SPECVERIFY_OK) return _s; \
    } while (0)

// A chain call's workspace: what the launch needs for (n_req, V), present,
// large enough and 8-byte aligned.  NULL is accepted when nothing is needed.
int check_chain_workspace(const char* fn, int64_t n_req, int64_t V, const void* workspace,
                          int64_t workspace_bytes) {
    const int64_t need = sv::chain_workspace_bytes(n_req, V);
    if (need == 0) return SPECVERIFY_OK;
    if (!workspace)
        return fail(SPECVERIFY_INVALID_ARGUMENT,
                    "%s: n_req=%lld V=%lld splits rows over workgroups and needs a workspace of %lld bytes "
                    "(specverify_chain_workspace_bytes); workspace is NULL",
                    fn, (long long)n_req, (long long)V, (long long)need);
    if (workspace_bytes < need)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: workspace_bytes=%lld, n_req=%lld V=%lld needs %lld", fn,
                    (long long)workspace_bytes, (long long)n_req, (long long)V, (long long)need);
    if (reinterpret_cast<uintptr_t>(workspace) % 8 != 0)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: workspace must be 8-byte aligned", fn);
    return SPECVERIFY_OK;
}

int launched(const char* fn, hipError_t e) {
    if (e != hipSuccess) return fail(SPECVERIFY_HIP_ERROR, "%s: launch failed: %s", fn, hipGetErrorString(e));
    g_last_error.clear();
    return SPECVERIFY_OK;
}

}  // namespace

extern "C" {

int specverify_softmax_renorm(const void* logits, int dtype, int64_t B, int64_t npos, int64_t V,
                              const float* temperature, const int32_t* top_k, const float* top_p,
                              const int32_t* req_index, int64_t n_req, float* probs_out, void* stream) {
    const char* fn = "specverify_softmax_renorm";
    SV_TRY(check_dtype(fn, dtype));
    if (npos < 1 || npos > 65535)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: npos=%lld must be in [1, 65535]", fn, (long long)npos);
    SV_TRY(check_sizes(fn, B, npos, V, req_index, n_req, 4));
    if (n_req == 0) return SPECVERIFY_OK;
    SV_REQUIRE(logits, "logits");
    SV_REQUIRE(temperature, "temperature");
    SV_REQUIRE(probs_out, "probs_out");
    SV_TRY(check_device());
    return launched(fn, sv::launch_softmax_renorm(logits, dtype, B, npos, V, temperature, top_k, top_p, req_index,
                                                  n_req, probs_out, static_cast<hipStream_t>(stream)));
}

int specverify_chain_workspace_bytes(int64_t n_req, int64_t V, int64_t* bytes) {
    const char* fn = "specverify_chain_workspace_bytes";
    SV_REQUIRE(bytes, "bytes");
    if (n_req < 0) return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: n_req=%lld must be >= 0", fn, (long long)n_req);
    if (V < 1 || V > kMaxV)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: V=%lld must be in [1, 2^31)", fn, (long long)V);
    if ((long double)n_req * (long double)V > 4.0e18L)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: size overflows", fn);
    *bytes = sv::chain_workspace_bytes(n_req, V);
    g_last_error.clear();
    return SPECVERIFY_OK;
}

int specverify_chain_reject(const float* draft_probs, const int32_t* draft_ids, const float* target_probs,
                            const uint64_t* seed, const uint64_t* offset, int64_t B, int64_t D, int64_t V,
                            const int32_t* req_index, int64_t n_req, int32_t* accepted_tokens,
                            int32_t* accept_length, void* workspace, int64_t workspace_bytes, void* stream) {
    const char* fn = "specverify_chain_reject";
    SV_TRY(check_draft(fn, D));
    SV_TRY(check_sizes(fn, B, D + 1, V, req_index, n_req, 4));
    if (n_req == 0) return SPECVERIFY_OK;
    if (D > 0) SV_REQUIRE(draft_ids, "draft_ids");   // draft_probs NULL: point-mass drafts
    SV_REQUIRE(target_probs, "target_probs");
    SV_REQUIRE(seed, "seed");
    SV_REQUIRE(offset, "offset");
    SV_REQUIRE(accepted_tokens, "accepted_tokens");
    SV_REQUIRE(accept_length, "accept_length");
    SV_TRY(check_chain_workspace(fn, n_req, V, workspace, workspace_bytes));
    SV_TRY(check_device());
    return launched(fn, sv::launch_chain_reject(draft_probs, draft_ids, target_probs, nullptr, 0, nullptr, V, seed,
                                                offset, B, (int)D, V, req_index, n_req, accepted_tokens,
                                                accept_length, workspace, static_cast<hipStream_t>(stream)));
}

int specverify_chain_reject_noalloc(const float* draft_probs, const int32_t* draft_ids, const float* target_probs,
                                    const uint64_t* seed, const uint64_t* offset, int64_t B, int64_t D, int64_t V,
                                    const int32_t* req_index, int64_t n_req, int32_t* accepted_tokens,
                                    int32_t* accept_length, void* stream) {
    const char* fn = "specverify_chain_reject_noalloc";
    SV_TRY(check_draft(fn, D));
    SV_TRY(check_sizes(fn, B, D + 1, V, req_index, n_req, 4));
    if (n_req == 0) return SPECVERIFY_OK;
    if (D > 0) SV_REQUIRE(draft_ids, "draft_ids");
    SV_REQUIRE(target_probs, "target_probs");
    SV_REQUIRE(seed, "seed");
    SV_REQUIRE(offset, "offset");
    SV_REQUIRE(accepted_tokens, "accepted_tokens");
    SV_REQUIRE(accept_length, "accept_length");
    const int64_t need = sv::chain_workspace_bytes(n_req, V);
    if (need > SPECVERIFY_STATIC_SCRATCH_BYTES)
        return fail(SPECVERIFY_INVALID_ARGUMENT,
                    "%s: n_req=%lld V=%lld needs %lld bytes of scratch; the static scratch holds %lld "
                    "(use specverify_chain_reject with a caller workspace)",
                    fn, (long long)n_req, (long long)V, (long long)need, (long long)SPECVERIFY_STATIC_SCRATCH_BYTES);
    SV_TRY(check_device());
    void* ptr = nullptr;
    if (need > 0) {
        const hipError_t e = sv::chain_static_scratch(static_cast<hipStream_t>(stream), &ptr);
        if (e != hipSuccess) return fail(SPECVERIFY_HIP_ERROR, "%s: static scratch: %s", fn, hipGetErrorString(e));
    }
    return launched(fn, sv::launch_chain_reject(draft_probs, draft_ids, target_probs, nullptr, 0, nullptr, V, seed,
                                                offset, B, (int)D, V, req_index, n_req, accepted_tokens,
                                                accept_length, ptr, static_cast<hipStream_t>(stream)));
}

int specverify_chain_reject_ragged(const float* draft_probs, const int32_t* t2d, int64_t Vd,
                                   const int32_t* draft_ids, const float* target_probs, const int32_t* qo_indptr,
                                   int64_t n_rows, const uint64_t* seed, const uint64_t* offset, int64_t B, int64_t D,
                                   int64_t V, const int32_t* req_index, int64_t n_req, int32_t* accepted_tokens,
                                   int32_t* accept_length, void* workspace, int64_t workspace_bytes, void* stream) {
    const char* fn = "specverify_chain_reject_ragged";
    SV_TRY(check_draft(fn, D));
    if (t2d && !draft_probs)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: t2d needs draft_probs (a draft vocabulary of Vd entries)", fn);
    if (t2d && (Vd < 1 || Vd > kMaxV))
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: Vd=%lld must be in [1, 2^31)", fn, (long long)Vd);
    if (t2d && (long double)B * (long double)D * (long double)Vd * 4.0L > 4.0e18L)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: tensor size overflows", fn);
    SV_TRY(check_sizes(fn, B, D + 1, V, req_index, n_req, 4));
    if (n_rows < 0 || n_rows > 2147483647LL)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: n_rows=%lld must be in [0, 2^31)", fn, (long long)n_rows);
    if ((long double)n_rows * (long double)V * 4.0L > 4.0e18L)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: tensor size overflows", fn);
    if (n_req == 0) return SPECVERIFY_OK;
    if (D > 0) SV_REQUIRE(draft_ids, "draft_ids");   // draft_probs NULL: point-mass drafts
    SV_REQUIRE(target_probs, "target_probs");
    SV_REQUIRE(qo_indptr, "qo_indptr");
    SV_REQUIRE(seed, "seed");
    SV_REQUIRE(offset, "offset");
    SV_REQUIRE(accepted_tokens, "accepted_tokens");
    SV_REQUIRE(accept_length, "accept_length");
    SV_TRY(check_chain_workspace(fn, n_req, V, workspace, workspace_bytes));
    SV_TRY(check_device());
    return launched(fn, sv::launch_chain_reject(draft_probs, draft_ids, target_probs, qo_indptr, n_rows, t2d,
                                                t2d ? Vd : V, seed, offset, B, (int)D, V, req_index, n_req,
                                                accepted_tokens, accept_length, workspace,
                                                static_cast<hipStream_t>(stream)));
}

int specverify_d2t_inverse(const int64_t* d2t, int64_t Vd, int64_t V, int32_t* t2d, void* stream) {
    const char* fn = "specverify_d2t_inverse";
    if (V < 1 || V > kMaxV)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: V=%lld must be in [1, 2^31)", fn, (long long)V);
    if (Vd < 1 || Vd > kMaxV)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: Vd=%lld must be in [1, 2^31)", fn, (long long)Vd);
    if (Vd > V)
        return fail(SPECVERIFY_INVALID_ARGUMENT,
                    "%s: Vd=%lld exceeds V=%lld (draft entries cannot map one-to-one into the target vocabulary)",
                    fn, (long long)Vd, (long long)V);
    SV_REQUIRE(t2d, "t2d");
    SV_TRY(check_device());
    return launched(fn, sv::launch_d2t_inverse(d2t, Vd, V, t2d, static_cast<hipStream_t>(stream)));
}

int specverify_d2t_expand(const float* draft_probs, const int32_t* t2d, int64_t rows, int64_t Vd, int64_t V,
                          float* full_draft_probs, void* stream) {
    const char* fn = "specverify_d2t_expand";
    if (rows < 0) return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: rows=%lld must be >= 0", fn, (long long)rows);
    if (V < 1 || V > kMaxV)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: V=%lld must be in [1, 2^31)", fn, (long long)V);
    if (Vd < 1 || Vd > kMaxV)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: Vd=%lld must be in [1, 2^31)", fn, (long long)Vd);
    if ((long double)rows * (long double)(V > Vd ? V : Vd) * 4.0L > 4.0e18L)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: tensor size overflows", fn);
    if (rows == 0) return SPECVERIFY_OK;
    SV_REQUIRE(draft_probs, "draft_probs");
    SV_REQUIRE(t2d, "t2d");
    SV_REQUIRE(full_draft_probs, "full_draft_probs");
    SV_TRY(check_device());
    return launched(fn, sv::launch_d2t_expand(draft_probs, t2d, rows, Vd, V, full_draft_probs,
                                              static_cast<hipStream_t>(stream)));
}

// Validates an optional row-parallel workspace of `need` bytes.
static int check_rowpar_workspace(const char* fn, const void* workspace, int64_t workspace_bytes, int64_t need,
                                  int64_t n_req, int64_t D) {
    if (!workspace || need == 0) return SPECVERIFY_OK;
    if (workspace_bytes < need)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: workspace_bytes=%lld, n_req=%lld D=%lld needs %lld", fn,
                    (long long)workspace_bytes, (long long)n_req, (long long)D, (long long)need);
    if (reinterpret_cast<uintptr_t>(workspace) % 8 != 0)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: workspace must be 8-byte aligned", fn);
    return SPECVERIFY_OK;
}

// Shared body of the row-parallel workspace size queries.
static int rowpar_query(const char* fn, int64_t n_req, int64_t D, int64_t* bytes,
                        int64_t (*size)(int64_t, int)) {
    SV_REQUIRE(bytes, "bytes");
    if (n_req < 0) return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: n_req=%lld must be >= 0", fn, (long long)n_req);
    SV_TRY(check_draft(fn, D));
    *bytes = size(n_req, (int)D);
    g_last_error.clear();
    return SPECVERIFY_OK;
}

int specverify_greedy_verify_workspace_bytes(int64_t n_req, int64_t D, int64_t* bytes) {
    return rowpar_query("specverify_greedy_verify_workspace_bytes", n_req, D, bytes, sv::greedy_workspace_bytes);
}

int specverify_gumbel_sample_workspace_bytes(int64_t n_req, int64_t D, int64_t* bytes) {
    return rowpar_query("specverify_gumbel_sample_workspace_bytes", n_req, D, bytes, sv::gumbel_workspace_bytes);
}

int specverify_greedy_verify(const void* target_logits, int dtype, const int32_t* draft_ids, int64_t B,
                             int64_t D, int64_t V, const int32_t* req_index, int64_t n_req,
                             int32_t* accepted_tokens, int32_t* accept_length, int32_t* predict,
                             int32_t* accept_index, int32_t* argmax_out, void* workspace, int64_t workspace_bytes,
                             void* stream) {
    const char* fn = "specverify_greedy_verify";
    SV_TRY(check_dtype(fn, dtype));
    SV_TRY(check_draft(fn, D));
    SV_TRY(check_sizes(fn, B, D + 1, V, req_index, n_req, dtype == SPECVERIFY_BF16 ? 2 : 4));
    if (n_req == 0) return SPECVERIFY_OK;
    SV_REQUIRE(target_logits, "target_logits");
    if (D > 0) SV_REQUIRE(draft_ids, "draft_ids");
    SV_REQUIRE(accepted_tokens, "accepted_tokens");
    SV_REQUIRE(accept_length, "accept_length");
    SV_TRY(check_rowpar_workspace(fn, workspace, workspace_bytes, sv::greedy_workspace_bytes(n_req, (int)D), n_req,
                                  D));
    SV_TRY(check_device());
    return launched(fn, sv::launch_greedy_verify(target_logits, dtype, draft_ids, B, (int)D, V, req_index, n_req,
                                                 accepted_tokens, accept_length, predict, accept_index, argmax_out,
                                                 workspace, static_cast<hipStream_t>(stream)));
}

int specverify_gumbel_sample(const void* target_logits, int dtype, const float* temperature,
                             const int32_t* draft_ids, const uint64_t* seed, const uint64_t* offset, int64_t B,
                             int64_t D, int64_t V, const int32_t* req_index, int64_t n_req,
                             int32_t* accepted_tokens, int32_t* accept_length, int32_t* sampled_out,
                             void* workspace, int64_t workspace_bytes, void* stream) {
    const char* fn = "specverify_gumbel_sample";
    SV_TRY(check_dtype(fn, dtype));
    SV_TRY(check_draft(fn, D));
    SV_TRY(check_sizes(fn, B, D + 1, V, req_index, n_req, dtype == SPECVERIFY_BF16 ? 2 : 4));
    if (n_req == 0) return SPECVERIFY_OK;
    SV_REQUIRE(target_logits, "target_logits");
    SV_REQUIRE(temperature, "temperature");
    if (D > 0) SV_REQUIRE(draft_ids, "draft_ids");
    SV_REQUIRE(seed, "seed");
    SV_REQUIRE(offset, "offset");
    SV_REQUIRE(accepted_tokens, "accepted_tokens");
    SV_REQUIRE(accept_length, "accept_length");
    SV_TRY(check_rowpar_workspace(fn, workspace, workspace_bytes, sv::gumbel_workspace_bytes(n_req, (int)D), n_req,
                                  D));
    SV_TRY(check_device());
    return launched(fn, sv::launch_gumbel_sample(target_logits, dtype, temperature, draft_ids, seed, offset, B,
                                                 (int)D, V, req_index, n_req, accepted_tokens, accept_length,
                                                 sampled_out, workspace, static_cast<hipStream_t>(stream)));
}

int specverify_sample(const void* logits, int dtype, const float* temperature, const int32_t* top_k,
                      const float* top_p, const float* min_p, const uint64_t* seed, const uint64_t* offset, int64_t B,
                      int64_t V, const int32_t* req_index, int64_t n_req, int32_t* tokens, void* stream) {
    const char* fn = "specverify_sample";
    SV_TRY(check_dtype(fn, dtype));
    SV_TRY(check_sizes(fn, B, 1, V, req_index, n_req, 4));
    if (V > sv::verify_fused_max_vocab())
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: V=%lld exceeds %lld", fn, (long long)V,
                    (long long)sv::verify_fused_max_vocab());
    if (n_req == 0) return SPECVERIFY_OK;
    SV_REQUIRE(logits, "logits");
    SV_REQUIRE(temperature, "temperature");
    SV_REQUIRE(seed, "seed");
    SV_REQUIRE(offset, "offset");
    SV_REQUIRE(tokens, "tokens");
    SV_TRY(check_device());
    return launched(fn, sv::launch_sample(logits, dtype, temperature, top_k, top_p, min_p, seed, offset, B, V,
                                          req_index, n_req, tokens, static_cast<hipStream_t>(stream)));
}

int specverify_verify_fused_workspace_bytes(int64_t n_req, int64_t D, int64_t* bytes) {
    const char* fn = "specverify_verify_fused_workspace_bytes";
    SV_REQUIRE(bytes, "bytes");
    if (n_req < 0) return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: n_req=%lld must be >= 0", fn, (long long)n_req);
    SV_TRY(check_draft(fn, D));
    *bytes = sv::verify_fused_workspace_bytes(n_req, (int)D);
    g_last_error.clear();
    return SPECVERIFY_OK;
}

int specverify_verify_fused(const void* target_logits, int dtype, const float* temperature, const int32_t* top_k,
                            const float* top_p, const float* draft_probs, const int32_t* draft_ids,
                            const uint64_t* seed, const uint64_t* offset, int64_t B, int64_t D, int64_t V,
                            const int32_t* req_index, int64_t n_req, int32_t* accepted_tokens,
                            int32_t* accept_length, void* workspace, int64_t workspace_bytes, void* stream) {
    const char* fn = "specverify_verify_fused";
    SV_TRY(check_dtype(fn, dtype));
    SV_TRY(check_draft(fn, D));
    SV_TRY(check_sizes(fn, B, D + 1, V, req_index, n_req, 4));
    if (V > sv::verify_fused_max_vocab())
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: V=%lld exceeds %lld", fn, (long long)V,
                    (long long)sv::verify_fused_max_vocab());
    if (n_req == 0) return SPECVERIFY_OK;
    SV_REQUIRE(target_logits, "target_logits");
    SV_REQUIRE(temperature, "temperature");
    if (D > 0) {
        SV_REQUIRE(draft_probs, "draft_probs");
        SV_REQUIRE(draft_ids, "draft_ids");
    }
    SV_REQUIRE(seed, "seed");
    SV_REQUIRE(offset, "offset");
    SV_REQUIRE(accepted_tokens, "accepted_tokens");
    SV_REQUIRE(accept_length, "accept_length");
    const int64_t need = sv::verify_fused_workspace_bytes(n_req, (int)D);
    if (workspace && need > 0 && workspace_bytes < need)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: workspace_bytes=%lld, n_req=%lld D=%lld needs %lld", fn,
                    (long long)workspace_bytes, (long long)n_req, (long long)D, (long long)need);
    if (workspace && reinterpret_cast<uintptr_t>(workspace) % 8 != 0)
        return fail(SPECVERIFY_INVALID_ARGUMENT, "%s: workspace must be 8-byte aligned", fn);
    SV_TRY(check_device());
    return launched(fn, sv::launch_verify_fused(target_logits, dtype, temperature, top_k, top_p, draft_probs,
                                                draft_ids, seed, offset, B, (int)D, V, req_index, n_req,
                                                accepted_tokens, accept_length, need > 0 ? workspace : nullptr,
                                                static_cast<hipStream_t>(stream)));
}

const char* specverify_status_string(int status) {
    switch (status) {
        case SPECVERIFY_OK: return "SPECVERIFY_OK";
        case SPECVERIFY_INVALID_ARGUMENT: return "SPECVERIFY_INVALID_ARGUMENT";
        case SPECVERIFY_UNSUPPORTED: return "SPECVERIFY_UNSUPPORTED";
        case SPECVERIFY_HIP_ERROR: return "SPECVERIFY_HIP_ERROR";
        default: return "SPECVERIFY_UNKNOWN_STATUS";
    }
}

const char* specverify_last_error(void) { return g_last_error.c_str(); }

int specverify_version(void) { return SPECVERIFY_VERSION; }

}  // extern "C"
