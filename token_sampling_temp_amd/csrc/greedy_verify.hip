// Greedy chain verify: target token y_j = lowest-index argmax of row j; the
// accept length L counts the leading draft ids equal to y (strict acceptance).
// One workgroup per request walks its rows in order and stops after the first
// mismatch unless every row's argmax is requested.
#include <atomic>

#include "sv_argmax.hpp"
#include "sv_launch.hpp"

namespace sv {

// Workgroup size: 1024 threads hold one workgroup per CU; 512 threads hold
// two, so a batch of at least two requests per CU starts every request at
// once (with 1024 threads the second half of such a batch waits for free
// slots, and late starters with long accept chains set the end time).
template <typename T, int kGreedyBlock>
__global__ __launch_bounds__(kGreedyBlock) void greedy_verify_kernel(
    const T* __restrict__ logits, const int32_t* __restrict__ draft_ids, int64_t B, int D, int64_t V,
    const int32_t* __restrict__ req_index, int32_t* __restrict__ accepted, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ predict, int32_t* __restrict__ accept_index, int32_t* __restrict__ argmax_out) {
    __shared__ ArgmaxShared<kGreedyBlock> sh;
    __shared__ int32_t s_y[kMaxDraft + 1];
    __shared__ int32_t s_x[kMaxDraft];
    const int64_t b = req_index ? (int64_t)req_index[blockIdx.x] : (int64_t)blockIdx.x;
    if (b < 0 || b >= B) return;
    const int N = D + 1;
    // draft ids fetched up front (visible after the first row's reduction)
    if (threadIdx.x < D) s_x[threadIdx.x] = draft_ids[(int64_t)b * D + threadIdx.x];
    const bool all_rows = argmax_out != nullptr;
    int L = -1;
    int rows = 0;
    for (int j = 0; j < N; ++j) {
        const T* row = logits + ((int64_t)b * N + j) * V;
        const int64_t y = row_argmax<kGreedyBlock, true>(row, V, sh);
        if (threadIdx.x == 0) s_y[j] = (int32_t)y;
        rows = j + 1;
        if (L < 0 && (j == D || s_x[j] != (int32_t)y)) {
            L = j;
            if (!all_rows) break;
        }
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < N) {
        const int64_t o = (int64_t)b * N + t;
        const int32_t yt = t <= L ? s_y[t] : -1;
        accepted[o] = yt;
        if (predict) predict[o] = yt;
        if (accept_index) accept_index[o] = t <= L ? (int32_t)o : -1;
        if (argmax_out) argmax_out[o] = t < rows ? s_y[t] : -1;
    }
    if (t == 0) accept_len[b] = L;
}

// Compute units of the current device (cached per device; 256 if unknown).
static int greedy_device_cus() {
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

template <typename T, int BLOCK>
static void launch_greedy(const void* logits, const int32_t* draft_ids, int64_t B, int D, int64_t V,
                          const int32_t* req_index, int64_t n_req, int32_t* accepted, int32_t* accept_len,
                          int32_t* predict, int32_t* accept_index, int32_t* argmax_out, hipStream_t stream) {
    hipLaunchKernelGGL((greedy_verify_kernel<T, BLOCK>), dim3((unsigned)n_req), dim3(BLOCK), 0, stream,
                       static_cast<const T*>(logits), draft_ids, B, D, V, req_index, accepted, accept_len, predict,
                       accept_index, argmax_out);
}

hipError_t launch_greedy_verify(const void* logits, int dtype, const int32_t* draft_ids, int64_t B, int D,
                                int64_t V, const int32_t* req_index, int64_t n_req, int32_t* accepted,
                                int32_t* accept_len, int32_t* predict, int32_t* accept_index,
                                int32_t* argmax_out, hipStream_t stream) {
    const bool half = n_req >= 2 * (int64_t)greedy_device_cus();
    if (dtype == kDtypeBF16) {
        if (half)
            launch_greedy<uint16_t, 512>(logits, draft_ids, B, D, V, req_index, n_req, accepted, accept_len, predict,
                                         accept_index, argmax_out, stream);
        else
            launch_greedy<uint16_t, 1024>(logits, draft_ids, B, D, V, req_index, n_req, accepted, accept_len, predict,
                                          accept_index, argmax_out, stream);
    } else {
        if (half)
            launch_greedy<float, 512>(logits, draft_ids, B, D, V, req_index, n_req, accepted, accept_len, predict,
                                      accept_index, argmax_out, stream);
        else
            launch_greedy<float, 1024>(logits, draft_ids, B, D, V, req_index, n_req, accepted, accept_len, predict,
                                       accept_index, argmax_out, stream);
    }
    return hipGetLastError();
}

}  // namespace sv
