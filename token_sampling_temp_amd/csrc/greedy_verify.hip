// Greedy chain verify: target token y_j = lowest-index argmax of row j; the
// accept length L counts the leading draft ids equal to y (strict acceptance).
// Two forms: one workgroup per request walking its rows in order and stopping
// after the first mismatch (no workspace), or, with a workspace, one
// workgroup per (request, row) with rows after a mismatch skipped through the
// request's stop word (sv_rowpar.hpp).  Every row is read when every row's
// argmax is requested.
#include "sv_argmax.hpp"
#include "sv_launch.hpp"
#include "sv_rowpar.hpp"

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

// Row-parallel form: workgroup g takes row j = g / n_req of request slot
// g % n_req.
template <typename T, int kGreedyBlock>
__global__ __launch_bounds__(kGreedyBlock) void greedy_rows_kernel(
    const T* __restrict__ logits, const int32_t* __restrict__ draft_ids, int64_t B, int D, int64_t V,
    const int32_t* __restrict__ req_index, int64_t n_req, void* __restrict__ ws, int32_t* __restrict__ accepted,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ predict, int32_t* __restrict__ accept_index,
    int32_t* __restrict__ argmax_out) {
    __shared__ ArgmaxShared<kGreedyBlock> sh;
    __shared__ uint32_t s_stop;
    const int N = D + 1;
    const int j = (int)(blockIdx.x / (uint64_t)n_req);
    const int64_t slot = (int64_t)blockIdx.x - (int64_t)j * n_req;
    const int64_t b = req_index ? (int64_t)req_index[slot] : slot;
    if (b < 0 || b >= B) return;
    const RowPar rp(ws, slot);
    const int32_t xj = j < D ? draft_ids[b * D + j] : -1;
    // the request's last workgroup writes the outputs
    auto finish = [&](int L, int32_t yt) {
        const int t = threadIdx.x;
        if (t < N) {
            const int64_t o = b * N + t;
            const int32_t v = t <= L ? yt : -1;
            accepted[o] = v;
            if (predict) predict[o] = v;
            if (accept_index) accept_index[o] = t <= L ? (int32_t)o : -1;
            if (argmax_out) argmax_out[o] = yt;
        }
        if (t == 0) accept_len[b] = L;
    };
    // row 0 is always needed, and every row when every argmax is asked for;
    // another row whose request already ended before it counts itself in and
    // leaves at once, else it stops as soon as an earlier row ends the chain
    const bool may_stop = !argmax_out && j > 0;
    if (threadIdx.x == 0)
        s_stop = may_stop && (__hip_atomic_load(rp.word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) &
                              (((uint64_t)1 << j) - 1)) != 0;
    __syncthreads();
    if (s_stop) {
        if (threadIdx.x >= kWave) return;
        int32_t yt = -1;
        const int L = rp.arrive(j, N, false, 0, yt);
        if (L >= 0) finish(L, yt);
        return;
    }
    RowStop stop(may_stop ? rp.word : nullptr, ((uint64_t)1 << j) - 1, &s_stop, false);
    const int64_t y = row_argmax<kGreedyBlock, true, T, true>(logits + ((int64_t)b * N + j) * V, V, sh, &stop);
    if (threadIdx.x >= kWave) return;
    int32_t yt = -1;
    const int L = rp.arrive(j, N, j == D || xj != (int32_t)y, (int32_t)y, yt);
    if (L >= 0) finish(L, yt);
}

template <typename T, int BLOCK>
static void launch_greedy(const void* logits, const int32_t* draft_ids, int64_t B, int D, int64_t V,
                          const int32_t* req_index, int64_t n_req, void* ws, int32_t* accepted, int32_t* accept_len,
                          int32_t* predict, int32_t* accept_index, int32_t* argmax_out, hipStream_t stream) {
    // One workgroup per row: 512-thread workgroups also take 60 KB of LDS
    // they do not use, so at most two share a CU.  Rows are dispatched in row
    // order, so rows 0 and 1 of every request run first; with up to four per
    // CU, rows 2 and 3 ran beside them before the rows' stops could show
    // (mixed batch, 256 requests x 8 rows: 66-69 us against 68-71 us).
    if (ws)
        hipLaunchKernelGGL((greedy_rows_kernel<T, BLOCK>), dim3((unsigned)(n_req * (D + 1))), dim3(BLOCK),
                           BLOCK == 512 ? 60 * 1024 : 0, stream, static_cast<const T*>(logits), draft_ids, B, D, V,
                           req_index, n_req, ws, accepted, accept_len, predict, accept_index, argmax_out);
    else
        hipLaunchKernelGGL((greedy_verify_kernel<T, BLOCK>), dim3((unsigned)n_req), dim3(BLOCK), 0, stream,
                           static_cast<const T*>(logits), draft_ids, B, D, V, req_index, accepted, accept_len,
                           predict, accept_index, argmax_out);
}

int64_t greedy_workspace_bytes(int64_t n_req, int D) {
    return (D > 0 && n_req > 0) ? rowpar_workspace_bytes(n_req) : 0;
}

hipError_t launch_greedy_verify(const void* logits, int dtype, const int32_t* draft_ids, int64_t B, int D,
                                int64_t V, const int32_t* req_index, int64_t n_req, int32_t* accepted,
                                int32_t* accept_len, int32_t* predict, int32_t* accept_index,
                                int32_t* argmax_out, void* workspace, hipStream_t stream) {
    const int64_t cus = device_compute_units();
    // a batch of at least two requests per CU keeps every CU busy one request
    // per workgroup; smaller batches spread each request's rows over CUs
    void* ws = (greedy_workspace_bytes(n_req, D) > 0 && n_req < 2 * cus) ? workspace : nullptr;
    // rows in flight: one per request, or one per (request, row)
    const int64_t units = ws ? n_req * (D + 1) : n_req;
    const bool half = units >= 2 * cus;
    if (dtype == kDtypeBF16) {
        if (half)
            launch_greedy<uint16_t, 512>(logits, draft_ids, B, D, V, req_index, n_req, ws, accepted, accept_len,
                                         predict, accept_index, argmax_out, stream);
        else
            launch_greedy<uint16_t, 1024>(logits, draft_ids, B, D, V, req_index, n_req, ws, accepted, accept_len,
                                          predict, accept_index, argmax_out, stream);
    } else {
        if (half)
            launch_greedy<float, 512>(logits, draft_ids, B, D, V, req_index, n_req, ws, accepted, accept_len,
                                      predict, accept_index, argmax_out, stream);
        else
            launch_greedy<float, 1024>(logits, draft_ids, B, D, V, req_index, n_req, ws, accepted, accept_len,
                                       predict, accept_index, argmax_out, stream);
    }
    return hipGetLastError();
}

}  // namespace sv
