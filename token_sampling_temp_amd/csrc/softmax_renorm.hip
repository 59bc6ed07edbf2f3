// Temperature softmax with top-k then top-p renormalisation (the row
// algorithms are in sv_softmax.hpp).  bf16 rows that fit the register-resident
// path go to one persistent workgroup per CU; other rows get one workgroup per
// (request, position) row, streamed.  T < 1e-5 writes a one-hot at the
// lowest-index argmax.
#include "sv_launch.hpp"
#include "sv_softmax.hpp"

namespace sv {

template <typename T>
__global__ __launch_bounds__(kSmBlock) void softmax_renorm_kernel(
    const T* __restrict__ logits, int64_t B, int npos, int64_t V, const float* __restrict__ temperature,
    const int32_t* __restrict__ top_k, const float* __restrict__ top_p, const int32_t* __restrict__ req_index,
    float* __restrict__ out) {
    __shared__ SmShared sh;
    const int64_t b = req_index ? (int64_t)req_index[blockIdx.x] : (int64_t)blockIdx.x;
    if (b < 0 || b >= B) return;
    const int64_t r = (int64_t)b * npos + blockIdx.y;
    softmax_row_streamed<T>(logits + r * V, out + r * V, V, temperature[b], top_k ? top_k[b] : 0,
                            top_p ? top_p[b] : 1.0f, sh);
}

// Persistent: workgroup g handles rows g, g + gridDim.x, ... of the
// n_req * npos rows (request-major).  Rows the register-resident path does
// not take (one-hot rows, unaligned rows, overflowed counters) are queued in
// LDS and redone by the streamed algorithm after the loop, so that code is
// not part of the loop that keeps a row in registers.
constexpr int kDeferMax = 512;

struct RrKernelShared {
    RrShared rr;
    int64_t defer[kDeferMax];
    uint32_t ndefer;
};

template <int NV>
__global__ __launch_bounds__(kRrBlock) void softmax_renorm_rr_kernel(
    const uint16_t* __restrict__ logits, int64_t B, int npos, int64_t V, const float* __restrict__ temperature,
    const int32_t* __restrict__ top_k, const float* __restrict__ top_p, const int32_t* __restrict__ req_index,
    int64_t n_req, float* __restrict__ out) {
    __shared__ RrKernelShared ks;
    const int64_t n_rows = n_req * npos;
    if (threadIdx.x == 0) ks.ndefer = 0;
    auto locate = [&](int64_t item, int64_t& b, int64_t& r) {
        const int64_t q = item / npos;
        b = req_index ? (int64_t)req_index[q] : q;
        r = b * npos + (item - q * npos);
        return b >= 0 && b < B;
    };
    for (int64_t item = blockIdx.x; item < n_rows; item += gridDim.x) {
        int64_t b, r;
        if (!locate(item, b, r)) continue;
        const uint16_t* row = logits + r * V;
        float* orow = out + r * V;
        const float Tm = temperature[b];
        bool done = false;
        if ((double)Tm >= kGreedyTemperature && (((uintptr_t)row | (uintptr_t)orow) & 15u) == 0 && (V & 7) == 0)
            done = rr_row<NV>(ks.rr, row, orow, V, Tm, top_k ? top_k[b] : 0, top_p ? top_p[b] : 1.0f);
        if (!done && threadIdx.x == 0) {
            const uint32_t i = ks.ndefer++;
            if (i < (uint32_t)kDeferMax) ks.defer[i] = item;
        }
    }
    __syncthreads();
    const uint32_t nd = ks.ndefer;
    // more deferred rows than the queue holds: redo every row of this workgroup
    const int64_t n_redo = nd <= (uint32_t)kDeferMax ? (int64_t)nd : (n_rows - blockIdx.x + gridDim.x - 1) / gridDim.x;
    for (int64_t i = 0; i < n_redo; ++i) {
        const int64_t item = nd <= (uint32_t)kDeferMax ? ks.defer[i] : blockIdx.x + i * gridDim.x;
        int64_t b, r;
        if (!locate(item, b, r)) continue;
        __syncthreads();
        softmax_row_streamed<uint16_t>(logits + r * V, out + r * V, V, temperature[b], top_k ? top_k[b] : 0,
                                       top_p ? top_p[b] : 1.0f, ks.rr.u.sm);
    }
}

// Largest register-resident row: 1024 threads x 8 x 20 = 163840 bf16 entries.
constexpr int kRrMaxNV = 20;

template <int NV>
static void launch_rr(unsigned grid, hipStream_t stream, const uint16_t* logits, int64_t B, int npos, int64_t V,
                      const float* temperature, const int32_t* top_k, const float* top_p, const int32_t* req_index,
                      int64_t n_req, float* out) {
    hipLaunchKernelGGL(softmax_renorm_rr_kernel<NV>, dim3(grid), dim3(kRrBlock), 0, stream, logits, B, npos, V,
                       temperature, top_k, top_p, req_index, n_req, out);
}

hipError_t launch_softmax_renorm(const void* logits, int dtype, int64_t B, int64_t npos, int64_t V,
                                 const float* temperature, const int32_t* top_k, const float* top_p,
                                 const int32_t* req_index, int64_t n_req, float* probs_out,
                                 hipStream_t stream) {
    const dim3 grid((unsigned)n_req, (unsigned)npos), block(kSmBlock);
    if (dtype == kDtypeBF16 && V <= (int64_t)kRrBlock * 8 * kRrMaxNV) {
        // one persistent workgroup per compute unit (the LDS footprint allows no more)
        const int64_t rows = n_req * npos;
        const unsigned g = (unsigned)(rows < (int64_t)device_compute_units() ? rows : (int64_t)device_compute_units());
        const int64_t nv = (V + kRrBlock * 8 - 1) / (kRrBlock * 8);
        const uint16_t* lg = static_cast<const uint16_t*>(logits);
        const int np = (int)npos;
        if (nv <= 1) launch_rr<1>(g, stream, lg, B, np, V, temperature, top_k, top_p, req_index, n_req, probs_out);
        else if (nv <= 2) launch_rr<2>(g, stream, lg, B, np, V, temperature, top_k, top_p, req_index, n_req, probs_out);
        else if (nv <= 4) launch_rr<4>(g, stream, lg, B, np, V, temperature, top_k, top_p, req_index, n_req, probs_out);
        else if (nv <= 8) launch_rr<8>(g, stream, lg, B, np, V, temperature, top_k, top_p, req_index, n_req, probs_out);
        else if (nv <= 12) launch_rr<12>(g, stream, lg, B, np, V, temperature, top_k, top_p, req_index, n_req, probs_out);
        else if (nv <= 16) launch_rr<16>(g, stream, lg, B, np, V, temperature, top_k, top_p, req_index, n_req, probs_out);
        else launch_rr<20>(g, stream, lg, B, np, V, temperature, top_k, top_p, req_index, n_req, probs_out);
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
