// Top-k softmax router (ferrum-kernels cuda/moe.rs, route_topk_softmax): per token,
// softmax over all experts, keep the top_k, optionally renormalise over them.  One wave64
// per token, four tokens per 256-thread block; the per-token body is route_tokens
// (route_common.h).  With at most 16 experts, one token per 16-lane row (route_row_token).
#include "launchers.h"
#include "route_common.h"

namespace moe {
namespace {

template <int EPL>
__global__ __launch_bounds__(256) void route_topk_softmax_kernel(const float* __restrict__ logits, int T, int E,
                                                                 int top_k, int renorm, int32_t* __restrict__ ids,
                                                                 float* __restrict__ w) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // whole wave leaves; no block-level barrier below
    route_tokens<EPL, 1>(logits, t, 0, T, E, top_k, renorm, ids, w, threadIdx.x & 63);
}

// E <= 16: one token per 16-lane row, sixteen tokens per 256-thread block
__global__ __launch_bounds__(256) void route_rows_kernel(const float* __restrict__ logits, int T, int E, int top_k,
                                                         int renorm, int32_t* __restrict__ ids,
                                                         float* __restrict__ w) {
    const int t0 = blockIdx.x * 16 + (threadIdx.x >> 6) * 4;
    if (t0 >= T) return;  // whole wave leaves; no block-level barrier below
    route_row_token(logits, t0 + ((threadIdx.x & 63) >> 4), T, E, top_k, renorm, ids, w, threadIdx.x & 63);
}

}  // namespace

hipError_t launch_route(const float* logits, int T, int E, int top_k, int renorm, int32_t* ids, float* w,
                        hipStream_t s) {
    if (E <= 16) {
        route_rows_kernel<<<(T + 15) / 16, 256, 0, s>>>(logits, T, E, top_k, renorm, ids, w);
        return hipGetLastError();
    }
    const dim3 grid((T + 3) / 4), block(256);
    const int epl = (E + 63) / 64;
    switch (epl) {
        case 1: route_topk_softmax_kernel<1><<<grid, block, 0, s>>>(logits, T, E, top_k, renorm, ids, w); break;
        case 2: route_topk_softmax_kernel<2><<<grid, block, 0, s>>>(logits, T, E, top_k, renorm, ids, w); break;
        case 3: route_topk_softmax_kernel<3><<<grid, block, 0, s>>>(logits, T, E, top_k, renorm, ids, w); break;
        default: route_topk_softmax_kernel<4><<<grid, block, 0, s>>>(logits, T, E, top_k, renorm, ids, w); break;
    }
    return hipGetLastError();
}

}  // namespace moe
