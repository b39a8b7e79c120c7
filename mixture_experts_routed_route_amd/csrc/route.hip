// Top-k softmax router (ferrum-kernels cuda/moe.rs, route_topk_softmax): per token,
// softmax over all experts, keep the top_k, optionally renormalise over them.
//
// One wave64 per token, four tokens per 256-thread block.  Each lane holds up to
// four logits (E <= 256) in registers.  Selection takes top_k rounds of a wave
// arg-max over a 64-bit key (order-preserving image of the fp32 logit, then the
// complement of the expert index, so equal logits pick the lower index).  The
// weights are computed in fp64 and rounded once to fp32.
#include "device_common.h"
#include "launchers.h"

namespace moe {
namespace {

__device__ __forceinline__ uint32_t order_bits(float v) {
    v = (v == 0.0f) ? 0.0f : v;  // -0.0 and +0.0 compare equal
    uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_order_bits(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint64_t o = __shfl_xor(v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

template <int EPL>
__global__ __launch_bounds__(256) void route_topk_softmax_kernel(const float* __restrict__ logits, int T, int E,
                                                                 int top_k, int renorm, int32_t* __restrict__ ids,
                                                                 float* __restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // whole wave leaves; no block-level barrier below
    const float* row = logits + static_cast<size_t>(t) * E;

    float v[EPL];
    uint64_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        if (e < E) {
            v[i] = row[e];
            key[i] = (static_cast<uint64_t>(order_bits(v[i])) << 32) | static_cast<uint32_t>(0xffff - e);
        } else {
            v[i] = 0.0f;
            key[i] = 0;  // below every real key
        }
    }

    int my_e = 0;
    float my_l = 0.0f, top = 0.0f;
    for (int j = 0; j < top_k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < EPL; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
        const int e = 0xffff - static_cast<int>(best & 0xffffu);
        const float l = from_order_bits(static_cast<uint32_t>(best >> 32));
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (lane + 64 * i == e) key[i] = 0;
        if (j == 0) top = l;
        if (lane == j) { my_e = e; my_l = l; }
    }

    // softmax denominator over every expert, fp64
    const double m = static_cast<double>(top);
    double part = 0.0;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
        if (lane + 64 * i < E) part += exp(static_cast<double>(v[i]) - m);
    const double S = wave_sum_f64(part);

    const double p = exp(static_cast<double>(my_l) - m) / S;
    double den = 0.0;
    for (int j = 0; j < top_k; ++j) den += __shfl(p, j, 64);
    if (lane < top_k) {
        const double wj = renorm ? p / den : p;
        ids[static_cast<size_t>(t) * top_k + lane] = my_e;
        w[static_cast<size_t>(t) * top_k + lane] = static_cast<float>(wj);
    }
}

}  // namespace

hipError_t launch_route(const float* logits, int T, int E, int top_k, int renorm, int32_t* ids, float* w,
                        hipStream_t s) {
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
