// Per-token top-k softmax routing body, shared by the router kernel and the fused
// route+align kernel (ferrum-kernels cuda/moe.rs, route_topk_softmax): softmax over all
// experts, keep the top_k, optionally renormalise over them.
//
// One wave64 per token.  Each lane holds up to four logits (E <= 256) in registers.
// Selection takes top_k rounds of a wave arg-max: a 32-bit wave max of an order-preserving
// image of the fp32 logit, then a ballot of the lanes that hold it, slot by slot, whose lowest
// set bit is the lowest expert index (so equal logits pick the lower index).  Selection j is
// kept by lane j % 64 in its slot j / 64, so top_k may reach E (up to 256).  The weights are
// computed in fp64 and rounded once to fp32.  With at most 16 experts, route_row_token takes one
// token per 16-lane row instead, with the same results.
#pragma once

#include "device_common.h"

namespace moe {

__device__ __forceinline__ uint32_t order_bits(float v) {
    v = (v == 0.0f) ? 0.0f : v;  // -0.0 and +0.0 compare equal
    uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_order_bits(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

// Cross-lane reductions over a wave64 without LDS round trips: inside each 16-lane row, DPP
// row rotations by 1, 2, 4 and 8 leave the row's result in every lane; the four row results
// are then read from lanes 0, 16, 32 and 48.
template <int N>
__device__ __forceinline__ uint64_t row_ror_u64(uint64_t v) {
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        0, static_cast<int>(static_cast<uint32_t>(v)), 0x120 + N, 0xF, 0xF, false));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        0, static_cast<int>(static_cast<uint32_t>(v >> 32)), 0x120 + N, 0xF, 0xF, false));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), l);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), l);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x121, 0xF, 0xF, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x122, 0xF, 0xF, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x124, 0xF, 0xF, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x128, 0xF, 0xF, false)));
    const uint32_t a = max(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 0)),
                           static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 16)));
    const uint32_t b = max(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 32)),
                           static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 48)));
    return max(a, b);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
    v += __builtin_bit_cast(double, row_ror_u64<1>(__builtin_bit_cast(uint64_t, v)));
    v += __builtin_bit_cast(double, row_ror_u64<2>(__builtin_bit_cast(uint64_t, v)));
    v += __builtin_bit_cast(double, row_ror_u64<4>(__builtin_bit_cast(uint64_t, v)));
    v += __builtin_bit_cast(double, row_ror_u64<8>(__builtin_bit_cast(uint64_t, v)));
    return (__builtin_bit_cast(double, readlane_u64(__builtin_bit_cast(uint64_t, v), 0)) +
            __builtin_bit_cast(double, readlane_u64(__builtin_bit_cast(uint64_t, v), 16))) +
           (__builtin_bit_cast(double, readlane_u64(__builtin_bit_cast(uint64_t, v), 32)) +
            __builtin_bit_cast(double, readlane_u64(__builtin_bit_cast(uint64_t, v), 48)));
}

// Route NTOK tokens t0, t0+dt, ... (those below T), called by all 64 lanes of one wave: writes
// ids/w[t*top_k .. +top_k) of each, and the ids also to lds_ids[] when it is given.  The tokens'
// selection rounds are independent, so their cross-lane reductions interleave and hide each
// other's latency.
template <int EPL, int NTOK>
__device__ __forceinline__ void route_tokens(const float* __restrict__ logits, int t0, int dt, int T, int E,
                                             int top_k, int renorm, int32_t* __restrict__ ids,
                                             float* __restrict__ w, int lane, int* lds_ids = nullptr) {
    float v[NTOK][EPL];
    uint32_t key[NTOK][EPL];  // order bits of the logit; 0: not a candidate (taken, or past E)
#pragma unroll
    for (int n = 0; n < NTOK; ++n) {
        const int t = t0 + n * dt;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            if (t < T && e < E) {
                v[n][i] = logits[static_cast<size_t>(t) * E + e];
                key[n][i] = order_bits(v[n][i]);  // > 0 for every finite logit
            } else {
                v[n][i] = 0.0f;
                key[n][i] = 0;  // below every real key
            }
        }
    }

    // selection j lives in lane j % 64, slot j / 64 (top_k <= E <= 64 * EPL)
    int my_e[NTOK][EPL];
    float my_l[NTOK][EPL], top[NTOK];
#pragma unroll
    for (int n = 0; n < NTOK; ++n) {
        top[n] = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) { my_e[n][i] = 0; my_l[n][i] = 0.0f; }
    }
    for (int j = 0; j < top_k; ++j) {
        uint32_t best[NTOK];
#pragma unroll
        for (int n = 0; n < NTOK; ++n) {
            best[n] = key[n][0];
#pragma unroll
            for (int i = 1; i < EPL; ++i) best[n] = max(best[n], key[n][i]);
        }
#pragma unroll
        for (int n = 0; n < NTOK; ++n) best[n] = wave_max_u32(best[n]);
#pragma unroll
        for (int n = 0; n < NTOK; ++n) {
            // the lowest expert holding the largest key: slot i holds experts 64 i + lane
            int e = 0x7fffffff;
#pragma unroll
            for (int i = EPL - 1; i >= 0; --i) {
                const uint64_t hit = __ballot(key[n][i] == best[n]);
                if (hit) e = 64 * i + __ffsll(static_cast<unsigned long long>(hit)) - 1;
            }
            const float l = from_order_bits(best[n]);
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (lane + 64 * i == e) key[n][i] = 0;
            if (j == 0) top[n] = l;
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (lane + 64 * i == j) { my_e[n][i] = e; my_l[n][i] = l; }
        }
    }

#pragma unroll
    for (int n = 0; n < NTOK; ++n) {
        const int t = t0 + n * dt;
        // softmax denominator over every expert, fp64
        const double m = static_cast<double>(top[n]);
        double part = 0.0;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (lane + 64 * i < E) part += exp(static_cast<double>(v[n][i]) - m);
        const double S = wave_sum_f64(part);
        double p[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) p[i] = exp(static_cast<double>(my_l[n][i]) - m) / S;
        // the kept probabilities summed in slot order j = 0 .. top_k-1
        double den = 0.0;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            for (int l = 0; l < 64 && 64 * i + l < top_k; ++l)
                den += __builtin_bit_cast(double, readlane_u64(__builtin_bit_cast(uint64_t, p[i]), l));
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int j = lane + 64 * i;
            if (t < T && j < top_k) {
                const double wj = renorm ? p[i] / den : p[i];
                ids[static_cast<size_t>(t) * top_k + j] = my_e[n][i];
                w[static_cast<size_t>(t) * top_k + j] = static_cast<float>(wj);
                if (lds_ids != nullptr) lds_ids[t * top_k + j] = my_e[n][i];
            }
        }
    }
}

// Route one token per 16-lane row (E <= 16): four tokens per wave at once, called by all 64 lanes
// (row r of the wave takes token t_row; rows with t_row >= T only take part in the cross-lane
// steps).  Every reduction stays inside the row: DPP row rotations by 1, 2, 4 and 8 leave the
// row's result in each of its lanes.  The softmax sum is the same sequence of additions as in
// route_tokens, whose other three rows hold zeros when E <= 16, and the kept weights are summed
// in slot order as there, so the results are bit-identical to it.
__device__ __forceinline__ void route_row_token(const float* __restrict__ logits, int t_row, int T, int E,
                                                int top_k, int renorm, int32_t* __restrict__ ids,
                                                float* __restrict__ w, int lane, int* lds_ids = nullptr) {
    const int c = lane & 15, row = lane >> 4;
    const bool tok = t_row < T;
    float v = 0.0f;
    uint32_t key = 0;  // order bits of the logit; 0: not a candidate (taken, past E, or no token)
    if (tok && c < E) {
        v = logits[static_cast<size_t>(t_row) * E + c];
        key = order_bits(v);
    }
    int my_e = 0;
    float my_l = 0.0f, top = 0.0f;
    for (int j = 0; j < top_k; ++j) {
        uint32_t best = key;
        best = max(best, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(best), 0x121, 0xF, 0xF, false)));
        best = max(best, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(best), 0x122, 0xF, 0xF, false)));
        best = max(best, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(best), 0x124, 0xF, 0xF, false)));
        best = max(best, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(best), 0x128, 0xF, 0xF, false)));
        // the lowest expert of the row holding the largest key (ties: the lower index)
        const uint64_t hit = __ballot(key == best);
        const uint32_t rh = static_cast<uint32_t>(hit >> (16 * row)) & 0xffffu;
        const int e = rh ? __builtin_ctz(rh) : 0;
        const float l = from_order_bits(best);
        if (c == e) key = 0;
        if (j == 0) top = l;
        if (c == j) { my_e = e; my_l = l; }
    }
    // softmax denominator over every expert of the row's token, fp64
    const double m = static_cast<double>(top);
    double S = (tok && c < E) ? exp(static_cast<double>(v) - m) : 0.0;
    S += __builtin_bit_cast(double, row_ror_u64<1>(__builtin_bit_cast(uint64_t, S)));
    S += __builtin_bit_cast(double, row_ror_u64<2>(__builtin_bit_cast(uint64_t, S)));
    S += __builtin_bit_cast(double, row_ror_u64<4>(__builtin_bit_cast(uint64_t, S)));
    S += __builtin_bit_cast(double, row_ror_u64<8>(__builtin_bit_cast(uint64_t, S)));
    const double p = exp(static_cast<double>(my_l) - m) / S;
    // the kept probabilities summed in slot order j = 0 .. top_k-1 (lane j of the row holds slot j)
    double den = 0.0;
    for (int j = 0; j < top_k; ++j) den += __shfl(p, row * 16 + j);
    if (tok && c < top_k) {
        const double wj = renorm ? p / den : p;
        ids[static_cast<size_t>(t_row) * top_k + c] = my_e;
        w[static_cast<size_t>(t_row) * top_k + c] = static_cast<float>(wj);
        if (lds_ids != nullptr) lds_ids[t_row * top_k + c] = my_e;
    }
}

}  // namespace moe
