// FP8 prefill variant of the grouped expert GEMMs (atlas moe_lora_grouped.rs module doc: fp8,
// like bf16, is a grouped prefill path that writes the same sorted BF16 expert_down_out).  The
// page fixes no format, so the reading is: OCP FP8 E4M3 weights [E, N, K] with one fp32 scale
// per output channel [E, N], and activations quantised per row at run time:
//   quantize_fp8_kernel   (this file) amax of a bf16 row; s = amax / 448 (dequantisation scale)
//                         and f = 448 / amax in fp32; codes = e4m3(x * f), round to nearest even
//   the GEMMs             (gemm_bf16.hip, its fp8 form) acc = sum_k a(r, k) w(n, k) over the e4m3
//                         values (products exact, fp32 sums) on the CDNA4 32x32x64 fp8 MFMA;
//                         out = acc * s_a[row] * s_w[n], then SiLU(gate) * up (gate/up) or the
//                         plain value (down), to bf16.  The tiles are the bf16 ones in bytes.
#include "device_common.h"
#include "launchers.h"

namespace moe {
namespace {

// ------------------------------------------------------------------ per-row quantisation
constexpr int kQThreads = 256;

// NC > 0: each thread holds its NC 16-byte chunks of the row in registers (rows of at most
// NC * 2048 elements), all loaded at once, so the row is read once and every load of a workgroup is
// in flight together; NC == 0: any K, the row read twice (the second pass mostly from L2).
template <int NC>
__global__ __launch_bounds__(kQThreads) void quantize_fp8_kernel(const uint16_t* __restrict__ x,
                                                                 uint8_t* __restrict__ q, float* __restrict__ scale,
                                                                 const int32_t* __restrict__ sorted_ids, int P,
                                                                 int K) {
    __shared__ float s_max[kQThreads / 64];
    const int64_t r = blockIdx.x;
    if (sorted_ids) {
        const int p = sorted_ids[r];
        if (p < 0 || p >= P) return;  // uniform over the workgroup
    }
    const uint16_t* xr = x + r * K;
    auto absmax8 = [](float m, const u32x4& v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            m = fmaxf(m, fabsf(__uint_as_float(v[i] << 16)));
            m = fmaxf(m, fabsf(__uint_as_float(v[i] & 0xffff0000u)));
        }
        return m;
    };
    // codes of 8 elements, element 0 in the lowest byte
    auto codes8 = [](const u32x4& v, float f) {
        uint32_t w[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            int pk = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(v[2 * h] << 16) * f,
                                                     __uint_as_float(v[2 * h] & 0xffff0000u) * f, 0, false);
            pk = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(v[2 * h + 1] << 16) * f,
                                                 __uint_as_float(v[2 * h + 1] & 0xffff0000u) * f, pk, true);
            w[h] = static_cast<uint32_t>(pk);
        }
        return make_uint2(w[0], w[1]);
    };
    float amax = 0.f;
    u32x4 v[NC > 0 ? NC : 1];
    if constexpr (NC > 0) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int c = (threadIdx.x + i * kQThreads) * 8;
            v[i] = c < K ? *reinterpret_cast<const u32x4*>(xr + c) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < NC; ++i) amax = absmax8(amax, v[i]);
    } else {
        for (int c = threadIdx.x * 8; c < K; c += kQThreads * 8)
            amax = absmax8(amax, *reinterpret_cast<const u32x4*>(xr + c));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    const float f = amax > 0.f ? 448.0f / amax : 1.0f;
    if (threadIdx.x == 0) scale[r] = amax > 0.f ? amax / 448.0f : 1.0f;
    uint8_t* qr = q + r * K;
    if constexpr (NC > 0) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int c = (threadIdx.x + i * kQThreads) * 8;
            if (c < K) *reinterpret_cast<uint2*>(qr + c) = codes8(v[i], f);
        }
    } else {
        for (int c = threadIdx.x * 8; c < K; c += kQThreads * 8)
            *reinterpret_cast<uint2*>(qr + c) = codes8(*reinterpret_cast<const u32x4*>(xr + c), f);
    }
}

}  // namespace

hipError_t launch_quantize_fp8(const uint16_t* x, int64_t rows, int K, const int32_t* sorted_ids, int P,
                               uint8_t* q, float* scale, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    const int chunks = (K + kQThreads * 8 - 1) / (kQThreads * 8);  // 16-byte chunks per thread
    const dim3 g(static_cast<unsigned>(rows));
    if (chunks <= 1) quantize_fp8_kernel<1><<<g, kQThreads, 0, s>>>(x, q, scale, sorted_ids, P, K);
    else if (chunks <= 2) quantize_fp8_kernel<2><<<g, kQThreads, 0, s>>>(x, q, scale, sorted_ids, P, K);
    else if (chunks <= 4) quantize_fp8_kernel<4><<<g, kQThreads, 0, s>>>(x, q, scale, sorted_ids, P, K);
    else if (chunks <= 8) quantize_fp8_kernel<8><<<g, kQThreads, 0, s>>>(x, q, scale, sorted_ids, P, K);
    else quantize_fp8_kernel<0><<<g, kQThreads, 0, s>>>(x, q, scale, sorted_ids, P, K);
    return hipGetLastError();
}

}  // namespace moe
