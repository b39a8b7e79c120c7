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
    float amax = 0.f;
    for (int c = threadIdx.x * 8; c < K; c += kQThreads * 8) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(xr + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            amax = fmaxf(amax, fabsf(__uint_as_float(v[i] << 16)));
            amax = fmaxf(amax, fabsf(__uint_as_float(v[i] & 0xffff0000u)));
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    const float f = amax > 0.f ? 448.0f / amax : 1.0f;
    if (threadIdx.x == 0) scale[r] = amax > 0.f ? amax / 448.0f : 1.0f;
    uint8_t* qr = q + r * K;
    for (int c = threadIdx.x * 8; c < K; c += kQThreads * 8) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(xr + c);
        uint32_t w[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // codes of elements 4h .. 4h+3, element 4h in the lowest byte
            int pk = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(v[2 * h] << 16) * f,
                                                     __uint_as_float(v[2 * h] & 0xffff0000u) * f, 0, false);
            pk = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(v[2 * h + 1] << 16) * f,
                                                 __uint_as_float(v[2 * h + 1] & 0xffff0000u) * f, pk, true);
            w[h] = static_cast<uint32_t>(pk);
        }
        *reinterpret_cast<uint2*>(qr + c) = make_uint2(w[0], w[1]);
    }
}

}  // namespace

hipError_t launch_quantize_fp8(const uint16_t* x, int64_t rows, int K, const int32_t* sorted_ids, int P,
                               uint8_t* q, float* scale, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    quantize_fp8_kernel<<<static_cast<unsigned>(rows), kQThreads, 0, s>>>(x, q, scale, sorted_ids, P, K);
    return hipGetLastError();
}

}  // namespace moe
