// Ceiling probes of gfx950 (declared in include/moe_probes.h): a streaming HBM read and a
// register-only bf16 MFMA loop.  Neither is a step of the MoE path; they measure what the chip
// delivers, for comparison with the path's roofline figures.
#include "device_common.h"
#include "launchers.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void probe_stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                uint32_t* __restrict__ sink) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    uint32_t acc = 0;
    // four independent 16-byte loads in flight per iteration
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
    }
    for (; i < n16; i += stride) {
        const u32x4 a = src[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    sink[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = acc;
}

// pseudo-random bf16 operand: random sign and mantissa, exponent field 0x78..0x7F (2^-7 .. 2^0),
// so products stay finite and the accumulators never overflow over the loop
__device__ __forceinline__ bf16x8 probe_operand(uint32_t seed) {
    uint32_t h = seed * 0x9E3779B9u + 0x7F4A7C15u;
    typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
    u16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        h ^= h >> 15; h *= 0x2C1B3C6Du; h ^= h >> 12; h *= 0x297A2D39u; h ^= h >> 15;
        v[i] = static_cast<uint16_t>((h & 0x807Fu) | (0x3C00u + ((h >> 8) & 0x380u)));
    }
    return __builtin_bit_cast(bf16x8, v);
}

__global__ __launch_bounds__(256) void probe_mfma_bf16_kernel(int64_t iters, float* __restrict__ sink) {
    const uint32_t tid = blockIdx.x * 256 + threadIdx.x;
    bf16x8 a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) { a[j] = probe_operand(tid * 8 + j); b[j] = probe_operand(tid * 8 + 4 + j); }
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;
    for (int64_t it = 0; it < iters; ++it) {
        // 8 MFMAs on 4 independent accumulators; each instruction takes another operand pair
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[(j + 1) & 3], acc[j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(j + 2) & 3], b[j], acc[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[j][v];
    sink[tid] = s;
}

}  // namespace

hipError_t launch_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int blocks, hipStream_t s) {
    probe_stream_read_kernel<<<blocks, 256, 0, s>>>(static_cast<const u32x4*>(src), bytes / 16, sink);
    return hipGetLastError();
}

hipError_t launch_probe_mfma_bf16(int64_t iters, float* sink, int blocks, hipStream_t s) {
    probe_mfma_bf16_kernel<<<blocks, 256, 0, s>>>(iters, sink);
    return hipGetLastError();
}

}  // namespace moe
