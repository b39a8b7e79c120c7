// SiLU(gate) * up between the gate/up GEMM and its LoRA folds on one side and the down GEMM on
// the other (atlas moe_lora_grouped.rs, moe_lora_gather_bgmv: the caller's moe_silu_mul into a
// BF16 buffer): h[r] = bf16(silu(g[r]) * u[r]) from the bf16 gate and up rows, for the real
// sorted rows r (sorted_ids[r] in [0, P); every row when sorted_ids is NULL).  Other rows are
// not written.  HBM-bound: one workgroup per (row, 2048 columns), 16-byte accesses.
#include "device_common.h"
#include "launchers.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kCols = kThreads * 8;

__global__ __launch_bounds__(kThreads) void silu_mul_kernel(const uint16_t* __restrict__ g,
                                                            const uint16_t* __restrict__ u,
                                                            uint16_t* __restrict__ h,
                                                            const int32_t* __restrict__ sorted_ids, int P, int N) {
    const int64_t r = blockIdx.x;
    const int col = blockIdx.y * kCols + threadIdx.x * 8;
    if (col >= N) return;
    if (sorted_ids) {
        const int p = sorted_ids[r];
        if (p < 0 || p >= P) return;
    }
    const int64_t off = r * N + col;
    const u32x4 gv = *reinterpret_cast<const u32x4*>(g + off);
    const u32x4 uv = *reinterpret_cast<const u32x4*>(u + off);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = pack_bf16x2(silu_mul(__uint_as_float(gv[i] << 16), __uint_as_float(uv[i] << 16)),
                           silu_mul(__uint_as_float(gv[i] & 0xffff0000u), __uint_as_float(uv[i] & 0xffff0000u)));
    *reinterpret_cast<u32x4*>(h + off) = o;
}

}  // namespace

hipError_t launch_silu_mul(const uint16_t* g, const uint16_t* u, uint16_t* h, const int32_t* sorted_ids, int P,
                           int64_t rows, int N, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(rows), (N + kCols - 1) / kCols), block(kThreads);
    silu_mul_kernel<<<grid, block, 0, s>>>(g, u, h, sorted_ids, P, N);
    return hipGetLastError();
}

}  // namespace moe
