// Top-k weighted combine (ferrum-kernels cuda/moe.rs, moe_combine and
// weighted_sum_batched): out[t] = bf16(sum_j w[t,j] * ys[row(t,j)]), fp32, j ascending.
//
// HBM-bound gather: one workgroup per (token, 2048-column slab); each lane owns
// eight consecutive columns and issues one 16-byte load per expert row, so the
// top_k row loads of a lane are all in flight together.
#include "device_common.h"
#include "launchers.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kCols = kThreads * 8;

__global__ __launch_bounds__(kThreads) void combine_kernel(const uint16_t* __restrict__ ys,
                                                           const int32_t* __restrict__ inv,
                                                           const float* __restrict__ w, uint16_t* __restrict__ out,
                                                           int k, int H, int64_t ys_rows) {
    const int t = blockIdx.x;
    const int col = blockIdx.y * kCols + threadIdx.x * 8;
    if (col >= H) return;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int j = 0; j < k; ++j) {
        const int64_t slot = static_cast<int64_t>(t) * k + j;
        const int64_t row = inv ? static_cast<int64_t>(inv[slot]) : slot;
        if (row < 0 || row >= ys_rows) continue;
        const float wt = w[slot];
        const u32x4 v = *reinterpret_cast<const u32x4*>(ys + row * H + col);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = fmaf(wt, __uint_as_float(v[i] << 16), acc[2 * i]);
            acc[2 * i + 1] = fmaf(wt, __uint_as_float(v[i] & 0xffff0000u), acc[2 * i + 1]);
        }
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    *reinterpret_cast<u32x4*>(out + static_cast<int64_t>(t) * H + col) = o;
}

}  // namespace

hipError_t launch_combine(const uint16_t* ys, const int32_t* inv, const float* w, uint16_t* out, int T, int k,
                          int H, int64_t ys_rows, hipStream_t s) {
    const dim3 grid(T, (H + kCols - 1) / kCols), block(kThreads);
    combine_kernel<<<grid, block, 0, s>>>(ys, inv, w, out, k, H, ys_rows);
    return hipGetLastError();
}

}  // namespace moe
