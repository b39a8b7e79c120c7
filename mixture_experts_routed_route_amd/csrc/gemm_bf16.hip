// Grouped expert GEMM, bf16 weights, one launch for all experts (the grouped gate/up and
// down roles of metrale cutlass/grouped.rs; gather through sorted ids and sentinel masking
// as in ferrum-kernels triton_fused_moe.rs).
//
// Tiling.  A tile is up to BM = 128 consecutive sorted rows of ONE expert: expert e's
// padded span [off[e], off[e+1]) is cut into ceil(span/128) tiles.  Each workgroup
// rebuilds that tile list from expert_offsets (a 256-wide LDS scan of the per-expert tile
// counts), so the grid is a static worst-case bound (ceil(max_pad/128) + E tiles per
// column panel) and tiles past the end exit at once.  The weight panel of a tile is
// BP = 256 weight rows: for gate/up, 128 gate rows and the 128 up rows of the same output
// columns (so SiLU(gate)*up is formed in registers); for down, 256 output columns.
//
// Schedule.  256 threads = 4 waves in a 2x2 grid; each wave owns 64 rows x 128 panel rows
// (4 x 8 MFMA 16x16x32 bf16 tiles, fp32 accumulators).  K advances 64 at a time through a
// double-buffered LDS stage (A 16 KB + B 32 KB per stage, rows XOR-swizzled in 16-byte
// chunks so the 16-byte fragment reads of one MFMA spread over the banks); the global
// loads of the next stage are issued before the MFMAs of the current one.  Workgroup ids
// are remapped so that each XCD (ids are dealt round-robin over the 8 XCDs) runs a
// contiguous range of tiles, and consecutive tiles share a weight panel (row tiles of the
// same expert and column panel), which then stays in that XCD's L2.
#include "device_common.h"
#include "launchers.h"

namespace moe {
namespace {

constexpr int BM = 128;
constexpr int BP = 256;
constexpr int BK = 64;
constexpr int NT = 256;
constexpr int A_CH = BM * BK / 8 / NT;  // 16-byte chunks of A per thread per stage
constexpr int B_CH = BP * BK / 8 / NT;
constexpr int kMaxE = 256;

__device__ __forceinline__ int swz(int row, int c) { return row * BK + ((c ^ (row & 7)) << 3); }

template <bool GATE_UP>
__global__ __launch_bounds__(NT, 1) void gemm_bf16_kernel(const uint16_t* __restrict__ A,
                                                          const uint16_t* __restrict__ W0,
                                                          const uint16_t* __restrict__ W1,
                                                          uint16_t* __restrict__ C,
                                                          const int32_t* __restrict__ sorted_ids,
                                                          const int32_t* __restrict__ offsets, int P, int top_k,
                                                          int E, int N, int K, int max_pad, int m_tiles,
                                                          int n_tiles) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][(BM + BP) * BK];
    __shared__ int s_scan[4];
    __shared__ int s_row[BM];
    __shared__ int s_info[3];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nwg = gridDim.x;
    const int bid = blockIdx.x;
    const int L = (bid & 7) * (nwg >> 3) + (bid >> 3);
    const int n_t = L / m_tiles, m_t = L % m_tiles;
    if (n_t >= n_tiles) return;

    // ---- which expert and rows this tile covers
    int lo = 0, hi = 0;
    if (tid < E) {
        lo = min(max(offsets[tid], 0), max_pad);
        hi = min(max(offsets[tid + 1], lo), max_pad);
    }
    const int nt_e = (hi - lo + BM - 1) / BM;
    const int incl = block_inclusive_scan_256(nt_e, s_scan);
    if (tid == 0) s_info[0] = -1;
    __syncthreads();
    if (tid < E && m_t >= incl - nt_e && m_t < incl) {
        s_info[0] = tid;
        s_info[1] = lo + (m_t - (incl - nt_e)) * BM;
        s_info[2] = hi;
    }
    __syncthreads();
    const int e = s_info[0];
    if (e < 0) return;
    const int r0 = s_info[1];
    const int r_end = min(r0 + BM, s_info[2]);
    for (int i = tid; i < BM; i += NT) {
        const int r = r0 + i;
        int src = -1;
        if (r < r_end) {
            const int p = sorted_ids[r];
            if (p >= 0 && p < P) src = GATE_UP ? p / top_k : r;
        }
        s_row[i] = src;
    }
    __syncthreads();

    const int n0 = n_t * (GATE_UP ? BP / 2 : BP);

    // ---- per-thread global source rows (fixed over K)
    const uint16_t* a_src[A_CH];
    const uint16_t* b_src[B_CH];
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
        const int c = tid + NT * i, row = c >> 3, kc = c & 7;
        const int src = s_row[row];
        a_src[i] = src >= 0 ? A + static_cast<size_t>(src) * K + kc * 8 : nullptr;
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
        const int c = tid + NT * i, row = c >> 3, kc = c & 7;
        int n;
        const uint16_t* W;
        if (GATE_UP) { n = n0 + (row & (BP / 2 - 1)); W = row < BP / 2 ? W0 : W1; }
        else { n = n0 + row; W = W0; }
        b_src[i] = n < N ? W + (static_cast<size_t>(e) * N + n) * K + kc * 8 : nullptr;
    }

    u32x4 ra[A_CH], rb[B_CH];
    auto load_stage = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int kc = (tid + NT * i) & 7;
            ra[i] = (a_src[i] && k0 + kc * 8 < K) ? *reinterpret_cast<const u32x4*>(a_src[i] + k0)
                                                  : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            const int kc = (tid + NT * i) & 7;
            rb[i] = (b_src[i] && k0 + kc * 8 < K) ? *reinterpret_cast<const u32x4*>(b_src[i] + k0)
                                                  : u32x4{0, 0, 0, 0};
        }
    };
    auto store_stage = [&](int buf) {
        uint16_t* la = lds[buf];
        uint16_t* lb = lds[buf] + BM * BK;
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int c = tid + NT * i, row = c >> 3, kc = c & 7;
            *reinterpret_cast<u32x4*>(la + swz(row, kc)) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            const int c = tid + NT * i, row = c >> 3, kc = c & 7;
            *reinterpret_cast<u32x4*>(lb + swz(row, kc)) = rb[i];
        }
    };

    const int wm = wave >> 1, wn = wave & 1;
    f32x4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (K + BK - 1) / BK;
    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_stage((kt + 1) * BK);
        const uint16_t* la = lds[buf];
        const uint16_t* lb = lds[buf] + BM * BK;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int c = kk * 4 + (lane >> 4);
            bf16x8 a[4], b[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wm * 64 + i * 16 + (lane & 15);
                a[i] = *reinterpret_cast<const bf16x8*>(la + swz(row, c));
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                int prow;
                if (GATE_UP) prow = (j < 4 ? wn * 64 + j * 16 : BP / 2 + wn * 64 + (j - 4) * 16);
                else prow = wn * 128 + j * 16;
                prow += lane & 15;
                b[j] = *reinterpret_cast<const bf16x8*>(lb + swz(prow, c));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) store_stage(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: C fragment lane holds rows 4*(lane/16)+v, column lane%16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int rl = wm * 64 + i * 16 + (lane >> 4) * 4 + v;
            if (s_row[rl] < 0) continue;
            uint16_t* crow = C + static_cast<size_t>(r0 + rl) * N;
            if (GATE_UP) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int col = n0 + wn * 64 + j * 16 + (lane & 15);
                    if (col < N) {
                        const float g = acc[i][j][v], u = acc[i][j + 4][v];
                        crow[col] = f32_to_bf16(g / (1.0f + __expf(-g)) * u);
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int col = n0 + wn * 128 + j * 16 + (lane & 15);
                    if (col < N) crow[col] = f32_to_bf16(acc[i][j][v]);
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_bf16(bool gate_up, const uint16_t* a, const uint16_t* w0, const uint16_t* w1, uint16_t* c,
                            const int32_t* sorted_ids, const int32_t* offsets, int P, int top_k, int E, int N,
                            int K, int max_pad, hipStream_t s) {
    const int m_tiles = (max_pad + BM - 1) / BM + E;
    const int ncols = gate_up ? BP / 2 : BP;
    const int n_tiles = (N + ncols - 1) / ncols;
    const long long tiles = static_cast<long long>(m_tiles) * n_tiles;
    const int grid = static_cast<int>((tiles + 7) / 8 * 8);
    if (gate_up)
        gemm_bf16_kernel<true><<<grid, NT, 0, s>>>(a, w0, w1, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad,
                                                   m_tiles, n_tiles);
    else
        gemm_bf16_kernel<false><<<grid, NT, 0, s>>>(a, w0, nullptr, c, sorted_ids, offsets, P, top_k, E, N, K,
                                                    max_pad, m_tiles, n_tiles);
    return hipGetLastError();
}

}  // namespace moe
