// Grouped expert GEMM with GPTQ int4 weights (stacked raw GPTQ layout of ferrum-kernels
// triton_fused_moe.rs: qweight [E,K/8,N] i32, scales [E,K/G,N] fp16, qzeros [E,K/G,N/8]),
// one launch for all experts.  Built for weight streaming (decode: a block holds a few
// real rows, so every weight byte is used by at most a handful of rows).
//
// Work unit: one workgroup = one 16-row tile of sorted rows (one expert, from expert_ids)
// x 64 output columns.  For gate/up, waves 0-1 compute the gate projection and waves 2-3 the up
// projection, each pair splitting the K groups in two; for down, the 4 waves split the K groups
// in four.  Partial sums meet in LDS.  One projection per wave keeps a wave's registers small
// enough for 4 waves per SIMD, so more weight loads are in flight per CU.
//
// Dequantisation without per-weight float work.  A qweight word holds 8 consecutive k of
// one column; OR-ing nibble pairs into bf16 0x4300 (= 128.0) gives the exact bf16 values
// 128+q in two ALU ops per pair, so the MFMA (16x16x32 bf16, fp32 accumulate) computes
// acc = sum_k x[k]*(128+q[k]) over one quantisation group.  With the group's scale s
// and zero z fixed per column, the group contributes
//     s * sum_k x[k]*(q[k]-z) = s * (acc - (128+z) * sum_k x[k]),
// and sum_k x[k] comes from one more MFMA against a ones matrix.  The pair trick takes
// nibbles (0,4),(1,5),(2,6),(3,7) of a word, so the x fragment is permuted to the same
// k order; a sum over k does not depend on the order.
// Loads: each lane reads 16 B of qweight = the same k-octet of 4 consecutive columns, one
// column per MFMA, so a wave reads 256 contiguous bytes per k-octet row; the next
// group's loads are issued before the current group's MFMAs.
#include "device_common.h"
#include "launchers.h"

namespace moe {
namespace {

constexpr int NW = 4;  // waves per workgroup (8, with half as many K groups each, measured slower)
constexpr int NT = NW * 64;
constexpr int NCOL = 64;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// x fragment k order (k0..k7) -> (k0,k4,k1,k5,k2,k6,k3,k7), matching the nibble pairs: one
// v_perm_b32 per output word (byte selectors 0-3 pick from the second operand, 4-7 the first).
__device__ __forceinline__ u32x4 permute_k(u32x4 a) {
    u32x4 r;
    r[0] = __builtin_amdgcn_perm(a[2], a[0], 0x05040100u);
    r[1] = __builtin_amdgcn_perm(a[2], a[0], 0x07060302u);
    r[2] = __builtin_amdgcn_perm(a[3], a[1], 0x05040100u);
    r[3] = __builtin_amdgcn_perm(a[3], a[1], 0x07060302u);
    return r;
}

// One qweight word (8 nibbles of consecutive k) -> bf16 (128+q) in the permuted k order.  The
// mask and the bf16 exponent pattern come in registers (opaque to the compiler) so that each
// pair is one v_and_or_b32: a VOP3 instruction cannot take them as literals.
__device__ __forceinline__ u32x4 dequant_word(uint32_t w, uint32_t mask, uint32_t magic) {
    u32x4 r;
    r[0] = (w & mask) | magic;
    r[1] = ((w >> 4) & mask) | magic;
    r[2] = ((w >> 8) & mask) | magic;
    r[3] = ((w >> 12) & mask) | magic;
    return r;
}

// Registers of one quantisation group for one lane (STEPS = G/32 MFMA k-steps).
template <int STEPS>
struct GroupRegs {
    u32x4 q[STEPS];  // qweight: 16 B = 4 columns x one k-octet, per step
    u32x4 a[STEPS];  // x fragment (8 bf16) per step
    uint2 s;         // 4 fp16 scales
    uint32_t z;      // qzeros word holding the 4 zero points
};

template <bool GATE_UP, int STEPS>
__global__ __launch_bounds__(NT, (STEPS <= 4 ? 16 : 8) / NW) void gemm_int4_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ qw0, const uint16_t* __restrict__ sc0,
    const int32_t* __restrict__ qz0, const int32_t* __restrict__ qw1, const uint16_t* __restrict__ sc1,
    const int32_t* __restrict__ qz1, uint16_t* __restrict__ C, const int32_t* __restrict__ sorted_ids,
    const int32_t* __restrict__ expert_ids, int P, int top_k, int E, int N, int K, int bs, int max_pad,
    int a_tok, int col_fast) {
    constexpr int NSPLIT = GATE_UP ? NW / 2 : NW;  // waves sharing one projection's K groups
    constexpr int G = STEPS * 32;
    __shared__ int s_row[16];
    __shared__ float red[NW][4][64][4];  // [wave][v][lane][j]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // with col_fast the column blocks are the grid's fast index: the workgroups of one tile,
    // dispatched together, read the whole rows of its expert's qweight (N * 4 bytes per k-octet)
    // at about the same time (grids too tall for the y dimension keep the tiles fast)
    const int r0 = (col_fast ? blockIdx.y : blockIdx.x) * 16;
    const int n0 = (col_fast ? blockIdx.x : blockIdx.y) * NCOL;
    const int m = lane & 15, kq = lane >> 4;  // A fragment row; k-octet within a k32 step

    // The tile's rows: every wave reads the 16 sorted ids itself (no barrier before the first
    // loads).  The id load is issued before the weight loads, so waiting for it does not wait for
    // them: vector loads complete in issue order.
    // (loads without branches around them, so the wait for the id can count the later loads)
    int p = sorted_ids[min(r0 + m, max_pad - 1)];
    if (r0 + m >= max_pad) p = -1;
    const int e = expert_ids[r0 / bs];
    if (e < 0 || e >= E) return;

    // this wave's projection and quantisation groups
    const int proj = GATE_UP ? wave / NSPLIT : 0;
    const int part = GATE_UP ? wave % NSPLIT : wave;
    const int ngroups = K / G;
    const int per = (ngroups + NSPLIT - 1) / NSPLIT;
    const int g_begin = part * per;
    const int g_end = min(ngroups, g_begin + per);
    const int ncol = n0 + 4 * m;              // first of this lane's 4 columns
    const int zshift = 16 * (m & 1);          // nibble of column ncol inside its qzeros word

    // per-lane weight and x sources of group g (g in [g0, g_last]: a wave without groups, or the
    // prefetch past its last group, reads its last group again, in bounds and unused)
    const int g0 = __builtin_amdgcn_readfirstlane(min(g_begin, ngroups - 1));  // wave-uniform
    const int g_last = __builtin_amdgcn_readfirstlane(max(g_end - 1, g0));
    const int32_t* q_base = (proj ? qw1 : qw0) + static_cast<size_t>(e) * (K / 8) * N + static_cast<size_t>(kq) * N + ncol;
    const uint16_t* s_base = (proj ? sc1 : sc0) + static_cast<size_t>(e) * (K / G) * N + ncol;
    const int32_t* z_base = (proj ? qz1 : qz0) + static_cast<size_t>(e) * (K / G) * (N / 8) + ncol / 8;
    auto load_w = [&](GroupRegs<STEPS>& R, int g) {
        const int32_t* q = q_base + static_cast<size_t>(g) * (G / 8) * N;
#pragma unroll
        for (int st = 0; st < STEPS; ++st)
            R.q[st] = *reinterpret_cast<const u32x4*>(q + static_cast<size_t>(st) * 4 * N);
        R.s = *reinterpret_cast<const uint2*>(s_base + static_cast<size_t>(g) * N);
        R.z = static_cast<uint32_t>(z_base[static_cast<size_t>(g) * (N / 8)]);
    };
    // the first group's weights depend only on the expert: they stream while the rows resolve
    const int ng = __builtin_amdgcn_readfirstlane(max(g_end - g_begin, 0));
    GroupRegs<STEPS> ra, rb;  // two register sets, groups alternating between them
    load_w(ra, g0);

    const int src = (p >= 0 && p < P) ? ((GATE_UP || a_tok) ? p / top_k : r0 + m) : -1;
    if (wave == 0 && lane < 16) s_row[lane] = src;  // read by the epilogue after the reduction barrier
    if (!__any(src >= 0)) return;  // the same 16 rows in every wave: the whole workgroup leaves

    // a row without a token reads a row that is always in bounds (token 0, or the tile's first
    // sorted row); its results are never stored
    const int arow_ok = src >= 0 ? src : ((GATE_UP || a_tok) ? 0 : r0);
    const uint16_t* a_base = A + static_cast<size_t>(arow_ok) * K + kq * 8;
    auto load_a = [&](GroupRegs<STEPS>& R, int g) {
#pragma unroll
        for (int st = 0; st < STEPS; ++st)
            R.a[st] = *reinterpret_cast<const u32x4*>(a_base + static_cast<size_t>(g) * G + st * 32);
    };
    load_a(ra, g0);

    f32x4 out[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    uint32_t nib_mask, bf16_128;
    asm volatile("v_mov_b32 %0, 0x000f000f" : "=v"(nib_mask));
    asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(bf16_128));

    auto compute_group = [&](const GroupRegs<STEPS>& cur) {
        f32x4 acc[4], accx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            const bf16x8 afr = as_bf16x8(permute_k(cur.a[st]));
            accx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, as_bf16x8(ones), accx, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    afr, as_bf16x8(dequant_word(cur.q[st][j], nib_mask, bf16_128)), acc[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t sbits = (j < 2 ? cur.s.x : cur.s.y) >> (16 * (j & 1));
            const float sc = f16_to_f32(static_cast<uint16_t>(sbits & 0xffffu));
            const float zz = 128.0f + static_cast<float>((cur.z >> (zshift + 4 * j)) & 0xfu);
#pragma unroll
            for (int v = 0; v < 4; ++v) out[j][v] = fmaf(sc, fmaf(-zz, accx[v], acc[j][v]), out[j][v]);
        }
    };

    // group g+1 loads while group g is computed, two groups per trip in fixed register sets (no
    // copies of registers with loads in flight); the loads are issued unconditionally (past the
    // wave's last group they re-read it) so that no branch separates a load from its use and the
    // wait before a group's MFMAs covers that group's loads only
    // (scheduling fences keep each group's loads together, ahead of the other group's MFMAs)
    int i = 0;
    for (; i + 1 < ng; i += 2) {
        load_w(rb, g0 + i + 1);
        load_a(rb, g0 + i + 1);
        __builtin_amdgcn_sched_barrier(0);
        compute_group(ra);
        __builtin_amdgcn_sched_barrier(0);
        const int gn = min(g0 + i + 2, g_last);
        load_w(ra, gn);
        load_a(ra, gn);
        __builtin_amdgcn_sched_barrier(0);
        compute_group(rb);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (i < ng) compute_group(ra);  // an odd count: the last group is in ra

    // split-K reduction over the waves, then the epilogue: 256 threads = 16 rows x 16 column quads
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int j = 0; j < 4; ++j) red[wave][v][lane][j] = out[j][v];
    __syncthreads();
    // the partial sums of waves w0 .. w0 + n - 1 (n = 2 or 4), added pairwise in a fixed order
    auto wsum = [&](int w0, int n, int v, int sl, int j) {
        if (n == 2) return red[w0][v][sl][j] + red[w0 + 1][v][sl][j];
        return (red[w0][v][sl][j] + red[w0 + 1][v][sl][j]) + (red[w0 + 2][v][sl][j] + red[w0 + 3][v][sl][j]);
    };
    {
        const int sl = tid & 63, v = tid >> 6;  // source lane and row-in-quad of the C fragment
        const int row = 4 * (sl >> 4) + v;
        if (s_row[row] < 0) return;
        const int col = n0 + 4 * (sl & 15);
        float res[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float res_j;
            if (GATE_UP) res_j = silu_mul(wsum(0, NSPLIT, v, sl, j), wsum(NSPLIT, NSPLIT, v, sl, j));
            else res_j = wsum(0, NSPLIT, v, sl, j);
            res[j] = res_j;
        }
        uint2 o;
        o.x = pack_bf16x2(res[0], res[1]);
        o.y = pack_bf16x2(res[2], res[3]);
        *reinterpret_cast<uint2*>(C + static_cast<size_t>(r0 + row) * N + col) = o;
    }
}

template <int STEPS>
void launch_int4_steps(int op, dim3 grid, int col_fast, hipStream_t s, const uint16_t* a, const int32_t* qw0,
                       const uint16_t* sc0, const int32_t* qz0, const int32_t* qw1, const uint16_t* sc1,
                       const int32_t* qz1, uint16_t* c, const int32_t* sorted_ids, const int32_t* expert_ids, int P,
                       int top_k, int E, int N, int K, int bs, int max_pad) {
    if (op == kOpGateUpSilu)
        gemm_int4_kernel<true, STEPS><<<grid, NT, 0, s>>>(a, qw0, sc0, qz0, qw1, sc1, qz1, c, sorted_ids, expert_ids,
                                                          P, top_k, E, N, K, bs, max_pad, 1, col_fast);
    else  // one projection: rows of a in sorted order (down) or by token (gather)
        gemm_int4_kernel<false, STEPS><<<grid, NT, 0, s>>>(a, qw0, sc0, qz0, nullptr, nullptr, nullptr, c,
                                                           sorted_ids, expert_ids, P, top_k, E, N, K, bs, max_pad,
                                                           op == kOpGather ? 1 : 0, col_fast);
}

}  // namespace

hipError_t launch_gemm_int4(int op, const uint16_t* a, const int32_t* qw0, const uint16_t* sc0,
                            const int32_t* qz0, const int32_t* qw1, const uint16_t* sc1, const int32_t* qz1,
                            int group_size, uint16_t* c, const int32_t* sorted_ids, const int32_t* expert_ids,
                            int P, int top_k, int E, int N, int K, int bs, int max_pad, hipStream_t s) {
    const int col_fast = max_pad / 16 <= 65535;  // column blocks fastest (see the kernel) when y can hold the tiles
    const dim3 grid = col_fast ? dim3(N / NCOL, max_pad / 16) : dim3(max_pad / 16, N / NCOL);
    switch (group_size) {
        case 32: launch_int4_steps<1>(op, grid, col_fast, s, a, qw0, sc0, qz0, qw1, sc1, qz1, c, sorted_ids, expert_ids, P, top_k, E, N, K, bs, max_pad); break;
        case 64: launch_int4_steps<2>(op, grid, col_fast, s, a, qw0, sc0, qz0, qw1, sc1, qz1, c, sorted_ids, expert_ids, P, top_k, E, N, K, bs, max_pad); break;
        case 128: launch_int4_steps<4>(op, grid, col_fast, s, a, qw0, sc0, qz0, qw1, sc1, qz1, c, sorted_ids, expert_ids, P, top_k, E, N, K, bs, max_pad); break;
        case 256: launch_int4_steps<8>(op, grid, col_fast, s, a, qw0, sc0, qz0, qw1, sc1, qz1, c, sorted_ids, expert_ids, P, top_k, E, N, K, bs, max_pad); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace moe
