// FP8 prefill variant of the grouped expert GEMMs (atlas moe_lora_grouped.rs module doc: fp8,
// like bf16, is a grouped prefill path that writes the same sorted BF16 expert_down_out).  The
// page fixes no format, so the reading is: OCP FP8 E4M3 weights [E, N, K] with one fp32 scale
// per output channel [E, N], and activations quantised per row at run time:
//   quantize_fp8_kernel   amax of a bf16 row; s = amax / 448 (dequantisation scale) and
//                         f = 448 / amax in fp32; codes = e4m3(x * f), round to nearest even
//   gemm_fp8_kernel       acc = sum_k a(r, k) w(n, k) over the e4m3 values (products exact, fp32
//                         sums) on the CDNA4 32x32x64 fp8 MFMA; out = acc * s_a[row] * s_w[n],
//                         then SiLU(gate) * up (gate/up) or the plain value (down), to bf16
//
// GEMM tiling.  A tile is up to BM (256, or 128 when experts average fewer than 128 rows)
// consecutive sorted rows of one expert (an expert's padded span is cut into ceil(span / BM)
// tiles; the list is rebuilt from expert_offsets by each workgroup with an LDS scan) x a BM-row
// weight panel (gate/up: BM/2 gate and BM/2 up rows of the same output columns, so SiLU * up is
// formed in the epilogue).  One workgroup per tile, BM/32 waves in a (BM/64) x 2 grid, each
// owning 64 rows x BM/2 panel rows as 32 x 32 blocks of fp32 accumulators.  K advances 128 bytes at a time through a 2-stage LDS ring filled by direct
// global->LDS loads (16 bytes per lane, no VGPR staging); chunks past K load zeros.  LDS rows are
// 128 bytes with the 16-byte chunk c of row r stored at c ^ ((r / 2) % 8), so the 32-row x
// 16-byte fragment reads are free of bank conflicts.  An MFMA's operand is 32 bytes per lane
// (two chunks); A and B fragments use the same lane -> k mapping, so every product pairs the
// same k.
#include "device_common.h"
#include "launchers.h"

namespace moe {
namespace {

constexpr int F8_BK = 128;                          // k (bytes = elements) per stage
constexpr int F8_STAGES = 2;
constexpr int F8_CPR = F8_BK / 16;                  // 16-byte chunks per LDS row
constexpr int F8_RPI = 1024 / F8_BK;                // rows one wave-wide 1 KB load fills
constexpr int kMaxE8 = 256;
#ifndef MOE_FP8_SPLIT_MIN_STAGES
#define MOE_FP8_SPLIT_MIN_STAGES 8  // K stages of 128 per piece of a split tail tile, at least
#endif
#ifndef MOE_FP8_SPLIT_MAX_ROUNDS
#define MOE_FP8_SPLIT_MAX_ROUNDS 4  // split the tail only of launches with fewer rounds of tiles
#endif
#ifndef MOE_FP8_ASYM
#define MOE_FP8_ASYM 1  // 8 waves: waves 0-3 issue all of a stage's loads
#endif

// A tile of BM sorted rows x a BM-row weight panel, NW waves in a (NW/2) x 2 grid; each wave
// owns 64 rows (two 32-row blocks) x BM/2 panel rows (NJ 32-wide blocks).
template <int BM, int NW>
struct F8Cfg {
    static constexpr int NT = 64 * NW;
    static constexpr int BP = BM;
    static constexpr int WAVES_M = NW / 2;
    static constexpr int WM = BM / WAVES_M;
    static constexpr int NJ = BP / 2 / 32;
    static constexpr int A_INST = BM / F8_RPI / NW;  // load instructions per wave per stage
    static constexpr int B_INST = BP / F8_RPI / NW;
    static constexpr int STAGE_BYTES = (BM + BP) * F8_BK;
    static_assert(WM == 64, "two 32-row A blocks per wave");
    static_assert(A_INST * NW * F8_RPI == BM && B_INST * NW * F8_RPI == BP, "load cover");
};

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int swz8(int row, int c) { return c ^ ((row >> 1) & 7); }

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

// ------------------------------------------------------------------ grouped GEMM
template <bool GATE_UP, int BM, int NW, bool SPLIT>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void gemm_fp8_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ a_scale, const uint8_t* __restrict__ W0,
    const float* __restrict__ ws0, const uint8_t* __restrict__ W1, const float* __restrict__ ws1,
    uint16_t* __restrict__ C, const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ offsets, int P,
    int top_k, int E, int N, int K, int max_pad, int n_tiles, float* __restrict__ sk_part,
    int32_t* __restrict__ sk_cnt, int sk_slots) {
    using F = F8Cfg<BM, NW>;
    constexpr int BP = F::BP, NJ = F::NJ;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[F8_STAGES * F::STAGE_BYTES];
    __shared__ int s_scan[NW];
    __shared__ int s_lo[kMaxE8], s_hi[kMaxE8], s_tb[kMaxE8 + 1];
    __shared__ int s_row[BM];
    __shared__ float s_as[BM];
    __shared__ int s_arrived;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS destinations are scalar

    // ---- expert spans and their row tiles
    {
        int lo = 0, hi = 0;
        if (tid < E) {
            lo = min(max(offsets[tid], 0), max_pad);
            hi = min(max(offsets[tid + 1], lo), max_pad);
        }
        const int nt_e = (hi - lo + BM - 1) / BM;
        const int incl = block_inclusive_scan<NW>(nt_e, s_scan, (E + 63) / 64);
        if (tid < E) { s_lo[tid] = lo; s_hi[tid] = hi; s_tb[tid + 1] = incl; }
        if (tid == 0) s_tb[0] = 0;
        __syncthreads();
    }
    const int m_real = __builtin_amdgcn_readfirstlane(s_tb[E]);
    const int nk = (K + F8_BK - 1) / F8_BK;
    // Workgroup ids go round-robin over the 8 XCDs: XCD x takes the contiguous range
    // [x*Tw/8, (x+1)*Tw/8) of the first Tw tiles (row tiles fastest), so the workgroups an XCD
    // runs together share weight panels in its L2.
    // Split tail (with a workspace, sk_slots > 0 = workgroups resident at once, and fewer than
    // MOE_FP8_SPLIT_MAX_ROUNDS rounds of tiles: over more rounds, the last partial one costs less
    // than the pieces' partials): the rest = T mod
    // sk_slots tiles of the last partial round are cut along K into s pieces of at least
    // MOE_FP8_SPLIT_MIN_STAGES stages (rest * s <= sk_slots), which run after the whole tiles on
    // the workgroups past each XCD's range.  Each piece writes its fp32 partial accumulators to
    // the workspace slot of its number and counts itself on the tile's counter; the last to
    // arrive adds the s partials in piece order (so results do not depend on arrival order),
    // stores the tile and resets the counter.
    const int T = m_real * n_tiles;
    int Tw = T, split = 1;
    if (SPLIT && sk_slots > 0 && T < MOE_FP8_SPLIT_MAX_ROUNDS * sk_slots) {
        const int rest = T % sk_slots;
        const int s_max = rest > 0 ? min(sk_slots / rest, nk / MOE_FP8_SPLIT_MIN_STAGES) : 1;
        if (s_max >= 2) { Tw = T - rest; split = s_max; }
    }
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int lo_x = static_cast<int>(static_cast<long long>(Tw) * xcd / 8);
    const int share = static_cast<int>(static_cast<long long>(Tw) * (xcd + 1) / 8) - lo_x;
    int L, kb = 0, ke = nk, piece = -1, tail_u = 0;
    if (slot < share) {
        L = lo_x + slot;
    } else {
        piece = (slot - share) * 8 + xcd;  // distinct over XCDs (piece mod 8 == xcd)
        if (piece >= (T - Tw) * split) return;  // uniform over the workgroup
        tail_u = piece / split;
        const int j = piece - tail_u * split;
        L = Tw + tail_u;
        kb = j * nk / split;
        ke = (j + 1) * nk / split;
    }
    const int n_t = L / m_real;
    const int m_t = L - n_t * m_real;
    int lo_e = 0, hi_e = E - 1;                   // largest expert whose first row tile is <= m_t
    while (lo_e < hi_e) {
        const int mid = (lo_e + hi_e + 1) >> 1;
        if (s_tb[mid] <= m_t) lo_e = mid; else hi_e = mid - 1;
    }
    const int e = __builtin_amdgcn_readfirstlane(lo_e);
    const int r0 = __builtin_amdgcn_readfirstlane(s_lo[e] + (m_t - s_tb[e]) * BM);
    const int r_end = __builtin_amdgcn_readfirstlane(min(r0 + BM, s_hi[e]));
    constexpr int NCOL = GATE_UP ? BP / 2 : BP;  // output columns per tile
    const int n0 = n_t * NCOL;

    // ---- the tile's A rows (token rows for gate/up, sorted rows for down) and their scales
    if (tid < BM) {
        const int r = r0 + tid;
        int src = -1;
        float sc = 0.f;
        if (r < r_end) {
            const int p = sorted_ids[r];
            if (p >= 0 && p < P) {
                src = GATE_UP ? p / top_k : r;
                sc = a_scale[src];
            }
        }
        s_row[tid] = src;
        s_as[tid] = sc;
    }
    __syncthreads();

    // ---- per-lane load sources: instruction q of this wave fills LDS rows
    // (wave * INST + q) * F8_RPI .. + F8_RPI - 1; this lane's 16 bytes are physical chunk pc of
    // row lrow, which holds logical chunk swz8(row, pc).  A row without a token reads a row that
    // is always in bounds (token 0, or the tile's first sorted row); its results are never stored.
    const int lrow = lane / F8_CPR, pc = lane % F8_CPR;
    // With 8 waves (two per SIMD), waves 0-3 issue the loads of their own row blocks and of
    // waves 4-7's, which issue none: while an issuing wave stalls on the address unit, the other
    // wave of its SIMD issues MFMAs.  Block j of an issuing wave is that of wave + j * NW/2.
    constexpr bool ASYM = MOE_FP8_ASYM != 0 && NW == 8;
    constexpr int NBLK = ASYM ? 2 : 1;
    const bool issuer = !ASYM || wave < NW / 2;
    const uint8_t* a_src[NBLK][F::A_INST];
    const uint8_t* b_src[NBLK][F::B_INST];
    int a_kc[NBLK][F::A_INST], b_kc[NBLK][F::B_INST];
    const uint8_t* wb0 = W0 + static_cast<size_t>(e) * N * K;
    const uint8_t* wb1 = GATE_UP ? W1 + static_cast<size_t>(e) * N * K : wb0;
#pragma unroll
    for (int j = 0; j < NBLK; ++j) {
        const int bw = wave + j * (NW / 2);
#pragma unroll
        for (int q = 0; q < F::A_INST; ++q) {
            const int row = (bw * F::A_INST + q) * F8_RPI + lrow;
            const int kc = swz8(row, pc);
            const int src = s_row[row];
            const int srow = src >= 0 ? src : (GATE_UP ? 0 : r0);
            a_src[j][q] = A + static_cast<size_t>(srow) * K + kc * 16;
            a_kc[j][q] = kc;
        }
#pragma unroll
        for (int q = 0; q < F::B_INST; ++q) {
            const int row = (bw * F::B_INST + q) * F8_RPI + lrow;
            const int kc = swz8(row, pc);
            int n = GATE_UP ? n0 + (row & (BP / 2 - 1)) : n0 + row;
            n = min(n, N - 1);  // columns past N are computed from a valid row and never stored
            const uint8_t* base = (GATE_UP && row >= BP / 2) ? wb1 : wb0;
            b_src[j][q] = base + static_cast<size_t>(n) * K + kc * 16;
            b_kc[j][q] = kc;
        }
    }
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void*)smem)));
    auto issue = [&](int t) __attribute__((always_inline)) {
        if (!issuer) return;
        const int k0 = t * F8_BK;
        const uint32_t sb = lds0 + static_cast<uint32_t>(t % F8_STAGES) * F::STAGE_BYTES;
        const bool full = k0 + F8_BK <= K;
#pragma unroll
        for (int j = 0; j < NBLK; ++j) {
            const int bw = wave + j * (NW / 2);
#pragma unroll
            for (int q = 0; q < F::B_INST; ++q) {
                const void* g = b_src[j][q] + k0;
                if (!full && k0 + b_kc[j][q] * 16 >= K) g = kZero16;
                dma16(g, sb + BM * F8_BK + (bw * F::B_INST + q) * 1024);
            }
#pragma unroll
            for (int q = 0; q < F::A_INST; ++q) {
                const void* g = a_src[j][q] + k0;
                if (!full && k0 + a_kc[j][q] * 16 >= K) g = kZero16;
                dma16(g, sb + (bw * F::A_INST + q) * 1024);
            }
        }
    };

    // ---- main loop
    const int wm = wave >> 1, wn = wave & 1;
    const int fr = lane & 31, fh = lane >> 5;  // fragment row / column, 32-byte k half
    int a_row[2], b_row[NJ];
#pragma unroll
    for (int i = 0; i < 2; ++i) a_row[i] = wm * 64 + i * 32 + fr;
    // panel rows of this wave's column blocks: down, BP/2 consecutive rows; gate/up, BP/4 gate rows
    // (blocks 0 .. NJ/2-1) and the up rows of the same columns (blocks NJ/2 ..)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
        b_row[j] = BM + (GATE_UP ? (j < NJ / 2 ? wn * (BP / 4) + j * 32 : BP / 2 + wn * (BP / 4) + (j - NJ / 2) * 32)
                                 : wn * (BP / 2) + j * 32) + fr;
    f32x16 acc[2][NJ];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    auto frag = [&](const uint8_t* st, int row, int c0) __attribute__((always_inline)) {
        const uint8_t* rp = st + row * F8_BK;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(rp + swz8(row, c0) * 16);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(rp + swz8(row, c0 + 1) * 16);
        return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    issue(kb);
    for (int s = kb; s < ke; ++s) {
        // this thread's loads of stage s have landed and every wave is past stage s - 1, whose
        // buffer is refilled with stage s + 1
        __builtin_amdgcn_s_waitcnt(0x0070 | (15 << 8));  // vmcnt(0)
        __builtin_amdgcn_s_waitcnt(0xc07f);              // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        if (s + 1 < ke) issue(s + 1);
        const uint8_t* st = smem + (s % F8_STAGES) * F::STAGE_BYTES;
#pragma unroll
        for (int ks = 0; ks < F8_BK / 64; ++ks) {
            const int c0 = ks * 4 + fh * 2;
            i32x8 fa[2], fb[NJ];
#pragma unroll
            for (int i = 0; i < 2; ++i) fa[i] = frag(st, a_row[i], c0);
#pragma unroll
            for (int j = 0; j < NJ; ++j) fb[j] = frag(st, b_row[j], c0);
            // format 0 (E4M3) for both operands; block scales 127 (2^0): plain fp8 products
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0, 0, 0,
                                                                               127, 0, 127);
        }
    }

    // ---- a piece of a split tail tile: partials through the workspace, with device-coherent
    // (sc1) buffer accesses (see gemm_bf16.hip: no fence writes back or invalidates the L2)
    if (SPLIT && piece >= 0) {
        constexpr int PART = 64 * NW * 2 * NJ * 16;  // floats per partial
        constexpr int kSc1 = 16;
        const __amdgpu_buffer_rsrc_t part =
            __builtin_amdgcn_make_buffer_rsrc(sk_part, 0, sk_slots * PART * 4, 0x00020000);
        uint32_t o = (static_cast<uint32_t>(piece) * PART + tid * 4) * 4;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 v{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                    __builtin_amdgcn_raw_buffer_store_b128(v, part, o, 0, kSc1);
                    o += 64 * NW * 16;
                }
        __builtin_amdgcn_s_waitcnt(0x0070 | (15 << 8));  // vmcnt(0): the partial is visible before it is counted
        __syncthreads();
        if (tid == 0)
            s_arrived = __hip_atomic_fetch_add(&sk_cnt[tail_u], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (s_arrived != split - 1) return;  // uniform: another piece stores the tile
        uint32_t base = (static_cast<uint32_t>(tail_u * split) * PART + tid * 4) * 4;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    f32x4 t{0.f, 0.f, 0.f, 0.f};
                    for (int jp = 0; jp < split; ++jp)
                        t += __builtin_amdgcn_raw_buffer_load_b128(part, base + jp * PART * 4, 0, kSc1);
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[i][j][4 * q + v] = t[v];
                    base += 64 * NW * 16;
                }
        if (tid == 0) __hip_atomic_store(&sk_cnt[tail_u], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- epilogue: scales, SiLU * up for gate/up; neighbour lanes (columns c, c+1) swap one
    // value so that each lane stores two adjacent bf16 columns of one row as 4 bytes
    const bool odd = (lane & 1) != 0;
    constexpr int NO = GATE_UP ? NJ / 2 : NJ;  // output column blocks of this wave
    float wsc[NO], wsu[NO];
    int colj[NO];
#pragma unroll
    for (int j = 0; j < NO; ++j) {
        colj[j] = n0 + (GATE_UP ? wn * (BP / 4) : wn * (BP / 2)) + j * 32 + fr;  // this lane's column
        const int cc = min(colj[j], N - 1);
        wsc[j] = ws0[static_cast<size_t>(e) * N + cc];
        wsu[j] = GATE_UP ? ws1[static_cast<size_t>(e) * N + cc] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
            const int rl = wm * 64 + i * 32 + (v >> 2) * 8 + fh * 4 + (v & 3);  // row of value v
            const float sa0 = s_as[rl], sa1 = s_as[rl + 1];
            const int row_l = rl + (odd ? 1 : 0);
            const bool ok = s_row[row_l] >= 0;
            uint16_t* crow = C + static_cast<size_t>(r0 + row_l) * N;
#pragma unroll
            for (int j = 0; j < NO; ++j) {
                float h0, h1;  // values v (row rl) and v+1 (row rl+1) of this lane's column
                if (GATE_UP) {
                    h0 = silu_mul(acc[i][j][v] * sa0 * wsc[j], acc[i][j + NO][v] * sa0 * wsu[j]);
                    h1 = silu_mul(acc[i][j][v + 1] * sa1 * wsc[j], acc[i][j + NO][v + 1] * sa1 * wsu[j]);
                } else {
                    h0 = acc[i][j][v] * sa0 * wsc[j];
                    h1 = acc[i][j][v + 1] * sa1 * wsc[j];
                }
                const float send = odd ? h0 : h1;
                const float got = __int_as_float(__builtin_amdgcn_update_dpp(
                    0, __float_as_int(send), 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
                const uint32_t pr = odd ? pack_bf16x2(got, h1) : pack_bf16x2(h0, got);
                const int col = colj[j] & ~1;
                if (ok && col < N) *reinterpret_cast<uint32_t*>(crow + col) = pr;
            }
        }
}

int device_cus8(hipError_t& err) {
    static int cus[64] = {0};
    int dev = 0;
    err = hipGetDevice(&dev);
    if (err != hipSuccess) return 0;
    if (dev < 0 || dev >= 64) { err = hipErrorInvalidDevice; return 0; }
    if (cus[dev] == 0) {
        int n = 0;
        err = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (err != hipSuccess) return 0;
        cus[dev] = n;
    }
    return cus[dev];
}

// workspace layout shared with the bf16 GEMM: 4 KB of int32 counters, then partial slots
constexpr int64_t kF8CounterBytes = 4096;
constexpr int64_t kF8PartBytes = 512LL * 2 * 64 * 4;   // largest partial: 512 threads x 128 fp32
constexpr int kF8MaxSlots = 256;

template <bool GATE_UP, int BM, int NW>
hipError_t launch_fp8_cfg(const uint8_t* a, const float* a_scale, const uint8_t* w0, const float* ws0,
                          const uint8_t* w1, const float* ws1, uint16_t* c, const int32_t* sorted_ids,
                          const int32_t* offsets, int P, int top_k, int E, int N, int K, int max_pad, void* ws,
                          int64_t ws_bytes, hipStream_t s) {
    static_assert(64 * NW * 2 * F8Cfg<BM, NW>::NJ * 16 * 4 <= kF8PartBytes, "partial larger than its slot");
    const int ncol = GATE_UP ? BM / 2 : BM;
    const int n_tiles = (N + ncol - 1) / ncol;
    const int m_bound = (max_pad + BM - 1) / BM + E;  // row tiles of any routing, at most
    // workgroups resident at once: one per compute unit (256-row tiles), two (128-row tiles)
    int slots = 0;
    if (ws != nullptr && ws_bytes >= kF8CounterBytes + kF8MaxSlots * kF8PartBytes) {
        hipError_t err = hipSuccess;
        slots = device_cus8(err) * (NW == 4 ? 2 : 1);
        if (err != hipSuccess) return err;
        slots = min(slots, kF8MaxSlots);
    }
    // each XCD's share of the whole tiles (rounded up) plus its pieces of a split tail, times 8
    const long long grid = ((static_cast<long long>(m_bound) * n_tiles + 7) / 8 + 1 + (slots + 7) / 8) * 8;
    int32_t* cnt = slots > 0 ? static_cast<int32_t*>(ws) : nullptr;
    float* part = slots > 0 ? reinterpret_cast<float*>(static_cast<char*>(ws) + kF8CounterBytes) : nullptr;
    // the split-tail code is compiled only into the kernel of launches that can have few rounds of
    // tiles (it costs the others about 1% through their register allocation)
    if (slots > 0 && static_cast<long long>(m_bound) * n_tiles < static_cast<long long>(MOE_FP8_SPLIT_MAX_ROUNDS) * slots)
        gemm_fp8_kernel<GATE_UP, BM, NW, true><<<static_cast<unsigned>(grid), 64 * NW, 0, s>>>(
            a, a_scale, w0, ws0, w1, ws1, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, n_tiles, part, cnt,
            slots);
    else
        gemm_fp8_kernel<GATE_UP, BM, NW, false><<<static_cast<unsigned>(grid), 64 * NW, 0, s>>>(
            a, a_scale, w0, ws0, w1, ws1, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, n_tiles, nullptr,
            nullptr, 0);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_fp8(const uint16_t* x, int64_t rows, int K, const int32_t* sorted_ids, int P,
                               uint8_t* q, float* scale, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    quantize_fp8_kernel<<<static_cast<unsigned>(rows), kQThreads, 0, s>>>(x, q, scale, sorted_ids, P, K);
    return hipGetLastError();
}

hipError_t launch_gemm_fp8(bool gate_up, const uint8_t* a, const float* a_scale, const uint8_t* w0,
                           const float* ws0, const uint8_t* w1, const float* ws1, uint16_t* c,
                           const int32_t* sorted_ids, const int32_t* offsets, int P, int top_k, int E, int N,
                           int K, int max_pad, void* ws, int64_t ws_bytes, hipStream_t s) {
    // 256-row tiles (8 waves, two per SIMD) when experts average at least 128 rows; 128-row
    // tiles (4 waves) for fewer
    const bool big = static_cast<long long>(P) >= 128LL * E;
    if (gate_up) {
        if (big) return launch_fp8_cfg<true, 256, 8>(a, a_scale, w0, ws0, w1, ws1, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, ws, ws_bytes, s);
        return launch_fp8_cfg<true, 128, 4>(a, a_scale, w0, ws0, w1, ws1, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, ws, ws_bytes, s);
    }
    if (big) return launch_fp8_cfg<false, 256, 8>(a, a_scale, w0, ws0, nullptr, nullptr, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, ws, ws_bytes, s);
    return launch_fp8_cfg<false, 128, 4>(a, a_scale, w0, ws0, nullptr, nullptr, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, ws, ws_bytes, s);
}

}  // namespace moe
