// LoRA fold on the sorted rows (atlas moe_lora_grouped.rs, moe_lora_grouped_down): for each
// real row r of an adapted expert e in the window,
//   xa    = bf16(x[r] A_e^T)                      (shrink, max_rank outputs; with x_gather, the
//                                                  gate/up form, x is the token-major input and
//                                                  row r reads its token sorted_ids[r] / top_k)
//   delta = bf16(xa B_e^T)                        (expand, n_out outputs)
//   base[r] = bf16(fp32(base[r]) + scale_e * fp32(delta))   (in place)
// Adapters (atlas MoeExpertRoute: adapter identity of a mixed batch comes from the per-row
// moe_row_adapter, not from the tables): the tables hold n_adapters rows of n_tab entries, and a row
// of token t uses row a = row_adapter[t] (0 without a map; < 0 or >= n_adapters folds nothing).  The
// rows of one sub-tile may belong to several adapters: the kernels take the adapters present one at
// a time (a uniform loop, usually one pass) and write only that adapter's rows in each pass.
// Two launches like the page: the shrink writes the bf16 xa scratch at the local row
// r - row_offset, the expand reads it.  The expert of a row is read on the device from
// expert_offsets (the row's span), so the grid is fixed by host scalars: a window is cut
// into 64-row tiles aligned to 16-row boundaries (one 16-row sub-tile per wave; block
// sizes are multiples of 16, so a sub-tile never straddles two experts' spans), and
// sub-tiles of unadapted experts, sentinel rows and rows outside the window do nothing.
// Both stages use 16x16x32 bf16 MFMA with fp32 accumulation.  The shrink gives each 16-row
// sub-tile a workgroup whose 4 waves split k_in.  The expand stages its bf16
// delta tile in LDS and then updates the base rows with 16-byte coalesced accesses.
#include "device_common.h"
#include "launchers.h"

namespace moe {
namespace {

constexpr int NT = 256;
#ifndef MOE_LORA_EXP_COLS
#define MOE_LORA_EXP_COLS 64
#endif
// expand output columns per workgroup (32 to 256; 64 measured best: 4 accumulators per wave keep
// 4 waves per SIMD and the base-row loads in flight)
constexpr int EXP_COLS = MOE_LORA_EXP_COLS;
static_assert(EXP_COLS >= 32 && EXP_COLS <= 256 && (EXP_COLS & (EXP_COLS - 1)) == 0, "expand tile width");
constexpr int FOLD_LPR = EXP_COLS / 8;       // fold: lanes per row (8 columns each)
constexpr int FOLD_RPS = 64 / FOLD_LPR;      // fold: rows per step
constexpr int FOLD_STEPS = 16 / FOLD_RPS;    // fold: steps over a 16-row sub-tile
constexpr int MAX_RANK_BLOCKS = 8;  // max_rank <= 128
#ifndef MOE_LORA_EXP_BLOCKS
#define MOE_LORA_EXP_BLOCKS 4
#endif
constexpr int EXP_BLOCKS = MOE_LORA_EXP_BLOCKS;  // column blocks of EXP_COLS per expand wave

// expert_offsets [E+1] (E <= 256) into LDS, so that each sub-tile's binary search over the
// expert spans costs LDS reads instead of a chain of dependent global loads
__device__ __forceinline__ void stage_offsets(const int32_t* off, int E, int* s_off) {
    for (int i = threadIdx.x; i <= E; i += blockDim.x) s_off[i] = off[i];
    __syncthreads();
}

struct SubTile {
    int e;          // expert of the 16-row sub-tile (-1: nothing to do)
    int span_end;   // end of that expert's padded span
};

__device__ __forceinline__ SubTile sub_tile_expert(int sub0, const int32_t* off, int E, int n_tab) {
    SubTile st{-1, 0};
    // expert spans are read from device memory: clamp the search to what it can address
    int lo = 0, hi = E;
    if (off[0] > sub0 || off[E] <= sub0) return st;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (off[mid] <= sub0) lo = mid; else hi = mid;
    }
    if (lo >= n_tab) return st;  // past every adapter's table: unadapted
    st.e = lo;
    st.span_end = off[lo + 1];
    return st;
}

constexpr int kNoAdapter = 0x7fffffff;  // "no adapter" key: above every real adapter id

// Adapter of sorted row r if it is folded (inside the window and the expert span, real, its token's
// adapter in [0, n_ad) and that adapter adapts expert e), else kNoAdapter.
__device__ __forceinline__ int row_adapter_of(int64_t r, int64_t row_offset, int64_t row_end, int span_end,
                                              const int32_t* sorted_ids, int P, int top_k,
                                              const int32_t* row_adapter, int n_ad, int n_tab, int e,
                                              const uint64_t* a_tab, const uint64_t* b_tab) {
    if (r < row_offset || r >= row_end || r >= span_end) return kNoAdapter;
    const int p = sorted_ids[r];
    if (p < 0 || p >= P) return kNoAdapter;
    const int a = row_adapter ? row_adapter[p / top_k] : 0;
    if (a < 0 || a >= n_ad) return kNoAdapter;
    const int64_t ix = static_cast<int64_t>(a) * n_tab + e;
    if (a_tab[ix] == 0 || b_tab[ix] == 0) return kNoAdapter;
    return a;
}

// Smallest adapter id above `after` held by any lane of the wave (kNoAdapter if none); the result is
// the same in every lane.
__device__ __forceinline__ int wave_next_adapter(int mine, int after) {
    int v = mine > after ? mine : kNoAdapter;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const int w = __shfl_xor(v, o);
        v = w < v ? w : v;
    }
    return v;
}

// Shrink: one workgroup per 16-row sub-tile; its 4 waves take a quarter of k_in each and add
// their partial sums in LDS, so one row's k loop is split over 4 waves.  NB = rank blocks of 16
// (max_rank / 16, up to 8); KU k-steps per round: every load of a round is issued before its
// MFMAs, so a wave waits for one memory round trip per KU steps.
template <int NB>
__global__ __launch_bounds__(NT) void lora_shrink_kernel(const uint16_t* __restrict__ x, const uint64_t* a_tab,
                                                         const uint64_t* b_tab, int n_tab, int n_ad, int k_in,
                                                         int max_rank,
                                                         const int32_t* __restrict__ off, int E,
                                                         const int32_t* __restrict__ sorted_ids, int P, int top_k,
                                                         const int32_t* __restrict__ row_adapter,
                                                         uint16_t* __restrict__ xa, int64_t row_offset,
                                                         int64_t row_end, int64_t base16, int x_gather) {
    constexpr int KU = NB <= 2 ? 8 : (NB <= 4 ? 4 : 2);
    __shared__ float red[4][NB][4][64];  // [wave][rank block][v][lane]
    __shared__ int s_off[257];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t sub0 = base16 + static_cast<int64_t>(blockIdx.x) * 16;
    if (sub0 >= row_end) return;  // uniform over the workgroup
    stage_offsets(off, E, s_off);
    const SubTile st = sub_tile_expert(static_cast<int>(sub0), s_off, E, n_tab);
    if (st.e < 0) return;  // uniform over the workgroup

    const int m = lane & 15, kq = lane >> 4;
    const int64_t r = sub0 + m;
    const int ad = row_adapter_of(r, row_offset, row_end, st.span_end, sorted_ids, P, top_k, row_adapter, n_ad,
                                  n_tab, st.e, a_tab, b_tab);
    const bool act = ad != kNoAdapter;
    // x row: the sorted row (down), or the row's token in the token-major input (gate/up form)
    const int64_t xrow = act && x_gather ? static_cast<int64_t>(sorted_ids[r] / top_k) : r;
    const uint16_t* xr = act ? x + xrow * k_in + kq * 8 : nullptr;
    const int kpart = ((k_in + 127) / 128) * 32;  // this wave's k range, a multiple of 32
    const int kb = wave * kpart, ke = min(k_in, kb + kpart);
    // the rows' adapters, one pass each (every wave holds the same 16 rows: the passes are uniform over
    // the workgroup); a row of another adapter is computed with this pass's A and not stored
    for (int cur = wave_next_adapter(ad, -1); cur != kNoAdapter; cur = wave_next_adapter(ad, cur)) {
    const uint16_t* Ae = reinterpret_cast<const uint16_t*>(a_tab[static_cast<int64_t>(cur) * n_tab + st.e]);

    f32x4 acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = kb; k0 < ke; k0 += 32 * KU) {
        u32x4 av[KU], bv[KU][NB];
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int kk = k0 + u * 32;
            const bool kin = kk + kq * 8 < ke;
            av[u] = (xr && kin) ? *reinterpret_cast<const u32x4*>(xr + kk) : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < NB; ++j)
                bv[u][j] = kin ? *reinterpret_cast<const u32x4*>(Ae + static_cast<int64_t>(j * 16 + m) * k_in + kk + kq * 8)
                               : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const bf16x8 afr = __builtin_bit_cast(bf16x8, av[u]);
#pragma unroll
            for (int j = 0; j < NB; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, __builtin_bit_cast(bf16x8, bv[u][j]), acc[j], 0, 0, 0);
        }
    }
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave][j][v][lane] = acc[j][v];
    __syncthreads();
    if (wave == 0) {
        // C fragment: rows 4*(lane/16)+v of the sub-tile, rank column 16*j + lane%16
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t rr = sub0 + 4 * kq + v;
            if (row_adapter_of(rr, row_offset, row_end, st.span_end, sorted_ids, P, top_k, row_adapter, n_ad, n_tab,
                               st.e, a_tab, b_tab) != cur)
                continue;
            uint16_t* dst = xa + (rr - row_offset) * max_rank;
#pragma unroll
            for (int j = 0; j < NB; ++j)
                dst[j * 16 + m] = f32_to_bf16((red[0][j][v][lane] + red[1][j][v][lane]) +
                                              (red[2][j][v][lane] + red[3][j][v][lane]));
        }
    }
    __syncthreads();  // red[] is rewritten by the next pass
    }
}

// Expand + fold: each wave takes one 16-row sub-tile and EXP_COLS * EXP_BLOCKS columns, one
// block of EXP_COLS at a time.  The row state (which rows fold, their xa fragments) is read once;
// the base rows and B_e columns of the next block are loaded while the current one is computed
// and written, so a wave keeps a block's loads in flight instead of paying its row lookups and
// a memory round trip per EXP_COLS columns.
template <int NKS>  // k-steps of 32 over max_rank
__global__ __launch_bounds__(NT) void lora_expand_fold_kernel(const uint16_t* __restrict__ xa,
                                                              const uint64_t* a_tab, const uint64_t* b_tab,
                                                              const float* __restrict__ s_tab, int n_tab,
                                                              int n_ad, int n_out, int max_rank,
                                                              const int32_t* __restrict__ off, int E,
                                                              const int32_t* __restrict__ sorted_ids, int P,
                                                              int top_k, const int32_t* __restrict__ row_adapter,
                                                              uint16_t* __restrict__ base, int64_t row_offset,
                                                              int64_t row_end, int64_t base16) {
    __shared__ __attribute__((aligned(16))) uint16_t s_delta[4][16][EXP_COLS];
    __shared__ int s_off[257];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t sub0 = base16 + static_cast<int64_t>(blockIdx.y) * 64 + wave * 16;
    const int slab0 = blockIdx.x * (EXP_COLS * EXP_BLOCKS);
    if (base16 + static_cast<int64_t>(blockIdx.y) * 64 >= row_end) return;  // uniform over the workgroup
    stage_offsets(off, E, s_off);
    if (sub0 >= row_end) return;
    const SubTile st = sub_tile_expert(static_cast<int>(sub0), s_off, E, n_tab);
    if (st.e < 0) return;

    const int m = lane & 15, kq = lane >> 4;
    const int64_t r = sub0 + m;
    const int ad = row_adapter_of(r, row_offset, row_end, st.span_end, sorted_ids, P, top_k, row_adapter, n_ad, n_tab,
                                  st.e, a_tab, b_tab);
    const bool act = ad != kNoAdapter;
    if (__ballot(act) == 0) return;
    u32x4 av[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
        av[ks] = act ? *reinterpret_cast<const u32x4*>(xa + (r - row_offset) * max_rank + ks * 32 + kq * 8)
                                   : u32x4{0, 0, 0, 0};
    // fold rows of this lane (FOLD_RPS rows x FOLD_LPR lanes x 8 columns per step)
    const int col = (lane % FOLD_LPR) * 8;
    int row_ad[FOLD_STEPS];
#pragma unroll
    for (int it = 0; it < FOLD_STEPS; ++it)
        row_ad[it] = row_adapter_of(sub0 + it * FOLD_RPS + lane / FOLD_LPR, row_offset, row_end, st.span_end,
                                    sorted_ids, P, top_k, row_adapter, n_ad, n_tab, st.e, a_tab, b_tab);
    // one pass per adapter present in the sub-tile (every row's xa already holds its own adapter's
    // shrink): the pass computes the delta with that adapter's B_e and folds only its rows
    for (int cur = wave_next_adapter(ad, -1); cur != kNoAdapter; cur = wave_next_adapter(ad, cur)) {
    const int64_t tix = static_cast<int64_t>(cur) * n_tab + st.e;
    const uint16_t* Be = reinterpret_cast<const uint16_t*>(b_tab[tix]);
    const float scale = s_tab[tix];
    bool row_ok[FOLD_STEPS];
#pragma unroll
    for (int it = 0; it < FOLD_STEPS; ++it) row_ok[it] = row_ad[it] == cur;

    u32x4 bvs[2][FOLD_STEPS], bw[2][NKS][EXP_COLS / 16];
    auto load_block = [&](int cb, int set) __attribute__((always_inline)) {
        const int n0 = slab0 + cb * EXP_COLS;
#pragma unroll
        for (int it = 0; it < FOLD_STEPS; ++it) {
            const int64_t rr = sub0 + it * FOLD_RPS + lane / FOLD_LPR;
            bvs[set][it] = (row_ok[it] && n0 + col < n_out)
                               ? *reinterpret_cast<const u32x4*>(base + rr * n_out + n0 + col)
                               : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int c = 0; c < EXP_COLS / 16; ++c) {
                const int n = n0 + c * 16 + m;
                bw[set][ks][c] = n < n_out
                                     ? *reinterpret_cast<const u32x4*>(Be + static_cast<int64_t>(n) * max_rank +
                                                                       ks * 32 + kq * 8)
                                     : u32x4{0, 0, 0, 0};
            }
    };
    load_block(0, 0);
#pragma unroll
    for (int cb = 0; cb < EXP_BLOCKS; ++cb) {
        const int set = cb & 1;
        const int n0 = slab0 + cb * EXP_COLS;
        if (cb + 1 < EXP_BLOCKS) load_block(cb + 1, set ^ 1);
        f32x4 acc[EXP_COLS / 16];
#pragma unroll
        for (int c = 0; c < EXP_COLS / 16; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const bf16x8 afr = __builtin_bit_cast(bf16x8, av[ks]);
#pragma unroll
            for (int c = 0; c < EXP_COLS / 16; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, __builtin_bit_cast(bf16x8, bw[set][ks][c]),
                                                                 acc[c], 0, 0, 0);
        }
        // bf16 delta tile to LDS (rows 4*(lane/16)+v, column 16*c + lane%16)
#pragma unroll
        for (int c = 0; c < EXP_COLS / 16; ++c)
#pragma unroll
            for (int v = 0; v < 4; ++v) s_delta[wave][4 * kq + v][c * 16 + m] = f32_to_bf16(acc[c][v]);
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
        __builtin_amdgcn_wave_barrier();
        // coalesced fold of the delta into the base rows
#pragma unroll
        for (int it = 0; it < FOLD_STEPS; ++it) {
            if (!row_ok[it] || n0 + col >= n_out) continue;
            const int rl = it * FOLD_RPS + lane / FOLD_LPR;
            const int64_t rr = sub0 + rl;
            const u32x4 bv = bvs[set][it];
            const u32x4 dv = *reinterpret_cast<const u32x4*>(&s_delta[wave][rl][col]);
            u32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float b_lo = __uint_as_float(bv[i] << 16), b_hi = __uint_as_float(bv[i] & 0xffff0000u);
                const float d_lo = __uint_as_float(dv[i] << 16), d_hi = __uint_as_float(dv[i] & 0xffff0000u);
                o[i] = pack_bf16x2(fmaf(scale, d_lo, b_lo), fmaf(scale, d_hi, b_hi));
            }
            *reinterpret_cast<u32x4*>(base + rr * n_out + n0 + col) = o;
        }
        __builtin_amdgcn_wave_barrier();  // this block's LDS reads before the next block's writes
    }
    }
}

// ------------------------------------------------------------------ slot-major gather fold
// The decode form of the fold (atlas moe_lora_grouped.rs, moe_lora_gather_bgmv): no sorted
// layout; flat (token, slot) row s takes its expert from indices[s] and its adapter decision
// from row_adapter[s / top_k].  One workgroup per (slot, output chunk), so the grid is fixed by
// the slot count alone.  With one row per expert visit these are matrix-vector products, so
// they run on the vector ALU with coalesced 16-byte loads rather than on MFMA.

struct GatherRow {
    int64_t e;      // table entry: adapter * n_tab + expert
    int64_t row;    // row of base (and of x for the down form)
    int64_t xrow;   // row of x
};

// Is slot s folded, and where?  Ids, map entries and rows are device data: anything outside
// the tables or the buffers skips the slot.
__device__ __forceinline__ bool gather_row(int64_t s, const int32_t* indices, const int32_t* row_map,
                                           const int32_t* row_adapter, int top_k, int x_gather, int n_tab,
                                           int n_ad, const uint64_t* a_tab, const uint64_t* b_tab,
                                           int64_t x_rows, int64_t base_rows, GatherRow& g) {
    const int e = indices[s];
    if (e < 0 || e >= n_tab) return false;
    const int a = row_adapter ? row_adapter[s / top_k] : 0;  // the token's adapter (0 without a map)
    if (a < 0 || a >= n_ad) return false;
    const int64_t ix = static_cast<int64_t>(a) * n_tab + e;
    if (a_tab[ix] == 0 || b_tab[ix] == 0) return false;
    const int64_t row = row_map ? static_cast<int64_t>(row_map[s]) : s;
    if (row < 0 || row >= base_rows) return false;
    const int64_t xrow = x_gather ? s / top_k : row;
    if (xrow >= x_rows) return false;
    g = GatherRow{ix, row, xrow};
    return true;
}

// acc + sum of the 8 products of two rows of 8 bf16, in index order, fp32 fma
__device__ __forceinline__ float dot8_bf16(u32x4 a, u32x4 b, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc = fmaf(__uint_as_float(a[i] << 16), __uint_as_float(b[i] << 16), acc);
        acc = fmaf(__uint_as_float(a[i] & 0xffff0000u), __uint_as_float(b[i] & 0xffff0000u), acc);
    }
    return acc;
}

__device__ __forceinline__ u32x4 load16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// Shrink: xa[s, j] = bf16(x[x row] . A_e[j]) for 16 rank rows per workgroup, its 4 waves taking
// every fourth 128-wide k chunk (so a slot's loads are spread over 4 * max_rank/16 waves and are
// in flight together).  Lanes 16g..16g+15 read one chunk of row 4p+g, 4 rows per load; each row's
// partial sum is reduced over its 16 lanes, then the 4 waves' partials are added in LDS in wave
// order.
__global__ __launch_bounds__(NT) void gather_shrink_kernel(const uint16_t* __restrict__ x,
                                                           const int32_t* __restrict__ indices,
                                                           const int32_t* __restrict__ row_map,
                                                           const int32_t* __restrict__ row_adapter,
                                                           const uint64_t* a_tab, const uint64_t* b_tab, int n_tab,
                                                           int n_ad, int top_k, int x_gather, int64_t x_rows,
                                                           int64_t base_rows, int k_in, int max_rank,
                                                           uint16_t* __restrict__ xa) {
    __shared__ float red[4][16];
    const int64_t s = blockIdx.x;
    GatherRow gr;
    if (!gather_row(s, indices, row_map, row_adapter, top_k, x_gather, n_tab, n_ad, a_tab, b_tab, x_rows, base_rows,
                    gr))
        return;  // uniform over the workgroup
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int j0 = blockIdx.y * 16;  // < max_rank: the grid has max_rank / 16 rows of workgroups
    const uint16_t* Ae = reinterpret_cast<const uint16_t*>(a_tab[gr.e]) + static_cast<int64_t>(j0 + g) * k_in;
    const uint16_t* xr = x + gr.xrow * k_in;
    constexpr int U = 3;  // chunks per wave in flight together
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int q0 = wave * 128; q0 < k_in; q0 += 4 * 128 * U) {
        u32x4 xv[U], av[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = q0 + u * 4 * 128 + c * 8;
            const bool in = k < k_in;
            xv[u] = in ? load16(xr + k) : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int p = 0; p < 4; ++p)
                av[u][p] = in ? load16(Ae + static_cast<int64_t>(4 * p) * k_in + k) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int p = 0; p < 4; ++p) acc[p] = dot8_bf16(xv[u], av[u][p], acc[p]);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) acc[p] += __shfl_xor(acc[p], o, 16);
    }
    if (c == 0) {
#pragma unroll
        for (int p = 0; p < 4; ++p) red[wave][4 * p + g] = acc[p];
    }
    __syncthreads();
    if (threadIdx.x < 16) {
        const int j = threadIdx.x;
        xa[s * max_rank + j0 + j] = f32_to_bf16((red[0][j] + red[1][j]) + (red[2][j] + red[3][j]));
    }
}

// Expand + fold: base[row, n] = bf16(base + scale_e * bf16(xa[s] . B_e[n])) for 256 outputs per
// workgroup, 64 per wave.  Lanes 8g..8g+7 read one 128-byte run of ranks of row n (8 rows per
// load); after the sums over those 8 lanes, lane 8g+c holds output n0 + 8c + g, and one
// cross-lane move gives lane L output n0 + L for a contiguous update of the base row.
__global__ __launch_bounds__(NT) void gather_expand_kernel(const uint16_t* __restrict__ xa,
                                                           const int32_t* __restrict__ indices,
                                                           const int32_t* __restrict__ row_map,
                                                           const int32_t* __restrict__ row_adapter,
                                                           const uint64_t* a_tab, const uint64_t* b_tab,
                                                           const float* __restrict__ s_tab, int n_tab, int n_ad,
                                                           int top_k, int x_gather, int64_t x_rows, int64_t base_rows,
                                                           int n_out, int max_rank, uint16_t* __restrict__ base) {
    const int64_t s = blockIdx.x;
    GatherRow gr;
    if (!gather_row(s, indices, row_map, row_adapter, top_k, x_gather, n_tab, n_ad, a_tab, b_tab, x_rows, base_rows,
                    gr))
        return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 3, c = lane & 7;
    const int n0 = blockIdx.y * 256 + wave * 64;
    if (n0 >= n_out) return;
    const uint16_t* Be = reinterpret_cast<const uint16_t*>(b_tab[gr.e]);
    const float scale = s_tab[gr.e];
    uint16_t* brow = base + gr.row * n_out;
    const int n_mine = n0 + lane;
    const uint16_t b_old = n_mine < n_out ? brow[n_mine] : uint16_t(0);
    // ranks c*8 + 64*i of this lane (max_rank <= 128)
    u32x4 xv[2];
    bool rin[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        rin[i] = c * 8 + 64 * i < max_rank;
        xv[i] = rin[i] ? load16(xa + s * max_rank + c * 8 + 64 * i) : u32x4{0, 0, 0, 0};
    }
    u32x4 bv[8][2];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int n = n0 + 8 * p + g;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            bv[p][i] = (rin[i] && n < n_out) ? load16(Be + static_cast<int64_t>(n) * max_rank + c * 8 + 64 * i)
                                             : u32x4{0, 0, 0, 0};
    }
    float mine = 0.f;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        float a = dot8_bf16(xv[0], bv[p][0], 0.f);
        a = dot8_bf16(xv[1], bv[p][1], a);
#pragma unroll
        for (int o = 4; o >= 1; o >>= 1) a += __shfl_xor(a, o, 8);
        if (c == p) mine = a;
    }
    const float v = __shfl(mine, (lane & 7) * 8 + (lane >> 3));
    if (n_mine < n_out) {
        const float delta = bf16_to_f32(f32_to_bf16(v));
        brow[n_mine] = f32_to_bf16(fmaf(scale, delta, bf16_to_f32(b_old)));
    }
}

}  // namespace

hipError_t launch_lora_shrink(const uint16_t* x, const uint64_t* a_tab, const uint64_t* b_tab, int n_tab, int n_ad, int k_in,
                              int max_rank, const int32_t* offsets, int E, const int32_t* sorted_ids, int P,
                              int top_k, const int32_t* row_adapter, uint16_t* xa, int64_t row_offset,
                              int64_t row_end, int x_gather, hipStream_t s) {
    if (row_end <= row_offset || n_tab <= 0) return hipSuccess;
    const int64_t base16 = (row_offset / 16) * 16;
    const int64_t subs = (row_end - base16 + 15) / 16;
    const dim3 sgrid(static_cast<unsigned>(subs));
#define MOE_SHRINK(NB_)                                                                                          \
    lora_shrink_kernel<NB_><<<sgrid, NT, 0, s>>>(x, a_tab, b_tab, n_tab, n_ad, k_in, max_rank, offsets, E, sorted_ids, \
                                                 P, top_k, row_adapter, xa, row_offset, row_end, base16, x_gather)
    switch (max_rank / 16) {
        case 1: MOE_SHRINK(1); break;
        case 2: MOE_SHRINK(2); break;
        case 3: MOE_SHRINK(3); break;
        case 4: MOE_SHRINK(4); break;
        case 5: MOE_SHRINK(5); break;
        case 6: MOE_SHRINK(6); break;
        case 7: MOE_SHRINK(7); break;
        default: MOE_SHRINK(8); break;
    }
#undef MOE_SHRINK
    return hipGetLastError();
}

hipError_t launch_lora_fold(const uint16_t* x, uint16_t* base, const uint64_t* a_tab, const uint64_t* b_tab,
                            const float* s_tab, int n_tab, int n_ad, int k_in, int n_out, int max_rank,
                            const int32_t* offsets, int E, const int32_t* sorted_ids, int P, int top_k,
                            const int32_t* row_adapter, uint16_t* xa, int64_t row_offset, int64_t row_end,
                            int x_gather, hipStream_t s) {
    if (row_end <= row_offset || n_tab <= 0) return hipSuccess;
    const int64_t base16 = (row_offset / 16) * 16;
    const int64_t tiles = (row_end - base16 + 63) / 64;
    const int64_t subs = (row_end - base16 + 15) / 16;
    const dim3 sgrid(static_cast<unsigned>(subs));
#define MOE_SHRINK(NB_)                                                                                          \
    lora_shrink_kernel<NB_><<<sgrid, NT, 0, s>>>(x, a_tab, b_tab, n_tab, n_ad, k_in, max_rank, offsets, E, sorted_ids, \
                                                 P, top_k, row_adapter, xa, row_offset, row_end, base16, x_gather)
    switch (max_rank / 16) {
        case 1: MOE_SHRINK(1); break;
        case 2: MOE_SHRINK(2); break;
        case 3: MOE_SHRINK(3); break;
        case 4: MOE_SHRINK(4); break;
        case 5: MOE_SHRINK(5); break;
        case 6: MOE_SHRINK(6); break;
        case 7: MOE_SHRINK(7); break;
        default: MOE_SHRINK(8); break;
    }
#undef MOE_SHRINK
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const dim3 grid((n_out + EXP_COLS * EXP_BLOCKS - 1) / (EXP_COLS * EXP_BLOCKS), static_cast<unsigned>(tiles));
#define MOE_EXPAND(NKS_)                                                                                        \
    lora_expand_fold_kernel<NKS_><<<grid, NT, 0, s>>>(xa, a_tab, b_tab, s_tab, n_tab, n_ad, n_out, max_rank, offsets, E, \
                                                      sorted_ids, P, top_k, row_adapter, base, row_offset, row_end, \
                                                      base16)
    switch (max_rank / 32) {
        case 1: MOE_EXPAND(1); break;
        case 2: MOE_EXPAND(2); break;
        case 3: MOE_EXPAND(3); break;
        default: MOE_EXPAND(4); break;
    }
#undef MOE_EXPAND
    return hipGetLastError();
}

hipError_t launch_lora_gather_fold(const uint16_t* x, int64_t x_rows, uint16_t* base, int64_t base_rows,
                                   const int32_t* indices, int64_t n_slots, int top_k, int x_gather,
                                   const int32_t* row_map, const int32_t* row_adapter, const uint64_t* a_tab,
                                   const uint64_t* b_tab, const float* s_tab, int n_tab, int n_ad, int k_in,
                                   int n_out, int max_rank, uint16_t* xa, hipStream_t s) {
    if (n_slots <= 0 || n_tab <= 0) return hipSuccess;
    const dim3 sgrid(static_cast<unsigned>(n_slots), static_cast<unsigned>(max_rank / 16));
    gather_shrink_kernel<<<sgrid, NT, 0, s>>>(x, indices, row_map, row_adapter, a_tab, b_tab, n_tab, n_ad, top_k, x_gather,
                                              x_rows, base_rows, k_in, max_rank, xa);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const dim3 egrid(static_cast<unsigned>(n_slots), static_cast<unsigned>((n_out + 255) / 256));
    gather_expand_kernel<<<egrid, NT, 0, s>>>(xa, indices, row_map, row_adapter, a_tab, b_tab, s_tab, n_tab, n_ad, top_k,
                                              x_gather, x_rows, base_rows, n_out, max_rank, base);
    return hipGetLastError();
}

}  // namespace moe
