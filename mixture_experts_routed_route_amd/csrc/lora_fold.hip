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
// rows of a tile may belong to several (expert, adapter) pairs: the kernels take the pairs present
// one at a time (a uniform loop, usually one pass) and write only that pair's rows in each pass.
// Two launches like the page: the shrink writes the bf16 xa scratch at the local row
// r - row_offset, the expand reads it.  The expert of a row is read on the device from
// expert_offsets (the row's span), so the grid is fixed by host scalars: a window is cut into
// 64-row tiles of four 16-row sub-tiles (block sizes are multiples of 16, so a sub-tile never
// straddles two experts' spans), taken with the tiles of adapted experts first; sentinel rows,
// rows of unadapted experts and rows outside the window do nothing.  Both stages use 16x16x32
// bf16 MFMA with fp32 accumulation.  The shrink gives each half tile a workgroup whose 4 waves
// split k_in and stream x and A_e through per-wave LDS rings; the expand gives each tile and 1024
// columns a workgroup, folds straight from the accumulators (B_e is the MFMA's first operand, its
// rows permuted so that a lane holds 8 consecutive columns of one row) and, for a tile of one
// (expert, adapter) pair, runs a branch-free path that prefetches the next slab.
#include "device_common.h"
#include "launchers.h"

namespace moe {
namespace {

constexpr int NT = 256;
constexpr int EXP_COLS = 64;  // expand: output columns per wave and slab
#ifndef MOE_LORA_EXP_SLABS
#define MOE_LORA_EXP_SLABS 4
#endif
constexpr int EXP_SLABS = MOE_LORA_EXP_SLABS;  // expand: slabs of 4 * EXP_COLS columns per workgroup

// ------------------------------------------------------------------ active tiles first
// A window's 64-row tiles (from base16) are taken in this order: the tiles that hold a row of an
// adapted expert first, in row order, then the rest.  Workgroups are dispatched in index order and
// a tile of an unadapted expert has nothing to do, so with this order the work starts at once
// instead of waiting for CU slots held by such tiles.  Every workgroup stages the expert offsets and
// a per-expert "adapted by some adapter" flag and maps its ordinal k to the k-th such tile (-1 past
// the last): each adapted expert's span sets its tiles' bits in an LDS bitmap (tiles shared by two
// experts are set twice), and one wave counts them.  Windows of more than kMapTiles tiles keep the
// plain order.
constexpr int kMapTiles = 2048;

struct TileMapLds {
    int off[257];
    int bits[kMapTiles / 32];
    unsigned char pres[256];
    int tile;
};

__device__ int stage_and_map_tile(int k, const int32_t* off, int E, const uint64_t* a_tab, const uint64_t* b_tab,
                                  int n_tab, int n_ad, int64_t row_offset, int64_t row_end, int64_t base16,
                                  TileMapLds& L) {
    const int t = threadIdx.x;
    for (int i = t; i <= E; i += blockDim.x) L.off[i] = off[i];
    // an expert is adapted if some adapter holds both of its tables (every expert below n_tab when
    // the tables are too many to look at here: a tile taken for nothing finds no row to fold)
    const bool look = static_cast<int64_t>(n_ad) * n_tab <= 4096;
    for (int e = t; e < E; e += blockDim.x) {
        bool p = false;
        if (e < n_tab) {
            if (!look) p = true;
            for (int a = 0; look && a < n_ad && !p; ++a) {
                const int64_t ix = static_cast<int64_t>(a) * n_tab + e;
                p = a_tab[ix] != 0 && b_tab[ix] != 0;
            }
        }
        L.pres[e] = p;
    }
    if (t < kMapTiles / 32) L.bits[t] = 0;
    if (t == 0) L.tile = -1;
    __syncthreads();
    const int64_t T = (row_end - base16 + 63) / 64;
    if (T > kMapTiles) return k < T ? k : -1;  // uniform over the workgroup
    for (int e = t; e < E; e += blockDim.x) {
        if (!L.pres[e]) continue;
        // the span's rows inside the window (offsets are device data: clamp to the window)
        const int64_t lo = max<int64_t>(L.off[e], row_offset), hi = min<int64_t>(L.off[e + 1], row_end);
        if (lo >= hi) continue;
        const int t0 = static_cast<int>((lo - base16) / 64), t1 = static_cast<int>((hi - 1 - base16) / 64);
        for (int w = t0 >> 5; w <= (t1 >> 5); ++w) {
            const int b0 = max(t0 - w * 32, 0), b1 = min(t1 - w * 32, 31);
            const uint32_t mask = (b1 == 31 ? 0xffffffffu : ((1u << (b1 + 1)) - 1u)) & ~((1u << b0) - 1u);
            atomicOr(reinterpret_cast<unsigned int*>(&L.bits[w]), mask);
        }
    }
    __syncthreads();
    if (t < 64) {  // the first wave: word t holds tiles 32 t .. 32 t + 31
        uint32_t word = t < kMapTiles / 32 ? static_cast<uint32_t>(L.bits[t]) : 0u;
        const int c = __builtin_popcount(word);
        const int incl = wave_inclusive_scan(c);
        if (k >= incl - c && k < incl) {
            for (int i = k - (incl - c); i > 0; --i) word &= word - 1;  // drop the lower set bits
            L.tile = t * 32 + __builtin_ctz(word);
        }
    }
    __syncthreads();
    return L.tile;
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
// adapter in [0, n_ad) and that adapter adapts expert e), else kNoAdapter.  With one adapter, `pres`
// (LDS: expert e adapted, staged with the tile map) stands for the table lookup.
__device__ __forceinline__ int row_adapter_of(int64_t r, int64_t row_offset, int64_t row_end, int span_end,
                                              const int32_t* sorted_ids, int P, int top_k,
                                              const int32_t* row_adapter, int n_ad, int n_tab, int e,
                                              const uint64_t* a_tab, const uint64_t* b_tab,
                                              const unsigned char* pres = nullptr) {
    if (r < row_offset || r >= row_end || r >= span_end) return kNoAdapter;
    const int p = sorted_ids[r];
    if (p < 0 || p >= P) return kNoAdapter;
    const int a = row_adapter ? row_adapter[p / top_k] : 0;
    if (a < 0 || a >= n_ad) return kNoAdapter;
    if (pres && n_ad == 1) return pres[e] ? a : kNoAdapter;
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
    return __builtin_amdgcn_readfirstlane(v);  // the same in every lane: let the compiler know
}

constexpr int kNoKey = 0x7fffffff;  // "no (expert, adapter) pair": above every real key
constexpr uint32_t kOob = 0x80000000u;  // a buffer offset past every range used here

// Smallest key above `after` held by any lane of the wave (kNoKey if none), the same in every lane.
__device__ __forceinline__ int wave_next_key(int mine, int after) {
    int v = mine > after ? mine : kNoKey;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const int w = __shfl_xor(v, o);
        v = w < v ? w : v;
    }
    return __builtin_amdgcn_readfirstlane(v);
}

// Shrink LDS: each wave's ring of R k-steps (x of the workgroup's SUBS * 16 rows, then A_e's 16 NB
// rank rows, 32 k each, in 1 KB blocks of 16 rows: block byte (c * 16 + r) * 16 holds chunk c (k
// 8c..8c+7) of row r, so that lane L of a fragment read takes bytes 16 L..16 L + 15); after the K
// loop the same memory holds the partial sums of the four waves.
template <int NB, int SUBS>
struct ShrinkLds {
    static constexpr int R = SUBS == 4 ? (NB <= 4 ? 4 : 3) : (NB <= 4 ? 3 : 2);  // k-steps in flight per wave
    static constexpr int X_BYTES = SUBS * 1024;
    static constexpr int STAGE = X_BYTES + NB * 1024;
    static constexpr int WAVE = R * STAGE;
    static constexpr int RING = 4 * WAVE;
    static constexpr int RED = 4 * SUBS * NB * 4 * 64 * 4;
    static constexpr int BYTES = RING > RED ? RING : RED;
    static constexpr int LOADS = SUBS + NB;  // load instructions per k-step and wave
};

#ifndef MOE_LORA_SHRINK_SUBS
#define MOE_LORA_SHRINK_SUBS 2
#endif
constexpr int SHRINK_SUBS = MOE_LORA_SHRINK_SUBS;  // 16-row sub-tiles per shrink workgroup (2 or 4)

// Shrink: a workgroup takes SUBS 16-row sub-tiles of a 64-row tile (SUBS = 2: the tile's two halves
// go to workgroups 8 ids apart, which run on the same XCD and share A_e in its L2); its 4 waves take
// a quarter of k_in each and add their partial sums in LDS.  The rows are taken one (expert,
// adapter) pair at a time (a uniform loop over the pairs present, usually one); in the pass of a
// pair, a wave streams its k range of x and of the pair's A_e through its LDS ring with direct
// global->LDS loads, R k-steps ahead, and each k-step's A_e fragments serve all SUBS sub-tiles.
// The loads are not tracked by the compiler (see dma16): each k-step waits with an explicit vmcnt
// for its own loads only.  Chunks past the wave's k range load zeros; x rows of other passes (or not
// folded) give results in their own output rows only, which this pass does not store.
// NB = rank blocks of 16 (max_rank / 16).
template <int NB, int SUBS>
__global__ __launch_bounds__(NT) void lora_shrink_kernel(const uint16_t* __restrict__ x, const uint64_t* a_tab,
                                                         const uint64_t* b_tab, int n_tab, int n_ad, int k_in,
                                                         int max_rank,
                                                         const int32_t* __restrict__ off, int E,
                                                         const int32_t* __restrict__ sorted_ids, int P, int top_k,
                                                         const int32_t* __restrict__ row_adapter,
                                                         uint16_t* __restrict__ xa, int64_t row_offset,
                                                         int64_t row_end, int64_t base16, int x_gather) {
    static_assert(SUBS == 2 || SUBS == 4, "sub-tiles per workgroup");
    constexpr int ROWS = SUBS * 16;
    using L = ShrinkLds<NB, SUBS>;
    constexpr int R = L::R;
    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    __shared__ TileMapLds tm;
    __shared__ int s_key[ROWS];       // (expert << 16) | adapter of each row, kNoKey: not folded
    __shared__ int64_t s_xrow[ROWS];  // its x row
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // tile ordinal and part: with two parts, ids 16 q + p and 16 q + 8 + p (p < 8) share tile 8 q + p
    const int b = blockIdx.x;
    const int kt = SUBS == 4 ? b : (b >> 4) * 8 + (b & 7);
    const int part = SUBS == 4 ? 0 : (b >> 3) & 1;
    const int tile = stage_and_map_tile(kt, off, E, a_tab, b_tab, n_tab, n_ad, row_offset, row_end, base16, tm);
    if (tile < 0) return;  // uniform over the workgroup
    const int64_t row0 = base16 + static_cast<int64_t>(tile) * 64 + part * ROWS;
    const int* s_off = tm.off;
    if (threadIdx.x < ROWS) {
        const int64_t r = row0 + threadIdx.x;
        const int64_t sub0 = row0 + (threadIdx.x & ~15);
        SubTile st{-1, 0};
        if (sub0 < row_end) st = sub_tile_expert(static_cast<int>(sub0), s_off, E, n_tab);
        const int a = st.e >= 0 ? row_adapter_of(r, row_offset, row_end, st.span_end, sorted_ids, P, top_k,
                                                 row_adapter, n_ad, n_tab, st.e, a_tab, b_tab, tm.pres)
                                : kNoAdapter;
        s_key[threadIdx.x] = a != kNoAdapter ? (st.e << 16) | a : kNoKey;
        // x row: the sorted row (down), or the row's token in the token-major input (gate/up form)
        s_xrow[threadIdx.x] = a != kNoAdapter ? (x_gather ? static_cast<int64_t>(sorted_ids[r] / top_k) : r) : 0;
    }
    __syncthreads();

    const int m = lane & 15, kq = lane >> 4;
    const int key_l = lane < ROWS ? s_key[lane] : kNoKey;  // lane l holds row l's key, for the pass loop
    // this lane's load sources: chunk kq of row m of x block q (sub-tile q), of rank row 16 j + m
    const uint16_t* xsrc[SUBS];
#pragma unroll
    for (int q = 0; q < SUBS; ++q) xsrc[q] = x + s_xrow[q * 16 + m] * k_in + kq * 8;
    const int kpart = ((k_in + 127) / 128) * 32;  // this wave's k range, a multiple of 32
    const int kb = wave * kpart, ke = min(k_in, kb + kpart);
    const int nsteps = ke > kb ? (ke - kb + 31) / 32 : 0;  // uniform over the wave
    const uint32_t ring = lds_u32(smem) + wave * L::WAVE;
    const char* ring_p = smem + wave * L::WAVE;

    for (int cur = wave_next_key(key_l, -1); cur != kNoKey; cur = wave_next_key(key_l, cur)) {
        const int e = cur >> 16, a = cur & 0xffff;
        const uint16_t* Ae = reinterpret_cast<const uint16_t*>(a_tab[static_cast<int64_t>(a) * n_tab + e]) +
                             static_cast<int64_t>(m) * k_in + kq * 8;
        // k-step t (k = kb + 32 t) into ring slot t % R
        auto issue = [&](int t) {
            const int k = kb + 32 * t;
            const bool in = k + kq * 8 < ke;
            const uint32_t slot = __builtin_amdgcn_readfirstlane(ring + (t % R) * L::STAGE);  // m0 takes a scalar
#pragma unroll
            for (int q = 0; q < SUBS; ++q)
                dma16(in ? static_cast<const void*>(xsrc[q] + k) : kZero16, slot + q * 1024);
#pragma unroll
            for (int j = 0; j < NB; ++j)
                dma16(in ? static_cast<const void*>(Ae + static_cast<int64_t>(j * 16) * k_in + k) : kZero16,
                      slot + L::X_BYTES + j * 1024);
        };
        f32x4 acc[SUBS][NB];
#pragma unroll
        for (int q = 0; q < SUBS; ++q)
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[q][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int t = 0; t < R && t < nsteps; ++t) issue(t);
        for (int t = 0; t < nsteps; ++t) {
            // k-step t has landed once at most `ahead` later k-steps' loads are still in flight
            const int ahead = min(R - 1, nsteps - 1 - t);
            if (ahead >= 3) wait_vmcnt<3 * L::LOADS>();
            else if (ahead == 2) wait_vmcnt<2 * L::LOADS>();
            else if (ahead == 1) wait_vmcnt<L::LOADS>();
            else wait_vmcnt<0>();
            asm volatile("" ::: "memory");  // the LDS reads stay below the wait
            const char* st = ring_p + (t % R) * L::STAGE + lane * 16;
            u32x4 xv[SUBS], av[NB];
#pragma unroll
            for (int q = 0; q < SUBS; ++q) xv[q] = *reinterpret_cast<const u32x4*>(st + q * 1024);
#pragma unroll
            for (int j = 0; j < NB; ++j) av[j] = *reinterpret_cast<const u32x4*>(st + L::X_BYTES + j * 1024);
            // the slot's reads are done before it is refilled (the clobber keeps them above this point)
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (t + R < nsteps) issue(t + R);
#pragma unroll
            for (int q = 0; q < SUBS; ++q)
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[q][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xv[q]),
                                                                        __builtin_bit_cast(bf16x8, av[j]),
                                                                        acc[q][j], 0, 0, 0);
        }
        // the four waves' partial sums (in the ring's memory, once every wave is past its K loop);
        // wave w adds and stores rank blocks w, w + 4
        float (*red)[SUBS][NB][4][64] = reinterpret_cast<float (*)[SUBS][NB][4][64]>(smem);
        __syncthreads();
#pragma unroll
        for (int q = 0; q < SUBS; ++q)
#pragma unroll
            for (int j = 0; j < NB; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) red[wave][q][j][v][lane] = acc[q][j][v];
        __syncthreads();
        // C fragment: rows 4*(lane/16)+v of sub-tile q, rank column 16*j + lane%16
#pragma unroll
        for (int q = 0; q < SUBS; ++q)
#pragma unroll
            for (int j = wave; j < NB; j += 4)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int rl = q * 16 + 4 * kq + v;
                    if (s_key[rl] != cur) continue;
                    xa[(row0 + rl - row_offset) * max_rank + j * 16 + m] =
                        f32_to_bf16((red[0][q][j][v][lane] + red[1][q][j][v][lane]) +
                                    (red[2][q][j][v][lane] + red[3][q][j][v][lane]));
                }
        __syncthreads();  // the ring is refilled by the next pass
    }
}

// Expand + fold: a workgroup takes a 64-row tile (four 16-row sub-tiles) and EXP_SLABS slabs of
// 4 * EXP_COLS columns; in each slab wave w owns EXP_COLS columns of all four sub-tiles.  The tile's
// row adapters are looked up once (a chain of dependent loads: offsets, sorted id, token adapter,
// table entry) and its xa rows loaded once, for all slabs.  The MFMA takes B_e as its first operand,
// delta^T = B_e xa^T, with B_e's rows permuted so that each lane ends up holding 8 consecutive
// columns of one row: the fold runs on the accumulators directly, with 16-byte loads and stores of
// the base rows.
//   16x16x32 block c (of 4) of a k-step, operand row i (lane i + 16 * kq) <- B_e row
//   n0 + 32 * (c >> 1) + 8 * (i >> 2) + 4 * (c & 1) + (i & 3); accumulator v of lane (j, kq) of block c
//   is then delta[row j][n0 + 32 * (c >> 1) + 8 * kq + 4 * (c & 1) + v].
// Two paths:
//  * one expert and one adapter in the tile (the usual case): straight-line code.  Base rows and B_e
//    are read and written with buffer instructions whose offsets are pushed out of range for lanes
//    and columns with nothing to do (out-of-range loads return 0, stores are dropped), and the next
//    slab's B_e and base rows are loaded before the current slab is computed.  With no branches
//    between a load and its use, the wait before each slab covers only that slab's loads, not the
//    stores of the slab before it (the vector memory counter is one in-order count of loads and
//    stores).
//  * otherwise (sub-tiles of several experts, rows of several adapters): per sub-tile, one pass per
//    adapter present, each loading that (expert, adapter)'s B_e.
template <int NKS>  // k-steps of 32 over max_rank
__global__ __launch_bounds__(NT) void lora_expand_fold_kernel(const uint16_t* __restrict__ xa,
                                                              const uint64_t* a_tab, const uint64_t* b_tab,
                                                              const float* __restrict__ s_tab, int n_tab,
                                                              int n_ad, int n_out, int max_rank,
                                                              const int32_t* __restrict__ off, int E,
                                                              const int32_t* __restrict__ sorted_ids, int P,
                                                              int top_k, const int32_t* __restrict__ row_adapter,
                                                              uint16_t* __restrict__ base, int64_t row_offset,
                                                              int64_t row_end, int64_t base16, int n_groups,
                                                              int fast_ok) {
    __shared__ TileMapLds tm;
    __shared__ int s_rad[64];  // adapter of each row of the tile (kNoAdapter: not folded)
    __shared__ int s_e[4];     // expert of each sub-tile (-1: nothing to do)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int k = blockIdx.x / n_groups, grp = blockIdx.x - k * n_groups;
    const int tile = stage_and_map_tile(k, off, E, a_tab, b_tab, n_tab, n_ad, row_offset, row_end, base16, tm);
    if (tile < 0) return;  // uniform over the workgroup
    const int64_t tile0 = base16 + static_cast<int64_t>(tile) * 64;
    const int* s_off = tm.off;
    // the 64 rows' adapters, one row per thread of the first wave, so that their chains of dependent
    // loads are in flight together
    if (threadIdx.x < 64) {
        const int64_t sub0 = tile0 + (threadIdx.x & ~15);
        SubTile st{-1, 0};
        if (sub0 < row_end) st = sub_tile_expert(static_cast<int>(sub0), s_off, E, n_tab);
        s_rad[threadIdx.x] = st.e >= 0 ? row_adapter_of(tile0 + threadIdx.x, row_offset, row_end, st.span_end,
                                                        sorted_ids, P, top_k, row_adapter, n_ad, n_tab, st.e,
                                                        a_tab, b_tab, tm.pres)
                                       : kNoAdapter;
        if ((threadIdx.x & 15) == 0) s_e[threadIdx.x >> 4] = st.e;
    }
    __syncthreads();
    // no workgroup barrier after this point: a wave with nothing to do leaves on its own
    constexpr int SLAB = 4 * EXP_COLS;
    const int cw = grp * (SLAB * EXP_SLABS) + wave * EXP_COLS;  // this wave's first column in slab 0
    if (cw >= n_out) return;
    const int m = lane & 15, kq = lane >> 4;

    // the four sub-tiles: expert, and for this lane the adapter and xa fragments of its row m; the
    // tile's first (expert, adapter) pair, and whether it is the only one
    int e_s[4], ad[4];
    u32x4 av[4][NKS];
    int pe = -1, pa = kNoAdapter;
    bool mixed = false;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        e_s[s] = __builtin_amdgcn_readfirstlane(s_e[s]);  // one value per sub-tile
        ad[s] = s_rad[s * 16 + m];
        // xa row (row 0 when not folded: a valid address whose values reach only output rows that
        // are not stored)
        const int64_t xrow = ad[s] != kNoAdapter ? tile0 + s * 16 + m - row_offset : 0;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            av[s][ks] = *reinterpret_cast<const u32x4*>(xa + xrow * max_rank + ks * 32 + kq * 8);
        if (e_s[s] < 0) continue;
        const int a0 = wave_next_adapter(ad[s], -1);
        if (a0 == kNoAdapter) continue;
        if (pe < 0) {
            pe = e_s[s];
            pa = a0;
        }
        mixed = mixed || e_s[s] != pe || a0 != pa || wave_next_adapter(ad[s], a0) != kNoAdapter;
    }
    if (pe < 0) return;  // nothing folded in this tile (uniform over the workgroup)

    if (!mixed && fast_ok) {
        // ---- one (expert, adapter) pair: straight-line, software-pipelined over the slabs
        const int64_t pix = static_cast<int64_t>(pa) * n_tab + pe;
        const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<void*>(b_tab[pix]), 0, n_out * max_rank * 2, 0x00020000);
        const float scale = s_tab[pix];
        const int rows_here = static_cast<int>(min<int64_t>(64, row_end - tile0));
        const __amdgpu_buffer_rsrc_t rc =
            __builtin_amdgcn_make_buffer_rsrc(base + tile0 * n_out, 0, rows_here * n_out * 2, 0x00020000);
        // byte offsets: B_e fragment (ks, c) at column base n0 = bo[ks][c] + 2 * n0 * max_rank (columns
        // past n_out fall past the range); base row of sub-tile s, column n: ro[s] + 2 n, or out of range
        int bo[NKS][4], ro[4];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                bo[ks][c] = ((32 * (c >> 1) + 8 * (m >> 2) + 4 * (c & 1) + (m & 3)) * max_rank + ks * 32 + kq * 8) * 2;
#pragma unroll
        for (int s = 0; s < 4; ++s) ro[s] = ad[s] == pa ? (s * 16 + m) * n_out * 2 : -1;
        auto load_b = [&](u32x4 (&w)[NKS][4], int n0) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    w[ks][c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                             rb, bo[ks][c] + 2 * n0 * max_rank, 0, 0));
        };
        auto c_off = [&](int s, int n) -> int {
            return (ro[s] >= 0 && n < n_out) ? ro[s] + 2 * n : static_cast<int>(kOob);
        };
        auto load_c = [&](u32x4 (&v)[4][2], int n0) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    v[s][h] = __builtin_bit_cast(
                        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, c_off(s, n0 + 32 * h + 8 * kq), 0, 0));
        };
        u32x4 bw[NKS][4], bwn[NKS][4], bv[4][2], bvn[4][2];
        load_b(bwn, cw);
        load_c(bvn, cw);
#pragma unroll
        for (int j = 0; j < EXP_SLABS; ++j) {
            const int n0 = cw + j * SLAB;
            if (n0 >= n_out) break;  // uniform over the wave
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int c = 0; c < 4; ++c) bw[ks][c] = bwn[ks][c];
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int h = 0; h < 2; ++h) bv[s][h] = bvn[s][h];
            if (j + 1 < EXP_SLABS) {  // the next slab's loads go out before this slab's work
                load_b(bwn, n0 + SLAB);
                load_c(bvn, n0 + SLAB);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                f32x4 acc[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bw[ks][c]),
                                                                         __builtin_bit_cast(bf16x8, av[s][ks]),
                                                                         acc[c], 0, 0, 0);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const u32x4 b = bv[s][h];
                    u32x4 o;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        // columns 2i, 2i + 1 of the chunk: accumulators 2(i & 1), 2(i & 1) + 1 of block 2h + (i >> 1)
                        const f32x4& a4 = acc[2 * h + (i >> 1)];
                        const uint32_t dv = pack_bf16x2(a4[2 * (i & 1)], a4[2 * (i & 1) + 1]);  // bf16 delta
                        const float d_lo = __uint_as_float(dv << 16), d_hi = __uint_as_float(dv & 0xffff0000u);
                        const float b_lo = __uint_as_float(b[i] << 16), b_hi = __uint_as_float(b[i] & 0xffff0000u);
                        o[i] = pack_bf16x2(fmaf(scale, d_lo, b_lo), fmaf(scale, d_hi, b_hi));
                    }
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), rc,
                                                           c_off(s, n0 + 32 * h + 8 * kq), 0, 0);
                }
            }
        }
        return;
    }

    // ---- general tile: per sub-tile, one pass per adapter present
    for (int j = 0; j < EXP_SLABS; ++j) {
        const int n0 = cw + j * SLAB;
        if (n0 >= n_out) break;  // uniform over the wave
        u32x4 bv[4][2];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int n = n0 + 32 * h + 8 * kq;
                bv[s][h] = (ad[s] != kNoAdapter && n < n_out)
                               ? *reinterpret_cast<const u32x4*>(base + (tile0 + s * 16 + m) * n_out + n)
                               : u32x4{0, 0, 0, 0};
            }
        u32x4 bw[NKS][4];
        int have_e = -1, have_a = -1;
        float scale = 0.f;
        for (int s = 0; s < 4; ++s) {
            if (e_s[s] < 0) continue;  // uniform over the wave
            for (int cur = wave_next_adapter(ad[s], -1); cur != kNoAdapter; cur = wave_next_adapter(ad[s], cur)) {
                if (e_s[s] != have_e || cur != have_a) {  // B_e of this expert and adapter, this slab
                    const int64_t tix = static_cast<int64_t>(cur) * n_tab + e_s[s];
                    const uint16_t* Be = reinterpret_cast<const uint16_t*>(b_tab[tix]);
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const int n = n0 + 32 * (c >> 1) + 8 * (m >> 2) + 4 * (c & 1) + (m & 3);
                            bw[ks][c] = n < n_out ? *reinterpret_cast<const u32x4*>(
                                                        Be + static_cast<int64_t>(n) * max_rank + ks * 32 + kq * 8)
                                                  : u32x4{0, 0, 0, 0};
                        }
                    scale = s_tab[tix];
                    have_e = e_s[s];
                    have_a = cur;
                }
                f32x4 acc[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bw[ks][c]),
                                                                         __builtin_bit_cast(bf16x8, av[s][ks]),
                                                                         acc[c], 0, 0, 0);
                if (ad[s] != cur) continue;  // this lane's row belongs to another pass (or is not folded)
                const int64_t row = tile0 + s * 16 + m;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int n = n0 + 32 * h + 8 * kq;
                    if (n >= n_out) continue;
                    const u32x4 b = bv[s][h];
                    u32x4 o;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const f32x4& a4 = acc[2 * h + (i >> 1)];
                        const uint32_t dv = pack_bf16x2(a4[2 * (i & 1)], a4[2 * (i & 1) + 1]);  // bf16 delta
                        const float d_lo = __uint_as_float(dv << 16), d_hi = __uint_as_float(dv & 0xffff0000u);
                        const float b_lo = __uint_as_float(b[i] << 16), b_hi = __uint_as_float(b[i] & 0xffff0000u);
                        o[i] = pack_bf16x2(fmaf(scale, d_lo, b_lo), fmaf(scale, d_hi, b_hi));
                    }
                    *reinterpret_cast<u32x4*>(base + row * n_out + n) = o;
                }
            }
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

// shrink workgroups for a window of `tiles` 64-row tiles: one per tile, or with two per tile, 16 per
// group of 8 tiles (the last group whole; its ids past the window find no tile)
int64_t shrink_blocks(int64_t tiles) { return SHRINK_SUBS == 4 ? tiles : (tiles + 7) / 8 * 16; }

}  // namespace

hipError_t launch_lora_shrink(const uint16_t* x, const uint64_t* a_tab, const uint64_t* b_tab, int n_tab, int n_ad, int k_in,
                              int max_rank, const int32_t* offsets, int E, const int32_t* sorted_ids, int P,
                              int top_k, const int32_t* row_adapter, uint16_t* xa, int64_t row_offset,
                              int64_t row_end, int x_gather, hipStream_t s) {
    if (row_end <= row_offset || n_tab <= 0) return hipSuccess;
    const int64_t base16 = (row_offset / 16) * 16;
    const dim3 sgrid(static_cast<unsigned>(shrink_blocks((row_end - base16 + 63) / 64)));
#define MOE_SHRINK(NB_)                                                                                          \
    lora_shrink_kernel<NB_, SHRINK_SUBS><<<sgrid, NT, 0, s>>>(x, a_tab, b_tab, n_tab, n_ad, k_in, max_rank, offsets, E, \
                                                              sorted_ids, P, top_k, row_adapter, xa, row_offset,   \
                                                              row_end, base16, x_gather)
    switch (max_rank / 32) {  // max_rank is 32, 64, 96 or 128
        case 1: MOE_SHRINK(2); break;
        case 2: MOE_SHRINK(4); break;
        case 3: MOE_SHRINK(6); break;
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
    const dim3 sgrid(static_cast<unsigned>(shrink_blocks(tiles)));
#define MOE_SHRINK(NB_)                                                                                          \
    lora_shrink_kernel<NB_, SHRINK_SUBS><<<sgrid, NT, 0, s>>>(x, a_tab, b_tab, n_tab, n_ad, k_in, max_rank, offsets, E, \
                                                              sorted_ids, P, top_k, row_adapter, xa, row_offset,   \
                                                              row_end, base16, x_gather)
    switch (max_rank / 32) {  // max_rank is 32, 64, 96 or 128
        case 1: MOE_SHRINK(2); break;
        case 2: MOE_SHRINK(4); break;
        case 3: MOE_SHRINK(6); break;
        default: MOE_SHRINK(8); break;
    }
#undef MOE_SHRINK
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int n_groups = (n_out + 4 * EXP_COLS * EXP_SLABS - 1) / (4 * EXP_COLS * EXP_SLABS);
    const dim3 grid(static_cast<unsigned>(tiles * n_groups));
    // the one-pair path addresses a tile's base rows and a B_e with 32-bit buffer offsets
    const int fast_ok = static_cast<int64_t>(64) * n_out * 2 < kOob && static_cast<int64_t>(n_out) * max_rank * 2 < kOob;
#define MOE_EXPAND(NKS_)                                                                                        \
    lora_expand_fold_kernel<NKS_><<<grid, NT, 0, s>>>(xa, a_tab, b_tab, s_tab, n_tab, n_ad, n_out, max_rank, offsets, E, \
                                                      sorted_ids, P, top_k, row_adapter, base, row_offset, row_end,  \
                                                      base16, n_groups, fast_ok)
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
