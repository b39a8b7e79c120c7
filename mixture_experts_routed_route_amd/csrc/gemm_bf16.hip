// Grouped expert GEMM, bf16 (or fp8) weights, one launch for all experts (the grouped gate/up and
// down roles of metrale cutlass/grouped.rs; gather through sorted ids and sentinel masking
// as in ferrum-kernels triton_fused_moe.rs).
//
// Tiling.  A tile is up to BM consecutive sorted rows of ONE expert: expert e's padded span
// [off[e], off[e+1]) is cut into ceil(span/BM) row tiles.  Each workgroup rebuilds that list from
// expert_offsets once (a 256-wide LDS scan of the per-expert row-tile counts), so launches depend
// on host scalars only.  The weight panel of a tile is BP = 256 weight rows: for gate/up the 128
// gate rows and the 128 up rows of the same output columns (SiLU(gate)*up is formed from the
// fp32 accumulators), for down 256 output columns.
//
// Pipeline.  NW waves in a (NW/2) x 2 grid, each owning 64 x 128 of the tile as 32x32x16 bf16
// MFMA blocks with fp32 accumulators.  256-row tiles use 8 waves, two per SIMD, so one wave's
// LDS and barrier waits overlap the other's MFMAs; there waves 0-3 issue all of a stage's loads
// (see the DMA sources below), so that the address unit stalls only one wave of each SIMD.  K advances BK at a time through a ring of
// STAGES LDS buffers filled by direct global->LDS loads (global_load_lds_dwordx4: no VGPR
// staging, no LDS store instructions; issued from inline asm, see dma16); STAGES-1 stages are in
// flight while one is computed.  Each thread waits on its own loads with an explicit vmcnt, then
// a bare s_barrier makes the stage visible to all waves (a fenced barrier would drain the later
// stages' loads too).  LDS rows are XOR-swizzled in 16-byte chunks so that the 32-row fragment
// reads are free of LDS bank conflicts.  Fragments of the next K step are read from LDS while the
// MFMAs of the current one run.  Rows that hold no token (sentinels, padding) load a harmless
// valid row and are never stored; k past K loads zeros.
//
// Ragged tails.  An expert's last tile usually holds fewer tokens than BM.  Its rows past the last
// token are sentinels, so each wave counts the 32-row A fragments of its own rows that hold a
// token (0, 1 or 2) and runs a main loop compiled for that count: empty fragments cost no LDS
// reads and no MFMAs, and the wave still loads and meets the barriers.
//
// Schedule.  Logical tiles run in bands of GM row tiles: within a band, GM row tiles of one
// column panel are consecutive.  Workgroup ids are dealt round-robin over the 8 XCDs, so XCD x
// takes the contiguous range [x*T/8, (x+1)*T/8) of the T real tiles and its workgroups stride
// through it; the ~32 tiles an XCD runs at once then cover a few panels x GM row tiles and share
// A tiles and weight panels in that XCD's L2.  With more than 4 tiles per compute unit the grid
// is persistent (one workgroup per compute unit): before a tile's epilogue the workgroup takes the
// next tile's rows and issues its first stage into the free LDS buffer, so the next tile's first
// load latency hides behind this epilogue; with 2 stages, the next tile's expert search and
// sorted-id loads already run inside this tile's main loop (see pf below).  With fewer tiles
// (and no workspace), one workgroup per tile.
//
// Split tail (only with a caller workspace).  When the tiles do not fill a whole number of
// rounds of the persistent grid, the last partial round would leave most compute units idle
// for a whole tile.  Instead every workgroup runs the same number of whole tiles and the
// remaining tiles are cut along K into pieces that together occupy the grid; pieces of one tile
// run on one XCD and pieces that run together start at the same K step, so they still share A
// tiles and weight panels in L2.  Pieces meet through fp32 partials in the workspace: each
// writes its partial with device-coherent stores and counts itself on the tile's counter; the
// last one sums all partials in piece order (so results do not depend on arrival order),
// stores the tile and resets the counter.  No workgroup ever waits for another.
//
// Epilogue.  Straight from the accumulators, no LDS: neighbouring lanes (columns c, c+1) swap
// one value through DPP so that each lane holds two adjacent columns of one row, converts them
// with one v_cvt_pk_bf16_f32 and stores 4 bytes.
//
// fp8 form (FP8 = true; the quantised prefill variant, codes from gemm_fp8.hip).  A and the
// weights are OCP E4M3 codes, one byte each, so the same tiles and LDS rows hold 128 k per
// stage instead of 64: a row is still 128 bytes with the same swizzle, and a load instruction
// still fills 1 KB.  The MFMA is the CDNA4 32x32x64 fp8 one (unit block scales), whose operand is
// two 16-byte chunks of a row; A and B take the same lane -> k map, so every product pairs the
// same k.  Its 32-byte fragments do not fit twice beside the accumulators of an 8-wave tile, so
// there a wave reads each k-step's fragments just before its MFMAs.  The epilogue multiplies by
// the row's activation scale and the column's weight scale before SiLU * up.
//
// LoRA epilogue (LORA > 0; atlas moe_lora_grouped.rs): before the stores, rows of adapted experts
// get bf16(bf16(acc) + scale * bf16(xa . B_e^T)), from the shrink's xa rows (by sorted row) and the
// adapter's B_e.  Gate/up folds the gate and up blocks with their own tables before SiLU * up;
// down folds the expert output.  The one-adapter down form at rank BK runs the delta as one more
// K stage through the last stage's LDS buffer; the other forms fetch the fragments from memory.
#include <type_traits>

#include "device_common.h"
#include "launchers.h"

namespace moe {
namespace {

constexpr int BP = 256;
#ifndef MOE_GEMM_BAND_ROWS
#define MOE_GEMM_BAND_ROWS 2048   // sorted rows per band of the tile schedule
#endif
#ifndef MOE_GEMM_BIG_BK
#define MOE_GEMM_BIG_BK 64       // k per LDS stage of the 256-row tiles
#endif
#ifndef MOE_GEMM_BIG_ROWS
#define MOE_GEMM_BIG_ROWS 128  // 256-row tiles when experts average at least this many rows
#endif
#ifndef MOE_GEMM_A_LATE
#define MOE_GEMM_A_LATE 1  // asymmetric issue: activation-row loads of a stage issued at this k-step
#endif
#ifndef MOE_FP8_A_LATE
#define MOE_FP8_A_LATE 1  // the same for the fp8 form (two k-steps per stage)
#endif
#ifndef MOE_GEMM_ASYM
#define MOE_GEMM_ASYM 1  // 8 waves, 2 stages: waves 0-3 issue all of a stage's loads
#endif
#ifndef MOE_GEMM_SPLIT_MIN_STAGES
#define MOE_GEMM_SPLIT_MIN_STAGES 8  // K stages per piece of a split tail tile, at least
#endif
#ifndef MOE_GEMM_BIG_STAGES
#define MOE_GEMM_BIG_STAGES 2    // LDS stages of the 256-row tiles (stage = 512 rows x BK bf16)
#endif
constexpr int kMaxE = 256;

// BK: k per stage in elements of ES bytes (bf16: 2, fp8: 1); an LDS row is BK * ES bytes.
template <bool GATE_UP, int BM, int BK, int STAGES, int NW, int ES = 2>
struct Cfg {
    static constexpr int NT = 64 * NW;                  // threads
    static constexpr int WAVES_M = NW / 2;              // wave grid WAVES_M x 2
    static constexpr int CE = 16 / ES;                  // elements per 16-byte chunk
    static constexpr int CPR = BK / CE;                 // 16-byte chunks per LDS row
    static constexpr int RP = 256 / (BK * ES);          // LDS rows per 256-byte line of the 64 banks
    static constexpr int A_ELEMS = BM * BK;
    static constexpr int B_ELEMS = BP * BK;
    static constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
    static constexpr int ROWS_PER_INST = 1024 / (BK * ES);  // rows one wave-wide 1 KB load fills
    static constexpr int A_INST = BM / ROWS_PER_INST / NW;  // load instructions per wave per stage
    static constexpr int B_INST = BP / ROWS_PER_INST / NW;
    static constexpr int LOADS = A_INST + B_INST;
    static constexpr int WM = BM / WAVES_M;              // rows per wave
    static constexpr int FI = WM / 32;                   // A fragments (32 rows) per wave
    static constexpr int NCOL = GATE_UP ? BP / 2 : BP;   // output columns per tile
    static constexpr int GM = MOE_GEMM_BAND_ROWS / BM;   // row tiles per band
    static constexpr int SMEM = STAGES * STAGE_ELEMS;    // elements
};

// 16-byte chunk c of LDS row `row` lives at chunk c ^ ((row / rp) % cpr): measured free of bank
// conflicts for the 32-row x 2-chunk fragment reads of the 32x32x16 MFMA.
__device__ __forceinline__ int swz_chunk(int row, int c, int rp, int cpr) { return c ^ ((row / rp) % cpr); }

// Logical tile L (0 <= L < m_real * n_tiles) -> (row tile, column panel): bands of GM row tiles,
// row tiles fastest inside a band, so the tiles an XCD runs together share A tiles and panels.
__device__ __forceinline__ void decode_tile(int L, int gm, int m_real, int n_tiles, int& m_t, int& n_t) {
    const int band_tiles = gm * n_tiles;
    const int band = L / band_tiles;
    const int in_band = L - band * band_tiles;
    const int gm_b = min(gm, m_real - band * gm);
    n_t = in_band / gm_b;
    m_t = band * gm + (in_band - n_t * gm_b);
}

// Element type of A and the weights: bf16 bits, or OCP E4M3 codes in the fp8 form.
template <bool FP8>
using Elem = std::conditional_t<FP8, uint8_t, uint16_t>;
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));  // a 32-byte fp8 MFMA operand

// 16 bytes from global memory as a global (not flat) load: a flat load is also counted by
// lgkmcnt, so waiting for it waits for LDS traffic too
__device__ __forceinline__ bf16x8 gload_bf16x8(const uint16_t* p) {
    return *(const __attribute__((address_space(1))) bf16x8*)(p);
}

// fp8 form: dequantisation scales of the activation rows ([rows of A]) and of the weight rows
// ([E, N], one per output channel, for w0 and w1)
struct Fp8Scales {
    const float* a;
    const float* w0;
    const float* w1;
};

// LORA: 0 no LoRA epilogue (gate/up, or with GATE_UP false the down projection); 1 one adapter (every
// folded row is adapter 0; down: only at rank == BK, folded from LDS); 2 any adapters (the rows of one
// fragment may belong to different adapters: one pass per adapter present; down: any rank).  The
// one-adapter form is the common case and keeps the lean epilogue, which the loop of the general
// form would cost registers in the main loop.
template <bool GATE_UP, int BM, int BK, int STAGES, int NW, int LORA = 0, bool FP8 = false>
__global__ __launch_bounds__(64 * NW, 1) void gemm_bf16_kernel(const Elem<FP8>* __restrict__ A,
                                                          const Elem<FP8>* __restrict__ W0,
                                                          const Elem<FP8>* __restrict__ W1,
                                                          uint16_t* __restrict__ C,
                                                          const int32_t* __restrict__ sorted_ids,
                                                          const int32_t* __restrict__ offsets, int P, int top_k,
                                                          int E, int N, int K, int max_pad, int n_tiles,
                                                          float* __restrict__ sk_part, int32_t* __restrict__ sk_cnt,
                                                          int sk_on, int a_tok, GateUpLora lora, Fp8Scales f8) {
    static_assert(!(LORA && FP8), "no LoRA epilogue in the fp8 form");
    using TE = Elem<FP8>;
    constexpr int ES = sizeof(TE);
    using F = Cfg<GATE_UP, BM, BK, STAGES, NW, ES>;
    constexpr int NT = F::NT;
    constexpr int CE = F::CE;
    __shared__ __attribute__((aligned(1024))) TE smem[F::SMEM];
    __shared__ int s_scan[NW];
    __shared__ int s_lo[kMaxE], s_hi[kMaxE], s_tb[kMaxE + 1];  // expert span, first row tile
    __shared__ int s_row[2][BM];                                  // A source row per tile row
    __shared__ int s_rad[LORA ? 2 : 1][LORA ? BM : 1];            // LoRA: adapter id per tile row (-1: none)
    __shared__ float s_as[FP8 ? 2 : 1][FP8 ? BM : 1];             // fp8: dequantisation scale per tile row
    __shared__ int s_h[2];                                        // rows up to the last token
    __shared__ int s_arrived;                                     // split tile: the other side's count
    __shared__ int s_pf[STAGES == 2 ? BM : 1];                    // next segment's sorted ids
    __shared__ int s_nx[4];                                       // next segment: e, r0, r_end, n0

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: kept in a scalar register

    // ---- expert spans and their row tiles (once per workgroup)
    {
        int lo = 0, hi = 0;
        if (tid < E) {
            lo = min(max(offsets[tid], 0), max_pad);
            hi = min(max(offsets[tid + 1], lo), max_pad);
        }
        const int nt_e = (hi - lo + BM - 1) / BM;
        const int incl = block_inclusive_scan<NW>(nt_e, s_scan, (E + 63) / 64);
        if (tid < E) { s_lo[tid] = lo; s_hi[tid] = hi; s_tb[tid + 1] = incl; }
        if (tid == 0) { s_tb[0] = 0; s_h[0] = 0; s_h[1] = 0; }
        __syncthreads();
    }
    // values read from LDS are the same in every lane: readfirstlane keeps them (and everything
    // derived from them) in scalar registers
    const int m_real = __builtin_amdgcn_readfirstlane(s_tb[E]);

    // ---- this workgroup's work.  Workgroup ids go round-robin over the 8 XCDs; position
    // pos = xcd * per_xcd + slot orders the workgroups XCD by XCD.
    //  * whole tiles: XCD x takes the contiguous range [x*Tw/8, (x+1)*Tw/8) of the first Tw tiles
    //    and its workgroups stride through it, all at the same K step;
    //  * split tail (only with a workspace, and only when each XCD's share of the tail can be cut
    //    at least in two): Tw is the largest multiple of the grid, so every workgroup runs the
    //    same number of whole tiles, and the remaining T - Tw tiles (less than one round) are
    //    dealt XCD by XCD, n_x to XCD x, each cut along K into s_x pieces of at least
    //    MOE_GEMM_SPLIT_MIN_STAGES stages with s_x * n_x <= per_xcd.  Piece j of tail
    //    tile u runs on slot j * n_x + u of that XCD, so the pieces running together start at
    //    the same K step.  Every piece writes its fp32 partial accumulators to the workspace
    //    slot of its position and counts itself on the tile's counter; the last to arrive sums
    //    the s_x partials in piece order and stores the tile.  Nobody waits for anybody.
    const long long T = static_cast<long long>(m_real) * n_tiles;
    const int nk = (K + BK - 1) / BK;
    const int per_xcd = gridDim.x >> 3;
    const int xcd = blockIdx.x & 7;
    const int slot = blockIdx.x >> 3;
    const int pos = xcd * per_xcd + slot;
    long long Tw = T;
    if (sk_on) {
        // split only when every XCD's share of the tail is cut at least in two; otherwise whole
        // tiles throughout, as without a workspace
        const long long rounds = T / gridDim.x;
        const int rest = static_cast<int>(T - rounds * gridDim.x);
        if (rest > 0 && min(per_xcd / ((rest + 7) / 8), nk / MOE_GEMM_SPLIT_MIN_STAGES) >= 2)
            Tw = rounds * gridDim.x;
    }
    const int tail = static_cast<int>(T - Tw);
    const int l_hi = static_cast<int>(Tw * (xcd + 1) / 8);
    int L = static_cast<int>(Tw * xcd / 8) + slot;
    // this workgroup's tail piece (none: tail_L < 0)
    int tail_L = -1, tail_kb = 0, tail_ke = nk, tail_s = 1, tail_first = 0, tail_n = 1;
    if (tail > 0) {
        const int a_x = tail * xcd / 8;
        const int n_x = tail * (xcd + 1) / 8 - a_x;
        if (n_x > 0) {
            const int s_x = max(1, min(per_xcd / n_x, nk / MOE_GEMM_SPLIT_MIN_STAGES));
            if (slot < s_x * n_x) {
                const int u = slot % n_x, j = slot / n_x;
                tail_L = static_cast<int>(Tw) + a_x + u;
                tail_kb = j * nk / s_x;
                tail_ke = (j + 1) * nk / s_x;
                tail_s = s_x;
                tail_first = xcd * per_xcd + u;  // position of piece 0; piece j' at + j' * n_x
                tail_n = n_x;
            }
        }
    }
    int kb = 0, ke = nk;  // current segment: tile L, stages [kb, ke)
    if (slot >= per_xcd || L >= l_hi) {
        if (tail_L < 0) return;
        L = tail_L; kb = tail_kb; ke = tail_ke;
    }

    // tile L -> expert e, first sorted row r0, rows end r_end, first output column n0
    auto locate = [&](int Lt, int& e, int& r0, int& r_end, int& n0) __attribute__((always_inline)) {
        int m_t, n_t;
        decode_tile(Lt, F::GM, m_real, n_tiles, m_t, n_t);
        int a = 0, b = E - 1;  // largest expert whose first row tile is <= m_t
        while (a < b) {
            const int mid = (a + b + 1) >> 1;
            if (s_tb[mid] <= m_t) a = mid; else b = mid - 1;
        }
        e = __builtin_amdgcn_readfirstlane(a);
        r0 = __builtin_amdgcn_readfirstlane(s_lo[e] + (m_t - s_tb[e]) * BM);
        r_end = __builtin_amdgcn_readfirstlane(min(r0 + BM, s_hi[e]));
        n0 = __builtin_amdgcn_readfirstlane(n_t * F::NCOL);
    };
    // A source rows of a tile into s_row[buf] (rows without a token: -1) and s_h[buf]
    auto load_rows = [&](int buf, int r0, int r_end) __attribute__((always_inline)) {
        for (int i = tid; i < BM; i += NT) {
            const int r = r0 + i;
            int src = -1, tok = -1;
            if (r < r_end) {
                const int p = sorted_ids[r];
                if (p >= 0 && p < P) {
                    tok = p / top_k;
                    src = (GATE_UP || a_tok) ? tok : r;
                }
            }
            s_row[buf][i] = src;
            if constexpr (FP8) s_as[buf][i] = src >= 0 ? f8.a[src] : 0.f;
            if constexpr (LORA) {
                // the token's adapter (atlas: a mixed batch's adapter comes from the per-row map); 0
                // without a map; -1 for rows without a token or with an id outside [0, n_ad)
                int a = tok >= 0 ? (lora.row_adapter ? lora.row_adapter[tok] : 0) : -1;
                s_rad[buf][i] = (a >= 0 && a < lora.n_ad) ? a : -1;
            }
            if (src >= 0) atomicMax(&s_h[buf], i + 1);
        }
    };

    int e, r0, r_end, n0;
    locate(L, e, r0, r_end, n0);
    int buf = 0;
    load_rows(buf, r0, r_end);
    __syncthreads();

    // ---- per-lane DMA sources.  Instruction q of a wave's row block fills ROWS_PER_INST rows.
    // With MOE_GEMM_ASYM (8 waves, 2 stages) waves 0-3, one per SIMD, issue the loads of their own
    // row block and of wave w+4's, and waves 4-7 issue none: while an issuing wave stalls on the
    // address unit, the other wave of its SIMD issues MFMAs.  To hold twice the sources in the
    // same registers, those are byte offsets from scalar bases (A, and the tile's expert
    // matrices) and each load is a saddr-form instruction; otherwise they are 64-bit pointers.
    constexpr bool ASYM = MOE_GEMM_ASYM != 0 && NW == 8 && STAGES == 2;
    constexpr int NBLK = ASYM ? 2 : 1;  // row blocks issued per issuing wave
    const bool issuer = !ASYM || wave < NW / 2;
    const int lrow = lane / F::CPR;   // row within the instruction's block
    const int pc = lane % F::CPR;     // physical chunk this lane's 16 bytes land in
    using Src = std::conditional_t<ASYM, uint32_t, const TE*>;
    Src a_o[NBLK][F::A_INST], b_o[NBLK][F::B_INST];
    const TE* b_base0 = W0;     // the tile's expert matrices (uniform)
    const TE* b_base1 = W1;
    auto block_wave = [&](int j) __attribute__((always_inline)) { return wave + j * (NW / 2); };
    auto set_sources = [&](int bf, int e_, int r0_, int n0_) __attribute__((always_inline)) {
        b_base0 = W0 + static_cast<size_t>(e_) * N * K;
        b_base1 = GATE_UP ? W1 + static_cast<size_t>(e_) * N * K : b_base0;
        if (!issuer) return;
#pragma unroll
        for (int j = 0; j < NBLK; ++j) {
            const int bw = block_wave(j);
#pragma unroll
            for (int q = 0; q < F::A_INST; ++q) {
                const int row = (bw * F::A_INST + q) * F::ROWS_PER_INST + lrow;
                const int kc = swz_chunk(row, pc, F::RP, F::CPR);
                const int src = s_row[bf][row];
                // a row without a token reads a row that is always in bounds (token 0, or the
                // tile's first sorted row r0 < max_pad); its results are never stored
                const int srow = src >= 0 ? src : ((GATE_UP || a_tok) ? 0 : r0_);
                if constexpr (ASYM) a_o[j][q] = (static_cast<uint32_t>(srow) * K + kc * CE) * ES;
                else a_o[j][q] = A + static_cast<size_t>(srow) * K + kc * CE;
            }
#pragma unroll
            for (int q = 0; q < F::B_INST; ++q) {
                const int row = (bw * F::B_INST + q) * F::ROWS_PER_INST + lrow;
                const int kc = swz_chunk(row, pc, F::RP, F::CPR);
                int n = GATE_UP ? n0_ + (row & (BP / 2 - 1)) : n0_ + row;
                n = min(n, N - 1);  // columns past N are computed from a valid row and never stored
                if constexpr (ASYM) {
                    b_o[j][q] = (static_cast<uint32_t>(n) * K + kc * CE) * ES;
                } else {
                    const TE* bb = (GATE_UP && row >= BP / 2) ? b_base1 : b_base0;
                    b_o[j][q] = bb + static_cast<size_t>(n) * K + kc * CE;
                }
            }
        }
    };
    set_sources(buf, e, r0, n0);

    int nseg = ke - kb;  // stages of the current segment
    int sb = 0;  // running stage count: stage t of the current segment lives in LDS buffer (sb + t) % STAGES
    auto stage_ptr = [&](int t) __attribute__((always_inline)) { return smem + ((sb + t) % STAGES) * F::STAGE_ELEMS; };
    // LDS byte addresses of the A and B parts of stage buffer 0 (scalar)
    const uint32_t lds_a0 = lds_u32(smem);
    const uint32_t lds_b0 = lds_a0 + F::A_ELEMS * ES;
    // loads of segment stage t (K stage kbase + t) into its LDS buffer.  The stage's 16-byte
    // chunk of each lane is k0 + kc*8 with kc = swz_chunk(row, pc); only the stage that runs past
    // K (uniform test) recomputes kc to load zeros for k >= K.
    // (forced inline: the loads take scalar operands, which an outlined call would not keep)
    auto issue_at = [&](int t, int kbase, int parts = 3) __attribute__((always_inline)) {  // 1: A rows, 2: B rows
        if (!issuer) return;
        const int k0 = (kbase + t) * BK;
        const uint32_t sbuf = static_cast<uint32_t>((sb + t) % STAGES) * (F::STAGE_ELEMS * ES);
        // B instruction q of block j: its 8 rows lie on one side of the gate/up boundary
        auto b_base = [&](int bw, int q) __attribute__((always_inline)) {
            const int row0 = (bw * F::B_INST + q) * F::ROWS_PER_INST;
            return uniform_ptr((GATE_UP && row0 >= BP / 2) ? b_base1 : b_base0);
        };
        if (k0 + BK <= K) {
#pragma unroll
            for (int j = 0; j < NBLK; ++j) {
                const int bw = block_wave(j);
#pragma unroll
                for (int q = 0; q < F::A_INST; ++q) {
                    if (!(parts & 1)) break;
                    const uint32_t dst = lds_a0 + sbuf + (bw * F::A_INST + q) * 1024;
                    if constexpr (ASYM) dma16_s(A + k0, a_o[j][q], dst);
                    else dma16(a_o[j][q] + k0, dst);
                }
#pragma unroll
                for (int q = 0; q < F::B_INST; ++q) {
                    if (!(parts & 2)) break;
                    const uint32_t dst = lds_b0 + sbuf + (bw * F::B_INST + q) * 1024;
                    if constexpr (ASYM) dma16_s(b_base(bw, q) + k0, b_o[j][q], dst);
                    else dma16(b_o[j][q] + k0, dst);
                }
            }
        } else {
            // the stage that runs past K: chunks at k >= K load zeros
#pragma unroll
            for (int j = 0; j < NBLK; ++j) {
                const int bw = block_wave(j);
#pragma unroll
                for (int q = 0; q < F::A_INST; ++q) {
                    if (!(parts & 1)) break;
                    const uint32_t dst = lds_a0 + sbuf + (bw * F::A_INST + q) * 1024;
                    const int row = (bw * F::A_INST + q) * F::ROWS_PER_INST + lrow;
                    const void* src;
                    if constexpr (ASYM) src = reinterpret_cast<const char*>(A + k0) + a_o[j][q];
                    else src = a_o[j][q] + k0;
                    const bool in = k0 + swz_chunk(row, pc, F::RP, F::CPR) * CE < K;
                    dma16(in ? src : static_cast<const void*>(kZero16), dst);
                }
#pragma unroll
                for (int q = 0; q < F::B_INST; ++q) {
                    if (!(parts & 2)) break;
                    const uint32_t dst = lds_b0 + sbuf + (bw * F::B_INST + q) * 1024;
                    const int row = (bw * F::B_INST + q) * F::ROWS_PER_INST + lrow;
                    const void* src;
                    if constexpr (ASYM) src = reinterpret_cast<const char*>(b_base(bw, q) + k0) + b_o[j][q];
                    else src = b_o[j][q] + k0;
                    const bool in = k0 + swz_chunk(row, pc, F::RP, F::CPR) * CE < K;
                    dma16(in ? src : static_cast<const void*>(kZero16), dst);
                }
            }
        }
    };
    // MFMA k-steps per stage: 32x32x16 bf16 (16 k), or 32x32x64 fp8 (64 k)
    constexpr int KK = FP8 ? BK / 64 : BK / 16;
    // With the asymmetric issue and A_LATE_K > 0, a stage's weight-panel loads (the long ones,
    // from HBM) go out right after the barrier and its activation-row loads (mostly L2 hits) at
    // k-step A_LATE_K, which halves the burst of loads landing in LDS meanwhile.
    constexpr int A_LATE_K = FP8 ? MOE_FP8_A_LATE : MOE_GEMM_A_LATE;
    constexpr bool A_LATE = ASYM && A_LATE_K > 0 && A_LATE_K < KK;
    auto issue = [&](int t) __attribute__((always_inline)) { issue_at(t, kb, A_LATE ? 2 : 3); };

    const int wm = wave >> 1, wn = wave & 1;  // wave grid WAVES_M x 2
    // 32x32x16 MFMA blocks: each wave holds FI x 4 blocks of 32x32 fp32 accumulators
    f32x16 acc[F::FI][4];

    // fragment LDS offsets (elements) within a stage: lane row fr = lane%32, k-chunk fc = lane/32
    const int fr = lane & 31, fc = lane >> 5;
    int a_off[F::FI], b_off[4];
#pragma unroll
    for (int i = 0; i < F::FI; ++i) a_off[i] = (wm * F::WM + i * 32 + fr) * BK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        int prow;
        if (GATE_UP) prow = (j < 2 ? wn * 64 + j * 32 : BP / 2 + wn * 64 + (j - 2) * 32);
        else prow = wn * 128 + j * 32;
        b_off[j] = F::A_ELEMS + (prow + fr) * BK;
    }
    // every fragment starts on a multiple of 32 rows, so its swizzle depends on the lane only
    const int fswz = (fr / F::RP) % F::CPR;

    using Frag = std::conditional_t<FP8, i32x8, bf16x8>;
    // Fragment register sets: two (the next k-step's fragments are read while the current one's
    // MFMAs run), or one for the 8-wave fp8 form, whose 32-byte fragments would not fit twice
    // beside 128 accumulators in 256 registers; there the other wave of the SIMD covers the reads.
    constexpr int NSET = (FP8 && NW == 8) ? 1 : 2;
    Frag fa[NSET][F::FI], fb[NSET][4];
    // fragments of k-step kk of stage s into register set `set` (the first NF A fragments)
    auto read = [&](auto nf_c, int s, int kk, int set) __attribute__((always_inline)) {
        constexpr int NF = decltype(nf_c)::value;
        if constexpr (NF > 0) {
            const TE* st = stage_ptr(s);
            if constexpr (FP8) {
                // a 32-byte operand: logical chunks c0 and c0 + 1 of the row (A and B take the
                // same lane -> k map, so every product pairs the same k)
                const int c0 = kk * 4 + fc * 2;
                const int x0 = (c0 ^ fswz) * CE, x1 = ((c0 + 1) ^ fswz) * CE;
                auto frag = [&](int off) __attribute__((always_inline)) {
                    const u32x4 lo = *reinterpret_cast<const u32x4*>(st + off + x0);
                    const u32x4 hi = *reinterpret_cast<const u32x4*>(st + off + x1);
                    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                };
#pragma unroll
                for (int i = 0; i < NF; ++i) fa[set][i] = frag(a_off[i]);
#pragma unroll
                for (int j = 0; j < 4; ++j) fb[set][j] = frag(b_off[j]);
            } else {
                const int cx = ((kk * 2 + fc) ^ fswz) << 3;
#pragma unroll
                for (int i = 0; i < NF; ++i) fa[set][i] = *reinterpret_cast<const bf16x8*>(st + a_off[i] + cx);
#pragma unroll
                for (int j = 0; j < 4; ++j) fb[set][j] = *reinterpret_cast<const bf16x8*>(st + b_off[j] + cx);
            }
        }
    };
    auto mfma = [&](auto nf_c, int set) __attribute__((always_inline)) {
        constexpr int NF = decltype(nf_c)::value;
#pragma unroll
        for (int i = 0; i < NF; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if constexpr (FP8)  // E4M3 operands (format 0), unit block scales (127 = 2^0)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[set][i], fb[set][j], acc[i][j],
                                                                               0, 0, 0, 127, 0, 127);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[set][i], fb[set][j], acc[i][j], 0, 0, 0);
    };
    // The next segment's rows, prepared inside this segment's main loop (pf: 2 stages, at least 3
    // stages in the segment (4 with LoRA), a next segment exists): after the barrier of stage
    // 0 the waves of threads tid < BM locate it and load its sorted ids into LDS; after the
    // barrier of stage 1 (whose vmcnt(0) covered those loads) they write its rows to LDS buffer
    // buf ^ 1 (free: the previous segment's epilogue, its last reader, is behind both barriers),
    // with the fp8 activation scales or the LoRA adapter ids of those rows.  Later stage
    // barriers order those writes before the issuing waves read them for the next segment's
    // sources at this segment's end.  So the segment end no longer waits for the expert search,
    // a barrier and the sorted-id loads.
    constexpr bool PF = STAGES == 2 && BM <= NT && BM % 64 == 0;
    int L_next = 0, kb2 = 0, ke2 = nk, e2 = 0, r02 = 0, r_end2 = 0, n02 = 0;
    bool more = false, pf = false;
    // Stage t becomes readable: this thread's loads of t have landed (at most `ahead` later stages
    // still in flight), its own LDS reads of earlier stages are done, and after the barrier every
    // wave is past stage t-1, whose buffer is refilled with stage t+STAGES-1.
    auto ready = [&](int t) __attribute__((always_inline)) {
        const int ahead = min(STAGES - 2, nseg - 1 - t);
        if constexpr (STAGES >= 4) {
            if (ahead >= 2) wait_vmcnt<2 * F::LOADS>();
            else if (ahead == 1) wait_vmcnt<F::LOADS>();
            else wait_vmcnt<0>();
        } else if constexpr (STAGES == 3) {
            if (ahead >= 1) wait_vmcnt<F::LOADS>();
            else wait_vmcnt<0>();
        } else {
            wait_vmcnt<0>();
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        if (t + STAGES - 1 < nseg) issue(t + STAGES - 1);
    };
    // after the barrier of stage 0: locate the next segment, load its sorted ids
    auto pf_load = [&]() __attribute__((always_inline)) {
        if constexpr (PF) {
            // only the waves that hold its rows (with the asymmetric issue, the issuing waves,
            // which have slack in the main loop); wave 0 hands the result to the others in LDS
            if (pf && wave < BM / 64) {
                locate(L_next, e2, r02, r_end2, n02);
                if (tid == 0) {
                    s_h[buf ^ 1] = 0;
                    s_nx[0] = e2; s_nx[1] = r02; s_nx[2] = r_end2; s_nx[3] = n02;
                }
                // straight into LDS, untracked by the compiler: a tracked load here would be
                // waited for (vmcnt(0), draining the stage loads) where the loop variants join;
                // rows past the segment read its first row, never used
                dma4(sorted_ids + (r02 + tid < r_end2 ? r02 + tid : r02), lds_u32(s_pf) + wave * 256);
            }
        }
    };
    // after the barrier of stage 1: its rows into LDS
    auto pf_rows = [&]() __attribute__((always_inline)) {
        if constexpr (PF) {
            if (pf && tid < BM) {
                const int p = r02 + tid < r_end2 ? s_pf[tid] : -1;
                const int tok = (p >= 0 && p < P) ? p / top_k : -1;
                const int src = tok >= 0 ? ((GATE_UP || a_tok) ? tok : r02 + tid) : -1;
                s_row[buf ^ 1][tid] = src;
                if (src >= 0) atomicMax(&s_h[buf ^ 1], tid + 1);
                // fp8: the rows' activation scales, straight into LDS as well (a row without a
                // token takes row 0's, never used); the later stage waits cover the loads
                if constexpr (FP8) dma4(f8.a + (src >= 0 ? src : 0), lds_u32(s_as[buf ^ 1]) + wave * 256);
                // LoRA: the tokens' adapter ids, raw, straight into LDS (checked after the next
                // barrier, below); without a map every row with a token is adapter 0
                if constexpr (LORA) {
                    if (lora.row_adapter != nullptr)
                        dma4(lora.row_adapter + (tok >= 0 ? tok : 0), lds_u32(s_rad[buf ^ 1]) + wave * 256);
                    else
                        s_rad[buf ^ 1][tid] = src >= 0 ? 0 : -1;
                }
            }
        }
    };
    // LoRA, after the barrier of stage 2 (whose vmcnt(0) covered the id loads): -1 for rows without
    // a token and for ids outside [0, n_ad), as load_rows does
    auto pf_fix = [&]() __attribute__((always_inline)) {
        if constexpr (PF && LORA) {
            if (pf && tid < BM && lora.row_adapter != nullptr) {
                const int a = s_rad[buf ^ 1][tid];
                s_rad[buf ^ 1][tid] = (s_row[buf ^ 1][tid] >= 0 && a >= 0 && a < lora.n_ad) ? a : -1;
            }
        }
    };
    // Each k-step's MFMAs are issued after the next k-step's fragment reads (and, at a stage
    // boundary, after the barrier), so queued MFMAs cover both LDS latency and barrier waits.
    // NF = A fragments of this wave that hold tokens; every wave still loads and meets the barriers.
    auto main_loop = [&](auto nf_c) __attribute__((always_inline)) {
        if constexpr (NSET == 2) {
            ready(0);
            pf_load();
            read(nf_c, 0, 0, 0);
            for (int s = 0; s < nseg; ++s) {
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    if (A_LATE && kk == A_LATE_K && s + 1 < nseg) issue_at(s + 1, kb, 1);
                    if (kk + 1 < KK) {
                        read(nf_c, s, kk + 1, (kk + 1) & 1);
                    } else if (s + 1 < nseg) {
                        ready(s + 1);
                        if (s == 0) pf_rows();
                        else if (s == 1) pf_fix();
                        read(nf_c, s + 1, 0, 0);
                    }
                    mfma(nf_c, kk & 1);
                }
            }
        } else {
            // one set: each k-step's reads, then its MFMAs; the stage barrier opens each stage
            for (int s = 0; s < nseg; ++s) {
                ready(s);
                if (s == 0) pf_load();
                else if (s == 1) pf_rows();
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    if (A_LATE && kk == A_LATE_K && s + 1 < nseg) issue_at(s + 1, kb, 1);
                    read(nf_c, s, kk, 0);
                    mfma(nf_c, 0);
                }
            }
        }
    };
    static_assert(F::FI == 2, "tail skipping assumes two A fragments per wave");

    // The first segment issues its first STAGES-1 stages here; later segments find stage 0
    // already in flight (issued by the previous segment before its epilogue) and issue stages
    // 1..STAGES-2.
    for (int t = 0; t < STAGES - 1; ++t)
        if (t < nseg) issue_at(t, kb);

    while (true) {
        // the next segment: this XCD's next whole tile, else this workgroup's tail piece
        L_next = L + per_xcd; kb2 = 0; ke2 = nk;
        more = L != tail_L && L_next < l_hi;
        if (!more && L != tail_L && tail_L >= 0) {
            more = true;
            L_next = tail_L; kb2 = tail_kb; ke2 = tail_ke;
        }
        pf = PF && more && nseg >= (LORA ? 4 : 3);
        // rows up to the last token of this tile (an expert's sentinels follow its tokens): a wave
        // whose 32-row fragments all lie past it skips their MFMAs
        const int h_rows = s_h[buf];
#pragma unroll
        for (int i = 0; i < F::FI; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
        const int nf = __builtin_amdgcn_readfirstlane(min(max((h_rows - wm * F::WM + 31) / 32, 0), F::FI));
        if (nf == 2) main_loop(std::integral_constant<int, 2>{});
        else if (nf == 1) main_loop(std::integral_constant<int, 1>{});
        else main_loop(std::integral_constant<int, 0>{});

        // ---- a piece of a split tail tile: partial accumulators through the workspace.
        // Partials are written and read with device-coherent (sc1) buffer accesses, the same
        // accesses agent-scope atomic loads and stores use: a store is visible device-wide once
        // it has completed (vmcnt), and such a load sees it, so no fence has to write back or
        // invalidate the whole L2 (which would cost every other workgroup on the XCD its cached
        // A tiles and weight panels).
        constexpr int PART = F::NT * F::FI * 4 * 16;  // floats per partial
        constexpr int kSc1 = 16;                      // cache policy: device scope
        const bool split = L == tail_L && tail_s > 1;
        bool store = true;
        int np = 0;  // partials that make up the tile (the last piece of a split tile only)
        const __amdgpu_buffer_rsrc_t part = __builtin_amdgcn_make_buffer_rsrc(
            sk_part, 0, static_cast<int>(gridDim.x) * PART * 4, 0x00020000);
        uint32_t off = 0;  // byte offset of this thread's first 16 bytes in partial 0 to add
        if (split) {
            // layout [16-byte chunk c][thread]: every store and load instruction is coalesced
            uint32_t o = (static_cast<uint32_t>(pos) * PART + tid * 4) * 4;
#pragma unroll
            for (int i = 0; i < F::FI; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x4 v{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                      acc[i][j][4 * q + 3]};
                        __builtin_amdgcn_raw_buffer_store_b128(v, part, o, 0, kSc1);
                        o += F::NT * 16;
                    }
            wait_vmcnt<0>();  // this piece's partial is complete, hence visible, before it is counted
            __syncthreads();
            if (tid == 0)
                s_arrived = __hip_atomic_fetch_add(&sk_cnt[L - static_cast<int>(Tw)], 1, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            store = s_arrived == tail_s - 1;
            if (store) {
                off = (static_cast<uint32_t>(tail_first) * PART + tid * 4) * 4;
                np = tail_s;
                if (tid == 0)
                    __hip_atomic_store(&sk_cnt[L - static_cast<int>(Tw)], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        // only the last piece of a split tile (np > 0): the tile is the sum of every piece's partial
        // (its own included, from the workspace), in piece order, not its own accumulators
        if (np > 0) {
            const uint32_t pstride = static_cast<uint32_t>(tail_n) * PART * 4;
#pragma unroll
            for (int i = 0; i < F::FI; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        f32x4 t = {0.f, 0.f, 0.f, 0.f};
                        uint32_t o = off;
                        for (int jp = 0; jp < np; ++jp) {
                            t += __builtin_amdgcn_raw_buffer_load_b128(part, o, 0, kSc1);
                            o += pstride;
                        }
#pragma unroll
                        for (int v = 0; v < 4; ++v) acc[i][j][4 * q + v] = t[v];
                        off += F::NT * 16;
                    }
        }

        // ---- next segment: its rows (unless prepared in the main loop), sources and first stage,
        // before this segment's epilogue
        if (more) {
            if (pf && wave >= BM / 64) {  // located by wave 0 in the main loop
                e2 = __builtin_amdgcn_readfirstlane(s_nx[0]);
                r02 = __builtin_amdgcn_readfirstlane(s_nx[1]);
                r_end2 = __builtin_amdgcn_readfirstlane(s_nx[2]);
                n02 = __builtin_amdgcn_readfirstlane(s_nx[3]);
            }
            if (!pf) {
                locate(L_next, e2, r02, r_end2, n02);
                if (tid == 0) s_h[buf ^ 1] = 0;
                __syncthreads();  // every wave is past this segment's last stage reads and s_h is reset
                load_rows(buf ^ 1, r02, r_end2);
                __syncthreads();
            }
            set_sources(buf ^ 1, e2, r02, n02);
            // stage 0 of the next segment goes to buffer (sb + nseg) % STAGES, which held stage
            // nseg-STAGES+1 .. of this segment at the latest and is no longer read by any wave
            sb += nseg;
            issue_at(0, kb2);
            sb -= nseg;
        }

        // ---- LoRA epilogue (the page's order: the bf16 GEMM output, folded, then for gate/up SiLU * up):
        // every accumulator becomes a bf16 value, bf16(bf16(acc) + scale * bf16(xa . B_e^T)) where
        // the row is folded.  Gate/up: pass pj = 0 folds the gate blocks 0, 1 with the gate tables and
        // pj = 1 the up blocks 2, 3 with the up tables, over the same output columns.  Down (the
        // down-projection fold of the expert outputs): the host passes the one set of tables in both
        // slots, and pass pj folds blocks 2 pj, 2 pj + 1, the wave's columns 64 pj .. 64 pj + 63.  The bf16 values are held two to a register while the deltas are formed,
        // which leaves the registers for a projection's whole delta: its four 32x32 blocks as 32x32x16
        // MFMAs over the rank, fed by xa and B_e fragments read straight from memory, up to 64 of the
        // rank at a time.  A chunk's fragment loads are all issued before its MFMAs (the scheduling
        // barrier keeps the compiler from sinking each load to its MFMA), so a projection waits for
        // one or two memory latencies rather than one per MFMA.
        if constexpr (LORA) {
            if (store) {
                auto bf16r = [](float x) __attribute__((always_inline)) {
                    return __uint_as_float(static_cast<uint32_t>(f32_to_bf16(x)) << 16);
                };
                auto lo16 = [](uint32_t w) __attribute__((always_inline)) { return __uint_as_float(w << 16); };
                auto hi16 = [](uint32_t w) __attribute__((always_inline)) { return __uint_as_float(w & 0xffff0000u); };
                // values 2h and 2h+1 of block [i][j]: the same rounding as bf16r
                uint32_t pk[F::FI][4][8];
#pragma unroll
                for (int i = 0; i < F::FI; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int h = 0; h < 8; ++h) pk[i][j][h] = pack_bf16x2(acc[i][j][2 * h], acc[i][j][2 * h + 1]);
                // adapter id of the row of value v of fragment i (-1: not folded)
                auto row_ad = [&](int i, int v) __attribute__((always_inline)) {
                    return s_rad[buf][wm * F::WM + i * 32 + (v >> 2) * 8 + fc * 4 + (v & 3)];
                };
                // the adapters present among the wave's rows, smallest first: one pass each
                auto next_ad = [&](int after) __attribute__((always_inline)) {
                    int m = 0x7fffffff;
                    for (int i = 0; i < F::FI; ++i)
                        for (int v = 0; v < 16; ++v) {
                            const int a = row_ad(i, v);
                            if (a > after && a < m) m = a;
                        }
#pragma unroll
                    for (int o = 32; o >= 1; o >>= 1) m = min(m, __shfl_xor(m, o));
                    return m;
                };
                // adapter `cur`'s B_e and scale_e of projection pj (Be = nullptr: e not adapted by it)
                auto table = [&](int pj, int cur, const uint16_t*& Be, float& sc) __attribute__((always_inline)) {
                    Be = nullptr;
                    sc = 0.f;
                    if (e >= lora.n_tab[pj]) return;
                    const int64_t tix = static_cast<int64_t>(cur) * lora.n_tab[pj] + e;
                    if (lora.a_tab[pj][tix] == 0 || lora.b_tab[pj][tix] == 0) return;
                    Be = reinterpret_cast<const uint16_t*>(lora.b_tab[pj][tix]);
                    sc = lora.s_tab[pj][tix];
                };
                // one adapter: its tables for both projections, looked up once per tile
                const uint16_t* ad0_b[2] = {nullptr, nullptr};
                float ad0_s[2] = {0.f, 0.f};
                if constexpr (LORA == 1) {
                    table(0, 0, ad0_b[0], ad0_s[0]);
                    table(1, 0, ad0_b[1], ad0_s[1]);
                }
                // Down, one adapter (the host launches this form only with rank == BK): the delta is one
                // more K stage of the tile, with the xa rows as A and the B_e rows of the panel as the
                // weight panel.  The last stage's LDS buffer is free once every wave is past its reads
                // (the next tile's first stage went to another buffer), so the whole workgroup loads
                // that stage straight into it, in the main loop's layout and swizzle, and each wave's
                // delta blocks then run from LDS with the main loop's fragment reads: one memory round
                // trip per tile instead of one per column half and rank chunk, and no register form
                // beside it, whose pressure spilled into the main loop.  Uniform over the workgroup:
                // e and the tables are.
                if constexpr (LORA == 1 && !GATE_UP && !FP8) {
                    if (ad0_b[0] != nullptr) {
                        const int lb = (sb + nseg - 1) % STAGES;  // the last stage's buffer
                        const uint32_t lds_st = lds_u32(smem) + static_cast<uint32_t>(lb) * (F::STAGE_ELEMS * ES);
                        __syncthreads();  // every wave is past its reads of the last stage
                        constexpr int INSTS = (BM + BP) / F::ROWS_PER_INST;  // 1 KB loads for the stage
                        const uint16_t* Be = ad0_b[0];
                        for (int g = wave; g < INSTS; g += NW) {
                            const int row = g * F::ROWS_PER_INST + lrow;
                            const int kc = swz_chunk(row, pc, F::RP, F::CPR);
                            // rows past the span or past N read a row in bounds; never stored
                            const uint16_t* src =
                                row < BM ? lora.xa[0] + static_cast<size_t>(min(r0 + row, max_pad - 1)) * BK + kc * CE
                                         : Be + static_cast<size_t>(min(n0 + row - BM, N - 1)) * BK + kc * CE;
                            dma16(src, lds_st + g * 1024);
                        }
                        wait_vmcnt<0>();
                        __syncthreads();
                        const TE* st = smem + lb * F::STAGE_ELEMS;
                        const float sc = ad0_s[0];
                        // with a row map: bit i * 16 + v set when value v of fragment i is in a folded row
                        const bool has_map = lora.row_adapter != nullptr;
                        uint32_t fmask = 0;
                        if (has_map) {
#pragma unroll
                            for (int i = 0; i < F::FI; ++i)
#pragma unroll
                                for (int v = 0; v < 16; ++v) fmask |= (row_ad(i, v) == 0 ? 1u : 0u) << (i * 16 + v);
                        }
                        // k-step kk's fragments of column half pj into register set `set`
                        bf16x8 xf[2][F::FI], bw[2][2];
                        auto lread = [&](int pj, int kk, int set) __attribute__((always_inline)) {
                            const int cx = ((kk * 2 + fc) ^ fswz) << 3;
#pragma unroll
                            for (int i = 0; i < F::FI; ++i) xf[set][i] = *reinterpret_cast<const bf16x8*>(st + a_off[i] + cx);
#pragma unroll
                            for (int jj = 0; jj < 2; ++jj)
                                bw[set][jj] = *reinterpret_cast<const bf16x8*>(st + b_off[2 * pj + jj] + cx);
                        };
#pragma unroll
                        for (int pj = 0; pj < 2; ++pj) {  // the wave's column halves: blocks 2 pj, 2 pj + 1
                            f32x16 d[F::FI][2];
#pragma unroll
                            for (int i = 0; i < F::FI; ++i)
#pragma unroll
                                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                                    for (int v = 0; v < 16; ++v) d[i][jj][v] = 0.f;
                            // rank order, as the register form: every delta block sums k 0, 16, 32, 48;
                            // the next k-step's fragments are read while this one's MFMAs run
                            lread(pj, 0, 0);
#pragma unroll
                            for (int kk = 0; kk < KK; ++kk) {
                                if (kk + 1 < KK) lread(pj, kk + 1, (kk + 1) & 1);
#pragma unroll
                                for (int i = 0; i < F::FI; ++i)
#pragma unroll
                                    for (int jj = 0; jj < 2; ++jj)
                                        d[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf[kk & 1][i], bw[kk & 1][jj],
                                                                                          d[i][jj], 0, 0, 0);
                            }
                            // a pair of values (rows rl, rl + 1 of one column): the bf16 deltas in one
                            // conversion, the two folds, and the results rounded in one more; without a
                            // row map every row with a token is folded, and rows without one are never
                            // stored, so only a map needs the per-row choice
#pragma unroll
                            for (int i = 0; i < F::FI; ++i)
#pragma unroll
                                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                                    for (int h = 0; h < 8; ++h) {
                                        uint32_t& w = pk[i][pj * 2 + jj][h];
                                        const uint32_t dv = pack_bf16x2(d[i][jj][2 * h], d[i][jj][2 * h + 1]);
                                        uint32_t nw = pack_bf16x2(fmaf(sc, lo16(dv), lo16(w)), fmaf(sc, hi16(dv), hi16(w)));
                                        if (has_map) {
                                            const uint32_t keep = ((fmask >> (i * 16 + 2 * h)) & 1u ? 0u : 0xffffu) |
                                                                  ((fmask >> (i * 16 + 2 * h + 1)) & 1u ? 0u : 0xffff0000u);
                                            nw = (nw & ~keep) | (w & keep);
                                        }
                                        w = nw;
                                    }
                        }
                    }
                }
#pragma unroll
                for (int pj = 0; pj < 2; ++pj) {  // gate/up: 0 gate (blocks 0, 1), 1 up (blocks 2, 3); down: halves
                    if constexpr (LORA == 1 && !GATE_UP) break;  // folded from LDS above
                    if (e >= lora.n_tab[pj]) continue;  // past every adapter's table: not adapted
                    // this lane's xa rows (clamped: rows past the span are computed and never stored)
                    const uint16_t* xr[F::FI];
#pragma unroll
                    for (int i = 0; i < F::FI; ++i) {
                        const int rowf = min(r0 + wm * F::WM + i * 32 + fr, max_pad - 1);
                        xr[i] = lora.xa[pj] + static_cast<size_t>(rowf) * lora.rank + fc * 8;
                    }
                    // one pass per adapter: the delta of adapter `cur`, folded into its rows
                    auto pass = [&](int cur, const uint16_t* Be, float sc) __attribute__((always_inline)) {
                        if (Be == nullptr) return;
                        const uint16_t* br[2];
#pragma unroll
                        for (int jj = 0; jj < 2; ++jj) {
                            const int col = min(n0 + (GATE_UP ? wn * 64 : wn * 128 + pj * 64) + jj * 32 + fr, N - 1);
                            br[jj] = Be + static_cast<size_t>(col) * lora.rank + fc * 8;
                        }
                        f32x16 d[F::FI][2];
#pragma unroll
                        for (int i = 0; i < F::FI; ++i)
#pragma unroll
                            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                                for (int v = 0; v < 16; ++v) d[i][jj][v] = 0.f;
                        // NTK 16-deep steps of the rank from k0; each delta block sums in rank order
                        auto chunk = [&](int k0, auto ntk_c) __attribute__((always_inline)) {
                            constexpr int NTK = decltype(ntk_c)::value;
                            bf16x8 xf[F::FI][NTK], bw[2][NTK];
#pragma unroll
                            for (int t = 0; t < NTK; ++t) {
#pragma unroll
                                for (int i = 0; i < F::FI; ++i) xf[i][t] = gload_bf16x8(xr[i] + k0 + t * 16);
#pragma unroll
                                for (int jj = 0; jj < 2; ++jj) bw[jj][t] = gload_bf16x8(br[jj] + k0 + t * 16);
                            }
                            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                            for (int t = 0; t < NTK; ++t)
#pragma unroll
                                for (int i = 0; i < F::FI; ++i)
#pragma unroll
                                    for (int jj = 0; jj < 2; ++jj)
                                        d[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf[i][t], bw[jj][t], d[i][jj], 0, 0, 0);
                        };
                        for (int k0 = 0; k0 < lora.rank; k0 += 32) chunk(k0, std::integral_constant<int, 2>{});
#pragma unroll
                        for (int i = 0; i < F::FI; ++i)
#pragma unroll
                            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                                for (int h = 0; h < 8; ++h) {
                                    uint32_t& w = pk[i][pj * 2 + jj][h];
                                    float lo = lo16(w), hi = hi16(w);
                                    if (row_ad(i, 2 * h) == cur) lo = bf16r(fmaf(sc, bf16r(d[i][jj][2 * h]), lo));
                                    if (row_ad(i, 2 * h + 1) == cur) hi = bf16r(fmaf(sc, bf16r(d[i][jj][2 * h + 1]), hi));
                                    w = pack_bf16x2(lo, hi);  // exact: both are bf16 values
                                }
                    };
                    if constexpr (LORA == 1) {
                        pass(0, ad0_b[pj], ad0_s[pj]);
                    } else {
                        for (int cur = next_ad(-1); cur != 0x7fffffff; cur = next_ad(cur)) {
                            const uint16_t* Be;
                            float sc;
                            table(pj, cur, Be, sc);
                            pass(cur, Be, sc);
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < F::FI; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int h = 0; h < 8; ++h) {
                            acc[i][j][2 * h] = lo16(pk[i][j][h]);
                            acc[i][j][2 * h + 1] = hi16(pk[i][j][h]);
                        }
            }
        }

        // ---- epilogue straight from the accumulators: neighbour lanes (columns c, c+1) swap one
        // value so that each lane stores two adjacent bf16 columns of one row as 4 bytes
        const bool odd = (lane & 1) != 0;
        const int ccol = n0 + (fr & ~1);
        constexpr int NO = GATE_UP ? 2 : 4;  // output column blocks of this wave
        // fp8: the weight scales of this lane's accumulator column in each block (gate, up)
        float wsc[NO], wsu[NO];
        if constexpr (FP8) {
#pragma unroll
            for (int j = 0; j < NO; ++j) {
                const int cj = min(n0 + (GATE_UP ? wn * 64 : wn * 128) + j * 32 + fr, N - 1);
                wsc[j] = f8.w0[static_cast<size_t>(e) * N + cj];
                if constexpr (GATE_UP) wsu[j] = f8.w1[static_cast<size_t>(e) * N + cj];
            }
        }
        if (store)
#pragma unroll
        for (int i = 0; i < F::FI; ++i)
#pragma unroll
            for (int v = 0; v < 16; v += 2) {
                const int rl = wm * F::WM + i * 32 + (v >> 2) * 8 + fc * 4 + (v & 3);  // row of value v
                const int row_l = rl + (odd ? 1 : 0);
                const bool ok = s_row[buf][row_l] >= 0;
                uint16_t* crow = C + static_cast<size_t>(r0 + row_l) * N;
                float sa0 = 1.f, sa1 = 1.f;  // fp8: the rows' activation scales
                if constexpr (FP8) { sa0 = s_as[buf][rl]; sa1 = s_as[buf][rl + 1]; }
#pragma unroll
                for (int j = 0; j < NO; ++j) {
                    float h0, h1;  // values v (row rl) and v+1 (row rl+1) of this lane's column
                    float g0 = acc[i][j][v], g1 = acc[i][j][v + 1];
                    if constexpr (FP8) { g0 = g0 * sa0 * wsc[j]; g1 = g1 * sa1 * wsc[j]; }
                    if constexpr (GATE_UP) {
                        float u0 = acc[i][j + 2][v], u1 = acc[i][j + 2][v + 1];
                        if constexpr (FP8) { u0 = u0 * sa0 * wsu[j]; u1 = u1 * sa1 * wsu[j]; }
                        h0 = silu_mul(g0, u0);
                        h1 = silu_mul(g1, u1);
                    } else {
                        h0 = g0;
                        h1 = g1;
                    }
                    const float send = odd ? h0 : h1;
                    const float got = __int_as_float(__builtin_amdgcn_update_dpp(
                        0, __float_as_int(send), 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
                    const uint32_t pr = odd ? pack_bf16x2(got, h1) : pack_bf16x2(h0, got);
                    const int col = ccol + (GATE_UP ? wn * 64 + j * 32 : wn * 128 + j * 32);
                    if (ok && col < N) *reinterpret_cast<uint32_t*>(crow + col) = pr;
                }
            }
        if (!more) break;
        L = L_next;
        e = e2; r0 = r02; r_end = r_end2; n0 = n02;
        sb += nseg;
        kb = kb2; ke = ke2; nseg = ke - kb;
        buf ^= 1;
        for (int t = 1; t < STAGES - 1; ++t)
            if (t < nseg) issue_at(t, kb);
    }
}

int device_cus(hipError_t& err) {
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

constexpr int kMaxGrid = 1024;                          // persistent grid cap
constexpr int kSkMaxGrid = 256;                         // split-tail grid cap: partial slots in the workspace
constexpr int64_t kSkCounterBytes = 4096;               // one int32 counter per tail tile (< grid), padded
constexpr int64_t kSkPartBytes = 512LL * 2 * 64 * 4;    // largest partial: 512 threads x 128 fp32
constexpr int64_t kSkWorkspaceBytes = kSkCounterBytes + kSkMaxGrid * kSkPartBytes;
static_assert(kSkMaxGrid * 4 <= kSkCounterBytes, "split-tail counters overflow their area");

template <bool GATE_UP, int BM, int BK, int STAGES, int NW, int LORA = 0, bool FP8 = false>
hipError_t launch_cfg(const Elem<FP8>* a, const Elem<FP8>* w0, const Elem<FP8>* w1, uint16_t* c,
                      const int32_t* sorted_ids, const int32_t* offsets, int P, int top_k, int E, int N, int K,
                      int max_pad, void* ws, int64_t ws_bytes, int a_tok, hipStream_t s,
                      const GateUpLora& lora = GateUpLora{}, const Fp8Scales& f8 = Fp8Scales{}) {
    using F = Cfg<GATE_UP, BM, BK, STAGES, NW, sizeof(Elem<FP8>)>;
    static_assert(F::NT * F::FI * 64 * 4 <= kSkPartBytes, "partial accumulators larger than their workspace slot");
    const int n_tiles = (N + F::NCOL - 1) / F::NCOL;
    hipError_t err = hipSuccess;
    const int cus = device_cus(err);
    if (err != hipSuccess) return err;
    long long grid = cus / 8 * 8;
    if (grid < 8) grid = 8;
    // The split tail needs the persistent grid and a workspace of counters + one partial per
    // workgroup.
    const bool sk = ws != nullptr && ws_bytes >= kSkWorkspaceBytes;
    if (grid > (sk ? kSkMaxGrid : kMaxGrid)) grid = sk ? kSkMaxGrid : kMaxGrid;
    if (!sk) {
        // Persistent (one workgroup per compute unit) when there are more than 4 tiles per compute
        // unit at worst.  With fewer, one workgroup per tile lets the hardware dispatcher hand late
        // tiles to whichever compute unit frees up first, which balances better than a static
        // share when a few long tiles remain.
        const long long worst = static_cast<long long>((max_pad + BM - 1) / BM + E) * n_tiles;
        const long long worst8 = (worst + 7) / 8 * 8;
        if (worst8 <= 4 * grid) grid = worst8;
    }
    int32_t* cnt = sk ? static_cast<int32_t*>(ws) : nullptr;
    float* part = sk ? reinterpret_cast<float*>(static_cast<char*>(ws) + kSkCounterBytes) : nullptr;
    gemm_bf16_kernel<GATE_UP, BM, BK, STAGES, NW, LORA, FP8><<<static_cast<int>(grid), F::NT, 0, s>>>(
        a, w0, w1, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, n_tiles, part, cnt, sk ? 1 : 0, a_tok, lora,
        f8);
    return hipGetLastError();
}

}  // namespace

int64_t gemm_bf16_workspace_bytes() { return kSkWorkspaceBytes; }

hipError_t launch_gemm_bf16(int op, const uint16_t* a, const uint16_t* w0, const uint16_t* w1, uint16_t* c,
                            const int32_t* sorted_ids, const int32_t* offsets, int P, int top_k, int E, int N,
                            int K, int max_pad, void* ws, int64_t ws_bytes, hipStream_t s, const GateUpLora* lora) {
    // 256-row tiles (8 waves) when experts average at least MOE_GEMM_BIG_ROWS rows, where a 128-row
    // tiling would read most weight panels twice; 128-row tiles (4 waves) for fewer rows
    const bool big = static_cast<long long>(P) >= static_cast<long long>(MOE_GEMM_BIG_ROWS) * E;
    // down, one adapter at a rank equal to the stage depth: the delta as one more LDS stage
    if (op == kOpDown && lora && lora->n_ad == 1 && lora->rank == (big ? MOE_GEMM_BIG_BK : 64)) {
        if (big) return launch_cfg<false, 256, MOE_GEMM_BIG_BK, MOE_GEMM_BIG_STAGES, 8, 1>(a, w0, nullptr, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, ws, ws_bytes, 0, s, *lora);
        return launch_cfg<false, 128, 64, 3, 4, 1>(a, w0, nullptr, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, ws, ws_bytes, 0, s, *lora);
    }
    if (op == kOpDown && lora) {
        if (big) return launch_cfg<false, 256, MOE_GEMM_BIG_BK, MOE_GEMM_BIG_STAGES, 8, 2>(a, w0, nullptr, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, ws, ws_bytes, 0, s, *lora);
        return launch_cfg<false, 128, 64, 3, 4, 2>(a, w0, nullptr, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, ws, ws_bytes, 0, s, *lora);
    }
    if (op == kOpGateUpSilu && lora && lora->n_ad == 1) {
        if (big) return launch_cfg<true, 256, MOE_GEMM_BIG_BK, MOE_GEMM_BIG_STAGES, 8, 1>(a, w0, w1, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, ws, ws_bytes, 1, s, *lora);
        return launch_cfg<true, 128, 64, 3, 4, 1>(a, w0, w1, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, ws, ws_bytes, 1, s, *lora);
    }
    if (op == kOpGateUpSilu && lora) {
        if (big) return launch_cfg<true, 256, MOE_GEMM_BIG_BK, MOE_GEMM_BIG_STAGES, 8, 2>(a, w0, w1, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, ws, ws_bytes, 1, s, *lora);
        return launch_cfg<true, 128, 64, 3, 4, 2>(a, w0, w1, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, ws, ws_bytes, 1, s, *lora);
    }
    if (op == kOpGateUpSilu) {
        if (big) return launch_cfg<true, 256, MOE_GEMM_BIG_BK, MOE_GEMM_BIG_STAGES, 8>(a, w0, w1, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, ws, ws_bytes, 1, s);
        return launch_cfg<true, 128, 64, 3, 4>(a, w0, w1, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, ws, ws_bytes, 1, s);
    }
    // one projection, no activation: rows of a in sorted order (down) or by token (gather)
    const int a_tok = op == kOpGather ? 1 : 0;
    if (big) return launch_cfg<false, 256, MOE_GEMM_BIG_BK, MOE_GEMM_BIG_STAGES, 8>(a, w0, nullptr, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, ws, ws_bytes, a_tok, s);
    return launch_cfg<false, 128, 64, 3, 4>(a, w0, nullptr, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, ws, ws_bytes, a_tok, s);
}

hipError_t launch_gemm_fp8(bool gate_up, const uint8_t* a, const float* a_scale, const uint8_t* w0,
                           const float* ws0, const uint8_t* w1, const float* ws1, uint16_t* c,
                           const int32_t* sorted_ids, const int32_t* offsets, int P, int top_k, int E, int N,
                           int K, int max_pad, void* ws, int64_t ws_bytes, hipStream_t s) {
    // the bf16 tiles in bytes: a stage is 128 k of 1-byte codes, one 128-byte LDS row per tile row
    const Fp8Scales f8{a_scale, ws0, ws1};
    const bool big = static_cast<long long>(P) >= static_cast<long long>(MOE_GEMM_BIG_ROWS) * E;
    if (gate_up) {
        if (big) return launch_cfg<true, 256, 128, 2, 8, 0, true>(a, w0, w1, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, ws, ws_bytes, 1, s, GateUpLora{}, f8);
        return launch_cfg<true, 128, 128, 3, 4, 0, true>(a, w0, w1, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, ws, ws_bytes, 1, s, GateUpLora{}, f8);
    }
    if (big) return launch_cfg<false, 256, 128, 2, 8, 0, true>(a, w0, nullptr, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, ws, ws_bytes, 0, s, GateUpLora{}, f8);
    return launch_cfg<false, 128, 128, 3, 4, 0, true>(a, w0, nullptr, c, sorted_ids, offsets, P, top_k, E, N, K, max_pad, ws, ws_bytes, 0, s, GateUpLora{}, f8);
}

}  // namespace moe
