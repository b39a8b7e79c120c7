/*
 * moe_mi355x.h — C ABI of the routed mixture-of-experts expert path on MI355X (gfx950).
 *
 * The path, one layer of a routed MoE FFN on one GPU:
 *
 *   moe_route         top-k softmax routing of the router logits
 *   moe_align         per-expert histogram, block-padded expert_offsets,
 *                     sorted pair ids with sentinels, one expert id per block
 *   moe_align_noalloc moe_align without a workspace (static table; callers that cannot allocate)
 *   moe_route_align   the two above in one call (one launch for decode batches)
 *   moe_grouped_gemm  grouped gate/up GEMM with fused SiLU(gate)*up, the grouped
 *                     down GEMM, and one gathered projection without activation
 *                     (bf16 or GPTQ-int4 expert weights)
 *   moe_silu_mul      SiLU(gate)*up when gate and up are folded separately
 *   moe_quantize_fp8, moe_grouped_gemm_fp8   the fp8 prefill variant of the GEMMs
 *   moe_lora_fold     optional per-expert down-projection LoRA fold, in place
 *   moe_grouped_gemm_down_lora, moe_grouped_gemm_gate_up_lora   the LoRA folds run
 *                     in the grouped GEMMs' epilogues
 *   moe_lora_gather_fold  the same fold on slot-major rows (decode, no sorting)
 *   moe_combine       top-k weighted sum of the expert outputs per token
 *
 * Sources (cited by page and item; the pages are Rust host code of four
 * projects):  ferrum-kernels `src/backend/cuda/moe.rs` (route_topk_softmax,
 * moe_build_pairs_by_token, moe_align_block_size[_pair_ids], moe_combine,
 * weighted_sum_batched); ferrum-kernels `src/backend/cuda/triton_fused_moe.rs`
 * (stacked GPTQ layout, one launch over all pairs, sentinel masking); metrale
 * `gpu_runtime/cutlass/grouped.rs` (grouped gate/up/down roles, gather through
 * sorted ids, ensure_group_arrays); atlas `spark_model/layers/ops/
 * moe_lora_grouped.rs` (down-projection LoRA fold, device-side expert spans,
 * static worst-case grids, windows).
 *
 * Conventions for every entry point:
 *  - Array arguments of device entry points are DEVICE pointers, allocated and
 *    owned by the caller, 16-byte aligned.  bf16 and fp16 values travel as
 *    uint16_t bit patterns.  Layouts are row-major and contiguous.
 *  - The library allocates no memory, never synchronises, never reads device
 *    data on the host, and enqueues work only on `stream` (a hipStream_t; NULL
 *    is the null stream).  Its one piece of device memory of its own is the
 *    static 1 MiB table of moe_align_noalloc, part of the loaded code object.  Every launch grid is fixed by host scalars alone, so
 *    a sequence of calls can be captured in a HIP graph.
 *  - Return value: MOE_OK, or a negative moe_status.  Every precondition the
 *    host can check is checked before anything is enqueued; the failing call
 *    enqueues nothing and moe_last_error() names the offending argument.
 *    Device-resident values that the host cannot see (ids, offsets) get
 *    defined behaviour instead: out-of-range values are skipped, never used to
 *    address memory.
 *  - Thread safety: all entry points are re-entrant; moe_last_error() is
 *    per calling thread.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
#define MOE_OK 0
#define MOE_EINVAL (-1)        /* a host-checkable argument is invalid               */
#define MOE_EUNSUPPORTED (-2)  /* valid but outside what the kernels support (E>256)  */
#define MOE_ELAUNCH (-3)       /* the HIP runtime refused the launch                  */

typedef void* moe_stream; /* hipStream_t */

/* Text of the last non-OK status returned on this thread ("" if none). */
const char* moe_last_error(void);

/* ABI version of this header (bumped on any signature change). */
int32_t moe_abi_version(void);

/* ============================================================== pure host helpers (no GPU) */

/* Rows the sorted layout needs in the worst case: roundup(P + E*(bs-1), bs).
 * The capacity `sorted_max_size` of ferrum moe.rs moe_align_block_size, which
 * that page passes without a formula.  Returns -1 on invalid arguments. */
int64_t moe_align_max_padded(int64_t num_pairs, int32_t num_experts, int32_t block_size);

/* Bytes of device workspace moe_align needs (per-chunk expert histograms). */
int64_t moe_align_workspace_bytes(int64_t num_pairs, int32_t num_experts);

/* Group-array check of metrale cutlass/grouped.rs, ensure_group_arrays:
 * `offsets` (host, `offsets_len` entries) must have num_experts+1 entries,
 * offsets[0] >= 0 and never decrease; each of the `n_arrays` per-expert host
 * arrays, whose lengths are `lens[i]` and names `names[i]`, must have
 * num_experts entries.  MOE_EINVAL with a message naming the first offender. */
moe_status moe_check_group_arrays(int32_t num_experts, const int64_t* lens, const char* const* names,
                                  int32_t n_arrays, const int32_t* offsets, int64_t offsets_len);

/* Dense per-expert LoRA tables, atlas moe_lora_grouped.rs pack_expert_tables:
 * entries (ids[i], a[i], b[i], s[i]) for i < n are scattered into tables of
 * length n_tab = max id + 1 (written to *n_tab); unadapted slots hold 0 / 0.0;
 * a repeated id keeps its last entry; n == 0 gives *n_tab = 0 (no route).
 * Output arrays are host arrays of capacity `cap` entries.  Ids must be in
 * [0, 65535] (the page keys experts by u16). */
moe_status moe_lora_pack_tables(const int32_t* ids, const uint64_t* a, const uint64_t* b, const float* s,
                                int32_t n, uint64_t* a_out, uint64_t* b_out, float* s_out, int32_t cap,
                                int32_t* n_tab);

/* Row tiles (64 rows each) of one fold window, atlas moe_lora_grouped.rs
 * grouped_down_wc: max(1, ceil((row_end - row_offset) / 64)). */
int64_t moe_lora_window_tiles(int64_t row_offset, int64_t row_end);

/* Contiguous [start, end) windows of at most `cap` rows covering 0..total_rows
 * (atlas moe_lora_grouped.rs grouped_down_windows).  Writes up to
 * `max_windows` pairs and returns the number of windows, or -1 if cap <= 0. */
int64_t moe_lora_windows(int64_t total_rows, int64_t cap, int64_t* starts, int64_t* ends,
                         int64_t max_windows);

/* ============================================================== device entry points */

/* A1 — top-k softmax routing (ferrum moe.rs, route_topk_softmax).
 *   logits   fp32 [num_tokens, num_experts]
 *   topk_ids i32  [num_tokens, top_k]   out: selected experts, most probable first
 *   topk_w   fp32 [num_tokens, top_k]   out: their weights
 * Per token: probabilities p = softmax over all experts; the top_k experts by
 * logit (ties: lower index first); with `renormalize` the kept p are divided
 * by their sum.  Weights are computed in fp64 and rounded once to fp32.
 * Logits must be finite.  1 <= top_k <= num_experts <= 256.  num_tokens == 0
 * enqueues nothing. */
moe_status moe_route(const float* logits, int32_t num_tokens, int32_t num_experts, int32_t top_k,
                     int32_t renormalize, int32_t* topk_ids, float* topk_w, moe_stream stream);

/* A2 — alignment of the P = num_tokens*top_k (token, slot) pairs by expert
 * (ferrum moe.rs, moe_build_pairs_by_token + moe_align_block_size_pair_ids).
 *   topk_ids       i32 [num_pairs]          flat pair p = t*top_k + j -> expert
 *   counts         i32 [num_experts]        out: real rows per expert
 *   expert_offsets i32 [num_experts + 1]    out: block-padded exclusive prefix sum;
 *                                           expert e owns sorted rows [off[e], off[e+1]),
 *                                           its real rows are the first counts[e]
 *   sorted_ids     i32 [max_pad]            out: pair id per sorted row, ascending p
 *                                           within an expert; every other row holds
 *                                           the sentinel num_pairs
 *   expert_ids     i32 [max_pad/block_size] out: expert of each block, -1 past the end
 *   total_padded   i32 [1]                  out: off[num_experts]
 *   inv_sorted     i32 [num_pairs]          out: sorted row of each pair (-1 if dropped)
 *   workspace      device, >= moe_align_workspace_bytes(num_pairs, num_experts) bytes
 * An id outside [0, num_experts) is dropped: not counted, inv_sorted = -1.
 * max_pad >= moe_align_max_padded(...) and a multiple of block_size;
 * block_size in {16, 32, 64, 128}; num_experts <= 256 (MOE_EUNSUPPORTED above,
 * the limit of ferrum's MAX_NUM_EXPERTS). */
moe_status moe_align(const int32_t* topk_ids, int64_t num_pairs, int32_t num_experts, int32_t block_size,
                     int32_t* counts, int32_t* expert_offsets, int32_t* sorted_ids, int32_t* expert_ids,
                     int32_t* total_padded, int32_t* inv_sorted, int64_t max_pad, void* workspace,
                     int64_t workspace_bytes, moe_stream stream);

/* A2 without a workspace, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same arguments, results and
 * error behaviour as moe_align, minus workspace/workspace_bytes: the per-chunk histogram table
 * lives in a static device array of the library (1 MiB per GPU, 2^18 int32 cells, held until the
 * process ends).  Batches of more than 2048 pairs are cut into chunks of 512 pairs, and
 * ceil(num_pairs / 512) * num_experts must not exceed 2^18 (for example 2^19 pairs at 256 experts,
 * 2^21 at 64); above that the call returns MOE_EUNSUPPORTED before anything is enqueued.
 * The call allocates nothing.  Every call on one GPU uses that GPU's one table and overwrites the
 * cells it reads, so calls ordered on one stream are independent, while calls that overlap on one
 * GPU (concurrent streams) race.  The first call on a device looks up the table's address; make it
 * outside graph capture. */
moe_status moe_align_noalloc(const int32_t* topk_ids, int64_t num_pairs, int32_t num_experts, int32_t block_size,
                             int32_t* counts, int32_t* expert_offsets, int32_t* sorted_ids, int32_t* expert_ids,
                             int32_t* total_padded, int32_t* inv_sorted, int64_t max_pad, moe_stream stream);

/* A1+A2 — moe_route followed by moe_align on its topk_ids, with the same
 * arguments, results and error behaviour as the two calls (topk_ids is both the
 * routing output and the alignment input; num_pairs = num_tokens*top_k).  When
 * the pairs fit one alignment workgroup (num_pairs <= 2048, decode batches) both
 * steps run in one single-workgroup launch; otherwise it enqueues the launches
 * of the two calls.  num_tokens == 0 aligns zero pairs (fills the sentinels). */
moe_status moe_route_align(const float* logits, int32_t num_tokens, int32_t num_experts, int32_t top_k,
                           int32_t renormalize, int32_t* topk_ids, float* topk_w, int32_t block_size,
                           int32_t* counts, int32_t* expert_offsets, int32_t* sorted_ids, int32_t* expert_ids,
                           int32_t* total_padded, int32_t* inv_sorted, int64_t max_pad, void* workspace,
                           int64_t workspace_bytes, moe_stream stream);

/* Expert weights of one projection, K = contraction, N = outputs.
 *   MOE_W_BF16:      data = bf16 [E, N, K] (K contiguous); scales, qzeros unused.
 *   MOE_W_INT4_GPTQ: data = int32 qweight [E, K/8, N], K index 8i+s in nibble s of
 *                    word i; scales = fp16 [E, K/G, N]; qzeros = int32 [E, K/G, N/8],
 *                    N index 8i+s in nibble s; W[k,n] = (q - z) * s, groups of G
 *                    consecutive k (ferrum triton_fused_moe.rs, TritonStackedGptqWeight).
 *   MOE_W_FP8:       data = uint8 OCP FP8 E4M3 codes [E, N, K] (K contiguous);
 *                    scales = fp32 [E, N]; W[n,k] = value(code) * scales[e, n].  Used by
 *                    moe_grouped_gemm_fp8 only. */
typedef enum { MOE_W_BF16 = 0, MOE_W_INT4_GPTQ = 1, MOE_W_FP8 = 2 } moe_wtype;
typedef struct moe_weight {
    int32_t type;            /* moe_wtype */
    int32_t group_size;      /* G (int4 only): multiple of 32, divides K */
    const void* data;
    const void* scales;      /* int4: fp16 [E, K/G, N]; fp8: fp32 [E, N] */
    const int32_t* qzeros;
} moe_weight;

typedef enum { MOE_OP_GATE_UP_SILU = 0, MOE_OP_DOWN = 1, MOE_OP_GATHER = 2 } moe_gemm_op;

/* A3/A4 — grouped expert GEMM over the sorted, block-padded rows (one launch
 * for all experts; metrale cutlass/grouped.rs nvfp4_grouped_gate_up_fused /
 * nvfp4_grouped_down roles, ferrum triton_fused_moe.rs masking).
 *   MOE_OP_GATE_UP_SILU: a = x [num_pairs/top_k, K] token-major; sorted row r
 *                        reads token sorted_ids[r]/top_k; w0 = gate, w1 = up;
 *                        c[r, :N] = bf16(silu(x Wg^T) * (x Wu^T))
 *   MOE_OP_DOWN:         a = Hs [max_pad, K] in sorted order; w0 = down, w1 = NULL;
 *                        c[r, :N] = bf16(Hs[r] Wd^T)
 *   MOE_OP_GATHER:       a = x token-major as for GATE_UP_SILU; w0 = one projection,
 *                        w1 = NULL; c[r, :N] = bf16(x[t] W^T), no activation.  The
 *                        gate and up outputs that a gate/up LoRA fold works on (atlas
 *                        moe_lora_grouped.rs: the fold with x_gather = 1 updates the
 *                        sorted BF16 expert_gate_out / expert_up_out); moe_silu_mul
 *                        then makes Hs.
 * The expert of row r is the block's expert (expert_ids / expert_offsets from
 * moe_align).  Sentinel and padding rows are neither read as tokens nor
 * written: c keeps its previous content there.  fp32 accumulation.
 *   c: bf16 [max_pad, N].  K % 8 == 0, N % 8 == 0 (int4: N % 64 == 0,
 *   K % group_size == 0).  Both weights must have the same type.  bf16: a
 *   and each expert's [N, K] matrix must each be under 4 GiB
 *   (MOE_EUNSUPPORTED otherwise).
 *   workspace: optional device buffer of >= moe_grouped_gemm_workspace_bytes()
 *   bytes, or NULL.  With it, a bf16 launch whose output tiles end in a
 *   partial round of the persistent grid cuts that round's tiles along K into
 *   pieces spread over the whole grid (split tail), so no compute unit idles
 *   through a last partial round; the pieces of a tile meet through fp32
 *   partials and a counter kept there.  It must be zero-filled once before
 *   its first use; every call leaves its
 *   counters at zero again.  Calls that share one workspace must not run
 *   concurrently.  A smaller non-NULL buffer is rejected (MOE_EINVAL).  int4
 *   launches check its size but do not use it.  Results with and without it
 *   agree to fp32 summation order; with it they are deterministic (pieces are
 *   summed in a fixed order). */
moe_status moe_grouped_gemm(int32_t op, const uint16_t* a, const moe_weight* w0, const moe_weight* w1,
                            uint16_t* c, const int32_t* sorted_ids, const int32_t* expert_ids,
                            const int32_t* expert_offsets, int64_t num_pairs, int32_t top_k,
                            int32_t num_experts, int32_t n, int32_t k, int32_t block_size, int64_t max_pad,
                            void* workspace, int64_t workspace_bytes, moe_stream stream);

/* Size in bytes of the optional moe_grouped_gemm workspace (fixed; it does not
 * depend on the problem). */
int64_t moe_grouped_gemm_workspace_bytes(void);

/* FP8 prefill (atlas moe_lora_grouped.rs module doc: an fp8 grouped prefill path
 * that writes the same sorted BF16 expert_down_out; the page fixes no format, so the
 * reading is OCP FP8 E4M3 with per-row activation and per-channel weight scales).
 *
 * moe_quantize_fp8: per-row dynamic quantisation of bf16 rows, in fp32:
 *   amax = max |x[r]|; scale[r] = amax / 448; q[r] = e4m3(x[r] * (448 / amax)),
 *   round to nearest even (scale 1 and zero codes for an all-zero row).
 *   x bf16 [rows, k], q uint8 [rows, k], scale fp32 [rows].  With sorted_ids
 *   (i32 [rows]) only rows r with sorted_ids[r] in [0, num_pairs) are written (the
 *   real sorted rows of Hs); NULL writes every row (the token rows of x).
 *   k % 16 == 0.  rows == 0 enqueues nothing. */
moe_status moe_quantize_fp8(const uint16_t* x, int64_t rows, int32_t k, const int32_t* sorted_ids,
                            int64_t num_pairs, uint8_t* q, float* scale, moe_stream stream);

/* moe_grouped_gemm_fp8: the grouped GEMMs with fp8 operands; arguments as for
 * moe_grouped_gemm, plus
 *   a        uint8 e4m3 codes: GATE_UP_SILU x [num_pairs/top_k, K] by token; DOWN Hs
 *            [max_pad, K] in sorted order (moe_quantize_fp8 outputs)
 *   a_scale  fp32 per row of a ([num_pairs/top_k] or [max_pad])
 *   w0, w1   MOE_W_FP8 weights (gate and up, or down)
 *   c        bf16 [max_pad, N]: GATE_UP_SILU silu(g)*u, DOWN y, where
 *            g[r, n] = a_scale[row] * scales[e, n] * sum_k a(row, k) W(n, k)
 *            (exact fp8 products, fp32 sums)
 * Sentinel and padding rows are not written.  op is MOE_OP_GATE_UP_SILU or
 * MOE_OP_DOWN; K % 16 == 0; N % 8 == 0.  As for the bf16 form, a (its rows:
 * num_pairs/top_k for gate/up, max_pad for down) and each expert's [N, K] matrix
 * must each be under 4 GiB (else MOE_EUNSUPPORTED).  workspace: as for
 * moe_grouped_gemm (the same buffer serves both; the tiles of a last partial round
 * are split along K, with results deterministic and equal to those without it up
 * to fp32 order). */
moe_status moe_grouped_gemm_fp8(int32_t op, const uint8_t* a, const float* a_scale, const moe_weight* w0,
                                const moe_weight* w1, uint16_t* c, const int32_t* sorted_ids,
                                const int32_t* expert_offsets, int64_t num_pairs, int32_t top_k,
                                int32_t num_experts, int32_t n, int32_t k, int32_t block_size, int64_t max_pad,
                                void* workspace, int64_t workspace_bytes, moe_stream stream);

/* A5 — LoRA fold, in place, on one window [row_offset, row_end) of the sorted
 * rows (atlas moe_lora_grouped.rs, moe_lora_grouped_down).
 *   x           x_gather == 0 (down):    bf16 [max_pad, k_in], post-SiLU sorted activations (Hs)
 *               x_gather == 1 (gate/up): bf16 [num_pairs/top_k, k_in], the token-major layer
 *                                        input; sorted row r reads token sorted_ids[r]/top_k
 *   base        bf16 [max_pad, n_out]  sorted expert_down_out (Ys), or a sorted gate or up
 *                                      output (MOE_OP_GATHER) for x_gather == 1; in place
 *   a_table     u64  [n_adapters, n_tab] device  address of A_e of adapter a at [a, e],
 *                                      bf16 [max_rank, k_in]; 0 = e not adapted by a
 *   b_table     u64  [n_adapters, n_tab] device  address of B_e, bf16 [n_out, max_rank]; 0 = unadapted
 *   scale_table f32  [n_adapters, n_tab] device  scale_e of adapter a
 *   n_adapters  adapters installed (>= 1): the rows of the tables
 *   row_adapter i32  [num_pairs/top_k] or NULL: the adapter of each token (atlas: a mixed batch's
 *                                      adapter identity comes from this per-row map, not from the
 *                                      tables); < 0 = base (not folded), an id >= n_adapters is not
 *                                      folded either; NULL = adapter 0 for every token
 *   xa          bf16 [cap, max_rank]   scratch, indexed by the local row r - row_offset
 * For each real row r in the window whose token's adapter a adapts the row's expert e (e < n_tab,
 * non-zero table entries at [a, e]):
 *   xa = bf16(x[x row] A_e^T); delta = bf16(xa B_e^T); base[r] = bf16(base[r] + scale_e*delta)
 * with fp32 sums and adapter a's A_e, B_e, scale_e.  Other rows are not touched.  Windows may be
 * applied one after the other with the same xa scratch (stream order).  max_rank % 32 == 0,
 * k_in % 8 == 0, n_out % 8 == 0, cap >= row_end - row_offset, n_tab <= num_experts,
 * 1 <= n_adapters <= 65536. */
moe_status moe_lora_fold(const uint16_t* x, uint16_t* base, const uint64_t* a_table, const uint64_t* b_table,
                         const float* scale_table, int32_t n_tab, int32_t n_adapters, int32_t k_in, int32_t n_out,
                         int32_t max_rank,
                         const int32_t* expert_offsets, int32_t num_experts, const int32_t* sorted_ids,
                         int64_t num_pairs, int32_t top_k, const int32_t* row_adapter, uint16_t* xa, int64_t cap,
                         int64_t row_offset, int64_t row_end, int64_t max_pad, int32_t x_gather,
                         moe_stream stream);

/* The gate/up LoRA fused into the gate/up GEMM (bf16 weights): the same
 * result as MOE_OP_GATHER for gate and up, moe_lora_fold with x_gather = 1 on
 * each, and moe_silu_mul, in one GEMM whose epilogue folds a rank-r product
 * (atlas moe_lora_grouped.rs: the gate/up fold over token-major x on the sorted
 * BF16 expert_gate_out / expert_up_out before SiLU).  For each real sorted row
 * r of expert e (token t = sorted_ids[r] / top_k):
 *   g = bf16(x[t] Wg[e]^T); if the gate tables of the token's adapter a (row_adapter[t],
 *   0 without a map) adapt e: g = bf16(g + s_gate[a,e] * bf16(bf16(x[t] A_gate[a,e]^T) B_gate[a,e]^T));
 *   u likewise with the up tables; hs[r] = bf16(silu(g) * u).
 *   x, w_gate, w_up, hs, sorted ids ... max_pad, workspace: as moe_grouped_gemm
 *   with MOE_OP_GATE_UP_SILU (n = intermediate, k = hidden)
 *   a_*, b_*, s_*, n_tab_*: tables as for moe_lora_fold, [n_adapters, n_tab_*] (A [max_rank, k],
 *   B [n, max_rank]); n_tab 0 = no tables for that projection
 *   row_adapter  i32 [num_pairs/top_k] or NULL, as for moe_lora_fold
 *   xa           bf16 [2, max_pad, max_rank] scratch (the gate and up shrinks)
 * Launches the two shrinks and the GEMM.  MOE_EUNSUPPORTED for int4 weights.
 * max_rank in {32, 64, 96, 128}. */
moe_status moe_grouped_gemm_gate_up_lora(const uint16_t* x, const moe_weight* w_gate, const moe_weight* w_up,
                                         uint16_t* hs, const int32_t* sorted_ids, const int32_t* expert_offsets,
                                         int64_t num_pairs, int32_t top_k, int32_t num_experts, int32_t n, int32_t k,
                                         int32_t block_size, int64_t max_pad, const uint64_t* a_gate,
                                         const uint64_t* b_gate, const float* s_gate, int32_t n_tab_gate,
                                         const uint64_t* a_up, const uint64_t* b_up, const float* s_up,
                                         int32_t n_tab_up, int32_t n_adapters, int32_t max_rank,
                                         const int32_t* row_adapter,
                                         uint16_t* xa, void* workspace, int64_t workspace_bytes,
                                         moe_stream stream);

/* The down-projection LoRA fold fused into the down GEMM (bf16 weights): the same
 * result as moe_grouped_gemm with MOE_OP_DOWN followed by moe_lora_fold (x_gather = 0)
 * over all sorted rows, with the expand and the fold run in the GEMM's epilogue, so
 * the folded Ys rows are written once instead of written, read back and written again
 * (atlas moe_lora_grouped.rs, moe_lora_grouped_down: shrink, then expand and fold in
 * place into the sorted BF16 expert_down_out).  For each real sorted row r of expert e
 * (token t = sorted_ids[r] / top_k, adapter a = row_adapter[t], 0 without a map):
 *   y = bf16(Hs[r] Wd[e]^T); if adapter a adapts e (e < n_tab, non-zero entries at [a, e]):
 *   y = bf16(y + scale[a,e] * bf16(bf16(Hs[r] A[a,e]^T) B[a,e]^T)); ys[r] = y,
 * fp32 sums.  Sentinel and padding rows are not written.
 *   hs, w_down, ys, sorted ids ... max_pad, workspace: as moe_grouped_gemm with
 *   MOE_OP_DOWN (n = hidden, k = intermediate)
 *   a_table, b_table, scale_table, n_tab, n_adapters, row_adapter: as for moe_lora_fold,
 *   [n_adapters, n_tab] (A [max_rank, k], B [n, max_rank]); n_tab 0 = plain down GEMM
 *   xa           bf16 [max_pad, max_rank] scratch (the shrink's results, by sorted row)
 * Launches the shrink and the GEMM.  MOE_EUNSUPPORTED for non-bf16 weights.
 * max_rank in {32, 64, 96, 128}. */
moe_status moe_grouped_gemm_down_lora(const uint16_t* hs, const moe_weight* w_down, uint16_t* ys,
                                      const int32_t* sorted_ids, const int32_t* expert_offsets, int64_t num_pairs,
                                      int32_t top_k, int32_t num_experts, int32_t n, int32_t k, int32_t block_size,
                                      int64_t max_pad, const uint64_t* a_table, const uint64_t* b_table,
                                      const float* scale_table, int32_t n_tab, int32_t n_adapters, int32_t max_rank,
                                      const int32_t* row_adapter, uint16_t* xa, void* workspace,
                                      int64_t workspace_bytes, moe_stream stream);

/* SiLU(gate) * up of the gate/up LoRA path (atlas moe_lora_grouped.rs,
 * moe_lora_gather_bgmv: the caller's moe_silu_mul writes the BF16 activations
 * the down projection and its fold read).
 *   gate, up    bf16 [rows, n]
 *   out         bf16 [rows, n]   out[r] = bf16(silu(gate[r]) * up[r]), fp32 arithmetic
 *   sorted_ids  i32 [rows] or NULL: only rows with sorted_ids[r] in [0, num_pairs)
 *               are written (the real sorted rows); NULL writes every row
 * n % 8 == 0.  rows == 0 enqueues nothing. */
moe_status moe_silu_mul(const uint16_t* gate, const uint16_t* up, uint16_t* out, const int32_t* sorted_ids,
                        int64_t num_pairs, int64_t rows, int32_t n, moe_stream stream);

/* Decode form of the LoRA fold, slot-major, in place (atlas moe_lora_grouped.rs,
 * moe_lora_gather_bgmv, gather_row_token).  No sorted layout: flat (token, slot)
 * row s < n_slots (= tokens * top_k) takes its expert e = indices[s] and its
 * adapter a = row_adapter[s / top_k] (< 0 or >= n_adapters skips; NULL = adapter 0).
 *   x           bf16 [x_rows, k_in]     x_gather == 0: row = the slot's row (the
 *                                       post-SiLU activations of the down fold);
 *                                       x_gather == 1: row s / top_k (token-major
 *                                       input of the gate/up fold)
 *   base        bf16 [base_rows, n_out] folded in place at the slot's row
 *   indices     i32  [n_slots]          expert per slot (the router's topk_ids)
 *   row_map     i32  [n_slots] or NULL  the slot's row of base (and of x when
 *                                       x_gather == 0); NULL = s (slot-major, as on
 *                                       the page); a negative entry skips the slot.
 *                                       With moe_align's inv_sorted it folds buffers
 *                                       in sorted order.
 *   a_table, b_table, scale_table, n_tab, n_adapters: as for moe_lora_fold, [n_adapters, n_tab]
 *   xa          bf16 [n_slots, max_rank] scratch, indexed by s
 * For each slot whose adapter a adapts its expert (e in [0, n_tab), non-zero table
 * entries at [a, e]): xa = bf16(x[x row] A_e^T); delta = bf16(xa B_e^T);
 * base[row] = bf16(base[row] + scale_e*delta), fp32 sums.  Other rows are not
 * touched.  One workgroup per (slot, output chunk): the grid depends on n_slots
 * only.  Device values that the host cannot check get defined behaviour: an id
 * outside the tables, a map entry outside [0, base_rows) or an x row outside
 * [0, x_rows) skips the slot.  Two slots mapped to the same row race (the
 * caller keeps the map injective; inv_sorted is).  n_slots % top_k == 0;
 * x_rows >= n_slots / top_k (x_gather == 1) or >= n_slots (x_gather == 0, no
 * row_map); base_rows >= n_slots without a row_map; max_rank in {32, 64, 96,
 * 128}; k_in % 8 == 0; n_out % 8 == 0; n_tab <= 65536. */
moe_status moe_lora_gather_fold(const uint16_t* x, int64_t x_rows, uint16_t* base, int64_t base_rows,
                                const int32_t* indices, int64_t n_slots, int32_t top_k, int32_t x_gather,
                                const int32_t* row_map, const int32_t* row_adapter, const uint64_t* a_table,
                                const uint64_t* b_table, const float* scale_table, int32_t n_tab, int32_t n_adapters,
                                int32_t k_in, int32_t n_out, int32_t max_rank, uint16_t* xa, moe_stream stream);

/* A6 — top-k weighted combine (ferrum moe.rs, moe_combine / weighted_sum_batched).
 *   ys         bf16 [ys_rows, hidden]
 *   inv_sorted i32  [num_tokens*top_k] or NULL (slot-major: row t*top_k + j)
 *   topk_w     fp32 [num_tokens, top_k]
 *   out        bf16 [num_tokens, hidden]
 * out[t] = bf16(sum_{j<top_k} topk_w[t,j] * ys[row(t,j)]), fp32, j ascending;
 * a row outside [0, ys_rows) contributes nothing.  hidden % 8 == 0. */
moe_status moe_combine(const uint16_t* ys, const int32_t* inv_sorted, const float* topk_w, uint16_t* out,
                       int32_t num_tokens, int32_t top_k, int32_t hidden, int64_t ys_rows, moe_stream stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
