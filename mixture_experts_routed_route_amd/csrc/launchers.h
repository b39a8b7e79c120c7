// Host-side launchers of the gfx950 kernels (internal; the C ABI in api.cpp validates
// arguments and calls these).  Each returns the hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// grouped GEMM ops (the values of moe_gemm_op in the C header)
constexpr int kOpGateUpSilu = 0;  // x by token, gate and up, SiLU(gate) * up
constexpr int kOpDown = 1;        // sorted rows, one projection
constexpr int kOpGather = 2;      // x by token, one projection, no activation

// route.hip
hipError_t launch_route(const float* logits, int T, int E, int top_k, int renorm, int32_t* ids, float* w,
                        hipStream_t s);

// align.hip
int align_num_chunks(int64_t num_pairs);
// moe_align_noalloc: the per-chunk histogram table in a static device array of kAlignScratchCells
// int32 (1 MiB per device); align_scratch_ptr gives this device's copy (looked up on first use)
constexpr int64_t kAlignScratchCells = 1 << 18;
constexpr int kMaxDevices = 64;
hipError_t align_scratch_ptr(int32_t** out);
hipError_t launch_align(const int32_t* topk_ids, int P, int E, int bs, int32_t* counts, int32_t* offsets,
                        int32_t* sorted_ids, int32_t* expert_ids, int32_t* total, int32_t* inv, int max_pad,
                        int32_t* workspace, hipStream_t s);

// route + align in one launch when the pairs fit one chunk, else the two above
hipError_t launch_route_align(const float* logits, int T, int E, int top_k, int renorm, int32_t* ids, float* w,
                              int bs, int32_t* counts, int32_t* offsets, int32_t* sorted_ids, int32_t* expert_ids,
                              int32_t* total, int32_t* inv, int max_pad, int32_t* workspace, hipStream_t s);

// combine.hip
hipError_t launch_combine(const uint16_t* ys, const int32_t* inv, const float* w, uint16_t* out, int T, int k,
                          int H, int64_t ys_rows, hipStream_t s);

// LoRA folded in the bf16 grouped GEMM's epilogue.  Gate/up: for each projection p (0 gate, 1 up):
// xa[p] = bf16 shrink results [max_pad, rank] of the sorted rows, and the expert tables, n_ad rows of
// n_tab[p] entries, row a for the tokens of adapter a (n_tab[p] == 0: no tables, the projection is
// only rounded to bf16).  Down: the one projection's shrink results and tables in both slots.
struct GateUpLora {
    const uint16_t* xa[2];
    const uint64_t* a_tab[2];
    const uint64_t* b_tab[2];
    const float* s_tab[2];
    int n_tab[2];
    int n_ad;
    int rank;
    const int32_t* row_adapter;  // [tokens]: the token's adapter (< 0 or >= n_ad: no fold); NULL = adapter 0
};

// gemm_bf16.hip (ws: optional split-tail workspace, zero-filled before first use; NULL = none;
// lora: gate/up or down op, NULL = no fold)
int64_t gemm_bf16_workspace_bytes();
hipError_t launch_gemm_bf16(int op, const uint16_t* a, const uint16_t* w0, const uint16_t* w1, uint16_t* c,
                            const int32_t* sorted_ids, const int32_t* offsets, int P, int top_k, int E, int N,
                            int K, int max_pad, void* ws, int64_t ws_bytes, hipStream_t s,
                            const GateUpLora* lora = nullptr);

// gemm_int4.hip
hipError_t launch_gemm_int4(int op, const uint16_t* a, const int32_t* qw0, const uint16_t* sc0,
                            const int32_t* qz0, const int32_t* qw1, const uint16_t* sc1, const int32_t* qz1,
                            int group_size, uint16_t* c, const int32_t* sorted_ids, const int32_t* expert_ids,
                            int P, int top_k, int E, int N, int K, int bs, int max_pad, hipStream_t s);

// lora_fold.hip
hipError_t launch_lora_fold(const uint16_t* x, uint16_t* base, const uint64_t* a_tab, const uint64_t* b_tab,
                            const float* s_tab, int n_tab, int n_ad, int k_in, int n_out, int max_rank,
                            const int32_t* offsets, int E, const int32_t* sorted_ids, int P, int top_k,
                            const int32_t* row_adapter, uint16_t* xa, int64_t row_offset, int64_t row_end,
                            int x_gather, hipStream_t s);
// the shrink alone: xa[r - row_offset] = bf16(x[row] A_e^T) for the folded rows of the window
hipError_t launch_lora_shrink(const uint16_t* x, const uint64_t* a_tab, const uint64_t* b_tab, int n_tab, int n_ad, int k_in,
                              int max_rank, const int32_t* offsets, int E, const int32_t* sorted_ids, int P,
                              int top_k, const int32_t* row_adapter, uint16_t* xa, int64_t row_offset,
                              int64_t row_end, int x_gather, hipStream_t s);
// gemm_fp8.hip: per-row fp8 quantisation of bf16 rows (only real sorted rows with sorted_ids)
hipError_t launch_quantize_fp8(const uint16_t* x, int64_t rows, int K, const int32_t* sorted_ids, int P,
                               uint8_t* q, float* scale, hipStream_t s);
// gemm_bf16.hip, fp8 form: the grouped GEMM (gate/up + SiLU, or down) on E4M3 codes with per-row
// and per-channel scales (ws: the same optional split-tail workspace)
hipError_t launch_gemm_fp8(bool gate_up, const uint8_t* a, const float* a_scale, const uint8_t* w0,
                           const float* ws0, const uint8_t* w1, const float* ws1, uint16_t* c,
                           const int32_t* sorted_ids, const int32_t* offsets, int P, int top_k, int E, int N,
                           int K, int max_pad, void* ws, int64_t ws_bytes, hipStream_t s);
// silu_mul.hip: h[r] = bf16(silu(g[r]) * u[r]) on the real sorted rows (all rows without sorted_ids)
hipError_t launch_silu_mul(const uint16_t* g, const uint16_t* u, uint16_t* h, const int32_t* sorted_ids, int P,
                           int64_t rows, int N, hipStream_t s);
// slot-major gather fold (decode form): one workgroup per (slot, chunk)
hipError_t launch_lora_gather_fold(const uint16_t* x, int64_t x_rows, uint16_t* base, int64_t base_rows,
                                   const int32_t* indices, int64_t n_slots, int top_k, int x_gather,
                                   const int32_t* row_map, const int32_t* row_adapter, const uint64_t* a_tab,
                                   const uint64_t* b_tab, const float* s_tab, int n_tab, int n_ad, int k_in, int n_out,
                                   int max_rank, uint16_t* xa, hipStream_t s);

// probes.hip (ceiling probes, not steps of the path)
hipError_t launch_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int blocks, hipStream_t s);
hipError_t launch_probe_mfma_bf16(int64_t iters, float* sink, int blocks, hipStream_t s);

}  // namespace moe
