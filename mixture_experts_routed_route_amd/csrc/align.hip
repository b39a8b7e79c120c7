// Block-size alignment of the (token, slot) pairs by expert (ferrum-kernels cuda/moe.rs:
// moe_build_pairs_by_token, moe_align_block_size_pair_ids): a stable counting sort.
//
// The pairs are cut into chunks of kChunk ids; one 256-thread workgroup owns a chunk.
//   1. align_count: each workgroup builds its chunk's expert histogram in LDS and
//      writes it to the workspace row ws[chunk][0..E).
//   2. align_scatter: each workgroup reads the whole [chunks, E] table, derives the
//      per-expert totals, the block-padded offsets (LDS scan) and the first row its
//      chunk owns in every expert, then places its pairs.  Inside a chunk each wave
//      owns a contiguous run of pairs; the rank of a pair among earlier pairs of the
//      same expert comes from wavefront ballots on the bits of the expert id (peer
//      masks) plus per-wave LDS counters, so the order within an expert is ascending
//      pair id.  All workgroups also share the sentinel and expert_ids fills.
// Deterministic: no order-dependent atomics (the LDS histogram atomics only count).
#include "device_common.h"
#include "launchers.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kIters = 8;                            // 64-pair steps per wave
constexpr int kChunk = kThreads * kIters;            // pairs per workgroup
constexpr int kMaxE = 256;

__global__ __launch_bounds__(kThreads) void align_count_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                               int32_t* __restrict__ ws) {
    __shared__ int hist[kMaxE];
    const int g = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += kThreads) hist[e] = 0;
    __syncthreads();
    const int base = g * kChunk;
    for (int i = threadIdx.x; i < kChunk; i += kThreads) {
        const int p = base + i;
        if (p < P) {
            const int e = ids[p];
            if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kThreads) ws[static_cast<size_t>(g) * E + e] = hist[e];
}

// Peer mask of this lane: lanes of the wave holding the same key (9-bit keys).
__device__ __forceinline__ uint64_t peer_mask(int key, bool active) {
    uint64_t m = __ballot(active);
#pragma unroll
    for (int b = 0; b < 9; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    return m;
}

__global__ __launch_bounds__(kThreads) void align_scatter_kernel(
    const int32_t* __restrict__ ids, int P, int E, int bs, const int32_t* __restrict__ ws, int G,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ expert_ids, int32_t* __restrict__ total_out, int32_t* __restrict__ inv, int max_pad) {
    __shared__ int s_off[kMaxE + 1];   // block-padded offsets
    __shared__ int s_cnt[kMaxE];       // real rows per expert
    __shared__ int s_run[kWaves][kMaxE];
    __shared__ int s_scan[kWaves];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = blockIdx.x;

    // totals and this chunk's start inside each expert
    int tot = 0, before = 0;
    if (tid < E) {
        for (int c = 0; c < G; ++c) {
            const int v = ws[static_cast<size_t>(c) * E + tid];
            before += (c < g) ? v : 0;
            tot += v;
        }
    }
    const int padded = (tid < E) ? ((tot + bs - 1) / bs) * bs : 0;
    const int incl = block_inclusive_scan_256(padded, s_scan);
    if (tid < E) {
        s_off[tid] = incl - padded;
        s_cnt[tid] = tot;
    }
    if (tid == E - 1) s_off[E] = incl;
    for (int w = 0; w < kWaves; ++w)
        if (tid < E) s_run[w][tid] = 0;
    __syncthreads();
    const int total = s_off[E];

    if (g == 0) {
        if (tid < E) { counts[tid] = s_cnt[tid]; offsets[tid] = s_off[tid]; }
        if (tid == 0) { offsets[E] = total; total_out[0] = total; }
    }

    // expert_ids for every block, sentinels for every row that no pair will fill
    const int stride = G * kThreads;
    const int nblk = max_pad / bs;
    for (int b = g * kThreads + tid; b < nblk; b += stride) {
        const int r = b * bs;
        expert_ids[b] = (r < total) ? upper_index(s_off, E, r) : -1;
    }
    for (int r = g * kThreads + tid; r < max_pad; r += stride) {
        bool pad = r >= total;
        if (!pad) {
            const int e = upper_index(s_off, E, r);
            pad = r >= s_off[e] + s_cnt[e];
        }
        if (pad) sorted_ids[r] = P;
    }

    // pass A: per-wave counts of each expert over the wave's run of pairs
    const int run0 = g * kChunk + wave * (64 * kIters);
    for (int it = 0; it < kIters; ++it) {
        const int p = run0 + it * 64 + lane;
        const bool in = p < P;
        const int e = in ? ids[p] : -1;
        const bool valid = in && e >= 0 && e < E;
        const int key = valid ? e : 511;
        const uint64_t peers = peer_mask(key, in);
        const int rank = __popcll(peers & ((1ull << lane) - 1ull));
        if (valid && rank == 0) s_run[wave][e] += __popcll(peers);
    }
    __syncthreads();
    // per-wave start positions: expert base + this chunk's earlier chunks + earlier waves
    if (tid < E) {
        int pos = s_off[tid] + before;
        for (int w = 0; w < kWaves; ++w) {
            const int c = s_run[w][tid];
            s_run[w][tid] = pos;
            pos += c;
        }
    }
    __syncthreads();
    // pass B: place the pairs
    for (int it = 0; it < kIters; ++it) {
        const int p = run0 + it * 64 + lane;
        const bool in = p < P;
        const int e = in ? ids[p] : -1;
        const bool valid = in && e >= 0 && e < E;
        const int key = valid ? e : 511;
        const uint64_t peers = peer_mask(key, in);
        const int rank = __popcll(peers & ((1ull << lane) - 1ull));
        if (valid) {
            const int r = s_run[wave][e] + rank;
            sorted_ids[r] = p;
            inv[p] = r;
        } else if (in) {
            inv[p] = -1;
        }
        if (valid && rank == 0) s_run[wave][e] += __popcll(peers);
    }
}

}  // namespace

int align_num_chunks(int64_t num_pairs) {
    const int64_t g = (num_pairs + kChunk - 1) / kChunk;
    return static_cast<int>(g < 1 ? 1 : g);
}

hipError_t launch_align(const int32_t* topk_ids, int P, int E, int bs, int32_t* counts, int32_t* offsets,
                        int32_t* sorted_ids, int32_t* expert_ids, int32_t* total, int32_t* inv, int max_pad,
                        int32_t* workspace, hipStream_t s) {
    const int G = align_num_chunks(P);
    align_count_kernel<<<G, kThreads, 0, s>>>(topk_ids, P, E, workspace);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    align_scatter_kernel<<<G, kThreads, 0, s>>>(topk_ids, P, E, bs, workspace, G, counts, offsets, sorted_ids,
                                                 expert_ids, total, inv, max_pad);
    return hipGetLastError();
}

}  // namespace moe
