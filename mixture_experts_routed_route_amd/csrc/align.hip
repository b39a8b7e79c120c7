// Block-size alignment of the (token, slot) pairs by expert (ferrum-kernels cuda/moe.rs:
// moe_build_pairs_by_token, moe_align_block_size_pair_ids): a stable counting sort.
//
// The pairs are cut into chunks of kChunk ids; one 256-thread workgroup owns a chunk.  When
// all pairs fit the kChunkOne ids one workgroup can hold (decode batches), step 1 is folded into
// step 2: one launch.  Otherwise the chunks are small (512 ids), so that even a mid-size batch
// spreads its serial per-workgroup work (table sums, scan, fills, two passes) over many workgroups.
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
#include <mutex>

#include "device_common.h"
#include "launchers.h"
#include "route_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kIters = 2;                            // 64-pair steps per wave, several chunks
constexpr int kChunk = kThreads * kIters;            // pairs per workgroup, several chunks
constexpr int kItersOne = 8;                         // 64-pair steps per wave, one workgroup
constexpr int kChunkOne = kThreads * kItersOne;      // pairs one workgroup aligns alone
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

// SINGLE: all pairs fit one workgroup (at most kChunkOne); the workgroup builds the histogram
// itself, so the alignment is one launch with no workspace round trip.  Otherwise g = this
// workgroup's chunk of kChunk pairs.  NWAVES: waves of the workgroup (4, or 16 in the fused
// route+align kernel); pairs are held by the first kWaves waves only, the others take part in the
// scan, the fills and the barriers.
template <bool SINGLE, int NWAVES = kWaves>
__device__ __forceinline__ void align_scatter_body(
    const int32_t* __restrict__ ids, int P, int E, int bs, const int32_t* __restrict__ ws, int G,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ expert_ids, int32_t* __restrict__ total_out, int32_t* __restrict__ inv, int max_pad,
    int g) {
    __shared__ int s_off[kMaxE + 1];   // block-padded offsets
    __shared__ int s_cnt[kMaxE];       // real rows per expert
    __shared__ int s_run[kWaves][kMaxE];
    __shared__ int s_scan[NWAVES];
    constexpr int NT = 64 * NWAVES;
    static_assert(SINGLE || NWAVES == kWaves, "several chunks: 4 waves per workgroup");

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int ITERS = SINGLE ? kItersOne : kIters;  // 64-pair steps per wave
    constexpr int CHUNK = kWaves * 64 * ITERS;

    // this wave's run of pairs, loaded once (expert id, or -1 past the end / out of range); waves
    // past the first kWaves start past CHUNK >= P and hold none
    const int run0 = g * CHUNK + wave * (64 * ITERS);
    int e_reg[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int p = run0 + it * 64 + lane;
        const int e = p < P ? ids[p] : -1;
        e_reg[it] = (e >= 0 && e < E) ? e : -1;
    }

    // totals and this chunk's start inside each expert
    int tot = 0, before = 0;
    if constexpr (SINGLE) {
        for (int e = tid; e < E; e += NT) s_cnt[e] = 0;
        __syncthreads();
#pragma unroll
        for (int it = 0; it < ITERS; ++it)
            if (e_reg[it] >= 0) atomicAdd(&s_cnt[e_reg[it]], 1);
        __syncthreads();
        if (tid < E) tot = s_cnt[tid];
        __syncthreads();
    } else {
        if (tid < E) {
            // eight chunks' counts per round, loaded together: one memory round trip per eight
            // chunks instead of one per chunk
            int c = 0;
            for (; c + 8 <= G; c += 8) {
                int v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] = ws[static_cast<size_t>(c + u) * E + tid];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    before += (c + u < g) ? v[u] : 0;
                    tot += v[u];
                }
            }
            for (; c < G; ++c) {
                const int v = ws[static_cast<size_t>(c) * E + tid];
                before += (c < g) ? v : 0;
                tot += v;
            }
        }
    }
    const int padded = (tid < E) ? ((tot + bs - 1) / bs) * bs : 0;
    const int incl = block_inclusive_scan<NWAVES>(padded, s_scan, (E + 63) / 64);
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
    if constexpr (SINGLE) {
        // one thread per expert writes its blocks and its padding rows (at most bs-1); the rows
        // and blocks past the padded total are shared out
        if (tid < E) {
            for (int b = s_off[tid] / bs; b < s_off[tid + 1] / bs; ++b) expert_ids[b] = tid;
            for (int r = s_off[tid] + s_cnt[tid]; r < s_off[tid + 1]; ++r) sorted_ids[r] = P;
        }
        for (int b = total / bs + tid; b < nblk; b += NT) expert_ids[b] = -1;
        for (int r = total + tid; r < max_pad; r += NT) sorted_ids[r] = P;
    } else {
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
    }

    // pass A: per-wave counts of each expert over the wave's run of pairs
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        if (run0 + it * 64 >= P) break;  // wave-uniform
        const int p = run0 + it * 64 + lane;
        const bool in = p < P;
        const int e = e_reg[it];
        const bool valid = e >= 0;
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
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        if (run0 + it * 64 >= P) break;  // wave-uniform
        const int p = run0 + it * 64 + lane;
        const bool in = p < P;
        const int e = e_reg[it];
        const bool valid = e >= 0;
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

template <bool SINGLE>
__global__ __launch_bounds__(kThreads) void align_scatter_kernel(
    const int32_t* __restrict__ ids, int P, int E, int bs, const int32_t* __restrict__ ws, int G,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ expert_ids, int32_t* __restrict__ total_out, int32_t* __restrict__ inv, int max_pad) {
    align_scatter_body<SINGLE>(ids, P, E, bs, ws, G, counts, offsets, sorted_ids, expert_ids, total_out, inv,
                               max_pad, blockIdx.x);
}

// Routing and alignment of a small batch (at most kChunkOne pairs and kFusedTokens tokens) in one
// workgroup and one launch: 16 waves route the tokens (one wave per token, up to four tokens per
// wave interleaved), then the workgroup aligns the pairs they wrote.
constexpr int kFusedWaves = 16;
constexpr int kFusedTokens = 64;
template <int EPL>
__global__ __launch_bounds__(64 * kFusedWaves) void route_align_kernel(
    const float* __restrict__ logits, int T, int E, int top_k, int renorm, int32_t* topk_ids, float* topk_w,
    int bs, int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ expert_ids, int32_t* __restrict__ total_out, int32_t* __restrict__ inv, int max_pad) {
    __shared__ int s_ids[kChunkOne];  // the routed expert ids, handed to the alignment in LDS
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (E <= 16 && T > kFusedWaves) {
        // one token per 16-lane row: the 64 tokens in one pass
        route_row_token(logits, wave * 4 + (lane >> 4), T, E, top_k, renorm, topk_ids, topk_w, lane, s_ids);
    } else if (T <= kFusedWaves) {
        if (wave < T) route_tokens<EPL, 1>(logits, wave, 0, T, E, top_k, renorm, topk_ids, topk_w, lane, s_ids);
    } else {
        // four tokens per wave interleaved; two when each lane holds four logits (registers)
        constexpr int NTOK = EPL >= 4 ? 2 : 4;
        for (int t = wave; t < T; t += kFusedWaves * NTOK)
            route_tokens<EPL, NTOK>(logits, t, kFusedWaves, T, E, top_k, renorm, topk_ids, topk_w, lane, s_ids);
    }
    __syncthreads();
    align_scatter_body<true, kFusedWaves>(s_ids, T * top_k, E, bs, nullptr, 1, counts, offsets, sorted_ids,
                                          expert_ids, total_out, inv, max_pad, 0);
}

// Static histogram table of moe_align_noalloc: the [chunks, E] per-chunk counts live here instead
// of in a caller workspace.  Every call overwrites the cells it reads (align_count_kernel writes all
// E counts of each of its chunks before align_scatter_kernel reads them), so the table needs no
// clearing between calls.  Each device holds its own copy for the life of the process.
static __device__ __align__(256) __attribute__((used)) int32_t scratch[kAlignScratchCells];

}  // namespace

hipError_t align_scratch_ptr(int32_t** out) {
    // The array's device address, looked up once per device with that device current.  In host
    // code the name `scratch` is only a stand-in: kernels get this address, never the name.
    static std::mutex mu;
    static int32_t* ptrs[kMaxDevices] = {};
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (ptrs[dev] == nullptr) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (p == nullptr) return hipErrorInvalidSymbol;
        ptrs[dev] = static_cast<int32_t*>(p);
    }
    *out = ptrs[dev];
    return hipSuccess;
}

int align_num_chunks(int64_t num_pairs) {
    const int64_t g = (num_pairs + kChunk - 1) / kChunk;
    return static_cast<int>(g < 1 ? 1 : g);
}

hipError_t launch_align(const int32_t* topk_ids, int P, int E, int bs, int32_t* counts, int32_t* offsets,
                        int32_t* sorted_ids, int32_t* expert_ids, int32_t* total, int32_t* inv, int max_pad,
                        int32_t* workspace, hipStream_t s) {
    if (P <= kChunkOne) {
        align_scatter_kernel<true><<<1, kThreads, 0, s>>>(topk_ids, P, E, bs, workspace, 1, counts, offsets,
                                                          sorted_ids, expert_ids, total, inv, max_pad);
        return hipGetLastError();
    }
    const int G = align_num_chunks(P);
    align_count_kernel<<<G, kThreads, 0, s>>>(topk_ids, P, E, workspace);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    align_scatter_kernel<false><<<G, kThreads, 0, s>>>(topk_ids, P, E, bs, workspace, G, counts, offsets, sorted_ids,
                                                        expert_ids, total, inv, max_pad);
    return hipGetLastError();
}

hipError_t launch_route_align(const float* logits, int T, int E, int top_k, int renorm, int32_t* ids, float* w,
                              int bs, int32_t* counts, int32_t* offsets, int32_t* sorted_ids, int32_t* expert_ids,
                              int32_t* total, int32_t* inv, int max_pad, int32_t* workspace, hipStream_t s) {
    const int P = T * top_k;
    if (P > kChunkOne || T > kFusedTokens) {
        hipError_t err = launch_route(logits, T, E, top_k, renorm, ids, w, s);
        if (err != hipSuccess) return err;
        return launch_align(ids, P, E, bs, counts, offsets, sorted_ids, expert_ids, total, inv, max_pad, workspace, s);
    }
    const int epl = (E + 63) / 64;
    switch (epl) {
        case 1: route_align_kernel<1><<<1, 64 * kFusedWaves, 0, s>>>(logits, T, E, top_k, renorm, ids, w, bs, counts, offsets, sorted_ids, expert_ids, total, inv, max_pad); break;
        case 2: route_align_kernel<2><<<1, 64 * kFusedWaves, 0, s>>>(logits, T, E, top_k, renorm, ids, w, bs, counts, offsets, sorted_ids, expert_ids, total, inv, max_pad); break;
        case 3: route_align_kernel<3><<<1, 64 * kFusedWaves, 0, s>>>(logits, T, E, top_k, renorm, ids, w, bs, counts, offsets, sorted_ids, expert_ids, total, inv, max_pad); break;
        default: route_align_kernel<4><<<1, 64 * kFusedWaves, 0, s>>>(logits, T, E, top_k, renorm, ids, w, bs, counts, offsets, sorted_ids, expert_ids, total, inv, max_pad); break;
    }
    return hipGetLastError();
}

}  // namespace moe
