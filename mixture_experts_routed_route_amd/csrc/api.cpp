// C ABI of the MoE expert path (declared in include/moe_mi355x.h): host-side argument
// checks, pure host helpers, and the launches of the gfx950 kernels.
#include "../../include/moe_mi355x.h"
#include "../../include/moe_probes.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "launchers.h"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

moe_status ok() { return MOE_OK; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE(cond, ...)                                 \
    do {                                                   \
        if (!(cond)) return fail(MOE_EINVAL, __VA_ARGS__); \
    } while (0)

#define REQUIRE_PTR(who, p)                                                                 \
    do {                                                                                    \
        if ((p) == nullptr) return fail(MOE_EINVAL, "%s: %s is NULL", who, #p);             \
        if (!aligned16(p)) return fail(MOE_EINVAL, "%s: %s is not 16-byte aligned", who, #p); \
    } while (0)

moe_status launched(const char* who, hipError_t err) {
    if (err != hipSuccess) return fail(MOE_ELAUNCH, "%s: launch failed: %s", who, hipGetErrorString(err));
    return ok();
}

bool valid_block_size(int bs) { return bs == 16 || bs == 32 || bs == 64 || bs == 128; }

int64_t max_padded(int64_t P, int64_t E, int64_t bs) { return ((P + E * (bs - 1) + bs - 1) / bs) * bs; }

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_last_error.c_str(); }

int32_t moe_abi_version(void) { return 3; }

int64_t moe_align_max_padded(int64_t num_pairs, int32_t num_experts, int32_t block_size) {
    if (num_pairs < 0 || num_experts < 1 || block_size < 1) return -1;
    return max_padded(num_pairs, num_experts, block_size);
}

int64_t moe_grouped_gemm_workspace_bytes(void) { return moe::gemm_bf16_workspace_bytes(); }

int64_t moe_align_workspace_bytes(int64_t num_pairs, int32_t num_experts) {
    if (num_pairs < 0 || num_experts < 1) return -1;
    return static_cast<int64_t>(moe::align_num_chunks(num_pairs)) * num_experts * 4;
}

moe_status moe_check_group_arrays(int32_t num_experts, const int64_t* lens, const char* const* names,
                                  int32_t n_arrays, const int32_t* offsets, int64_t offsets_len) {
    const char* who = "moe_check_group_arrays";
    REQUIRE(num_experts >= 0, "%s: num_experts %d is negative", who, num_experts);
    REQUIRE(n_arrays >= 0 && (n_arrays == 0 || (lens && names)), "%s: per-expert arrays not given", who);
    if (offsets_len != static_cast<int64_t>(num_experts) + 1)
        return fail(MOE_EINVAL, "expert_offsets len %lld != num_experts+1 %lld", static_cast<long long>(offsets_len),
                    static_cast<long long>(num_experts) + 1);
    for (int i = 0; i < n_arrays; ++i)
        if (lens[i] != num_experts)
            return fail(MOE_EINVAL, "%s len %lld != num_experts %d", names[i] ? names[i] : "?",
                        static_cast<long long>(lens[i]), num_experts);
    REQUIRE(offsets != nullptr, "%s: offsets is NULL", who);
    if (offsets[0] < 0) return fail(MOE_EINVAL, "expert_offsets[0] = %d is negative", offsets[0]);
    for (int64_t i = 0; i + 1 < offsets_len; ++i)
        if (offsets[i + 1] < offsets[i])
            return fail(MOE_EINVAL,
                        "expert_offsets is not non-decreasing (%d then %d): a group would have a negative row count",
                        offsets[i], offsets[i + 1]);
    return ok();
}

moe_status moe_lora_pack_tables(const int32_t* ids, const uint64_t* a, const uint64_t* b, const float* s,
                                int32_t n, uint64_t* a_out, uint64_t* b_out, float* s_out, int32_t cap,
                                int32_t* n_tab) {
    const char* who = "moe_lora_pack_tables";
    REQUIRE(n_tab != nullptr, "%s: n_tab is NULL", who);
    REQUIRE(n >= 0, "%s: n %d is negative", who, n);
    if (n == 0) {
        *n_tab = 0;
        return ok();
    }
    REQUIRE(ids && a && b && s, "%s: an input array is NULL", who);
    int32_t mx = -1;
    for (int i = 0; i < n; ++i) {
        REQUIRE(ids[i] >= 0 && ids[i] <= 65535, "%s: ids[%d] = %d is not a u16 expert id", who, i, ids[i]);
        mx = ids[i] > mx ? ids[i] : mx;
    }
    const int32_t len = mx + 1;
    REQUIRE(len <= cap, "%s: table length %d exceeds cap %d", who, len, cap);
    REQUIRE(a_out && b_out && s_out, "%s: an output array is NULL", who);
    for (int i = 0; i < len; ++i) { a_out[i] = 0; b_out[i] = 0; s_out[i] = 0.0f; }
    for (int i = 0; i < n; ++i) { a_out[ids[i]] = a[i]; b_out[ids[i]] = b[i]; s_out[ids[i]] = s[i]; }
    *n_tab = len;
    return ok();
}

int64_t moe_lora_window_tiles(int64_t row_offset, int64_t row_end) {
    const int64_t n = row_end > row_offset ? row_end - row_offset : 0;
    const int64_t t = (n + 63) / 64;
    return t < 1 ? 1 : t;
}

int64_t moe_lora_windows(int64_t total_rows, int64_t cap, int64_t* starts, int64_t* ends, int64_t max_windows) {
    if (cap <= 0 || total_rows < 0) return -1;
    int64_t n = 0;
    for (int64_t s0 = 0; s0 < total_rows; s0 += cap, ++n) {
        if (n < max_windows && starts && ends) {
            starts[n] = s0;
            ends[n] = s0 + cap < total_rows ? s0 + cap : total_rows;
        }
    }
    return n;
}

moe_status moe_route(const float* logits, int32_t num_tokens, int32_t num_experts, int32_t top_k,
                     int32_t renormalize, int32_t* topk_ids, float* topk_w, moe_stream stream) {
    const char* who = "moe_route";
    REQUIRE(num_tokens >= 0, "%s: num_tokens %d is negative", who, num_tokens);
    REQUIRE(num_experts >= 1, "%s: num_experts %d < 1", who, num_experts);
    if (num_experts > 256)
        return fail(MOE_EUNSUPPORTED, "%s: num_experts=%d > 256", who, num_experts);
    REQUIRE(top_k >= 1 && top_k <= num_experts, "%s: top_k %d not in [1, num_experts=%d]", who, top_k,
            num_experts);
    if (num_tokens == 0) return ok();
    REQUIRE_PTR(who, logits);
    REQUIRE_PTR(who, topk_ids);
    REQUIRE_PTR(who, topk_w);
    return launched(who, moe::launch_route(logits, num_tokens, num_experts, top_k, renormalize ? 1 : 0, topk_ids,
                                           topk_w, static_cast<hipStream_t>(stream)));
}

moe_status moe_align(const int32_t* topk_ids, int64_t num_pairs, int32_t num_experts, int32_t block_size,
                     int32_t* counts, int32_t* expert_offsets, int32_t* sorted_ids, int32_t* expert_ids,
                     int32_t* total_padded, int32_t* inv_sorted, int64_t max_pad, void* workspace,
                     int64_t workspace_bytes, moe_stream stream) {
    const char* who = "moe_align";
    REQUIRE(num_pairs >= 0 && num_pairs < INT32_MAX, "%s: num_pairs %lld out of range", who,
            static_cast<long long>(num_pairs));
    REQUIRE(num_experts >= 1, "%s: num_experts %d < 1", who, num_experts);
    if (num_experts > 256)
        return fail(MOE_EUNSUPPORTED, "%s: num_experts=%d exceeds MAX_NUM_EXPERTS=256", who, num_experts);
    REQUIRE(valid_block_size(block_size), "%s: block_size %d not in {16,32,64,128}", who, block_size);
    const int64_t need = max_padded(num_pairs, num_experts, block_size);
    REQUIRE(max_pad >= need, "%s: max_pad %lld < required %lld", who, static_cast<long long>(max_pad),
            static_cast<long long>(need));
    REQUIRE(max_pad % block_size == 0, "%s: max_pad %lld is not a multiple of block_size %d", who,
            static_cast<long long>(max_pad), block_size);
    REQUIRE(max_pad < INT32_MAX, "%s: max_pad too large", who);
    const int64_t ws_need = moe_align_workspace_bytes(num_pairs, num_experts);
    REQUIRE(workspace_bytes >= ws_need, "%s: workspace_bytes %lld < required %lld", who,
            static_cast<long long>(workspace_bytes), static_cast<long long>(ws_need));
    if (num_pairs > 0) {
        REQUIRE_PTR(who, topk_ids);
        REQUIRE_PTR(who, inv_sorted);
    }
    REQUIRE_PTR(who, counts);
    REQUIRE_PTR(who, expert_offsets);
    REQUIRE_PTR(who, sorted_ids);
    REQUIRE_PTR(who, expert_ids);
    REQUIRE_PTR(who, total_padded);
    REQUIRE_PTR(who, workspace);
    return launched(who, moe::launch_align(topk_ids, static_cast<int>(num_pairs), num_experts, block_size, counts,
                                           expert_offsets, sorted_ids, expert_ids, total_padded, inv_sorted,
                                           static_cast<int>(max_pad), static_cast<int32_t*>(workspace),
                                           static_cast<hipStream_t>(stream)));
}

moe_status moe_align_noalloc(const int32_t* topk_ids, int64_t num_pairs, int32_t num_experts, int32_t block_size,
                             int32_t* counts, int32_t* expert_offsets, int32_t* sorted_ids, int32_t* expert_ids,
                             int32_t* total_padded, int32_t* inv_sorted, int64_t max_pad, moe_stream stream) {
    const char* who = "moe_align_noalloc";
    REQUIRE(num_pairs >= 0 && num_pairs < INT32_MAX, "%s: num_pairs %lld out of range", who,
            static_cast<long long>(num_pairs));
    REQUIRE(num_experts >= 1, "%s: num_experts %d < 1", who, num_experts);
    if (num_experts > 256)
        return fail(MOE_EUNSUPPORTED, "%s: num_experts=%d exceeds MAX_NUM_EXPERTS=256", who, num_experts);
    const int64_t cells = static_cast<int64_t>(moe::align_num_chunks(num_pairs)) * num_experts;
    if (cells > moe::kAlignScratchCells)
        return fail(MOE_EUNSUPPORTED,
                    "%s: ceil(num_pairs/512)*num_experts = %lld histogram cells exceed the static table of %lld "
                    "(use moe_align with a workspace)",
                    who, static_cast<long long>(cells), static_cast<long long>(moe::kAlignScratchCells));
    REQUIRE(valid_block_size(block_size), "%s: block_size %d not in {16,32,64,128}", who, block_size);
    const int64_t need = max_padded(num_pairs, num_experts, block_size);
    REQUIRE(max_pad >= need, "%s: max_pad %lld < required %lld", who, static_cast<long long>(max_pad),
            static_cast<long long>(need));
    REQUIRE(max_pad % block_size == 0, "%s: max_pad %lld is not a multiple of block_size %d", who,
            static_cast<long long>(max_pad), block_size);
    REQUIRE(max_pad < INT32_MAX, "%s: max_pad too large", who);
    if (num_pairs > 0) {
        REQUIRE_PTR(who, topk_ids);
        REQUIRE_PTR(who, inv_sorted);
    }
    REQUIRE_PTR(who, counts);
    REQUIRE_PTR(who, expert_offsets);
    REQUIRE_PTR(who, sorted_ids);
    REQUIRE_PTR(who, expert_ids);
    REQUIRE_PTR(who, total_padded);
    int32_t* table = nullptr;
    const hipError_t err = moe::align_scratch_ptr(&table);
    if (err != hipSuccess)
        return fail(MOE_ELAUNCH, "%s: static histogram table not found on this device: %s", who, hipGetErrorString(err));
    return launched(who, moe::launch_align(topk_ids, static_cast<int>(num_pairs), num_experts, block_size, counts,
                                           expert_offsets, sorted_ids, expert_ids, total_padded, inv_sorted,
                                           static_cast<int>(max_pad), table, static_cast<hipStream_t>(stream)));
}

moe_status moe_route_align(const float* logits, int32_t num_tokens, int32_t num_experts, int32_t top_k,
                           int32_t renormalize, int32_t* topk_ids, float* topk_w, int32_t block_size,
                           int32_t* counts, int32_t* expert_offsets, int32_t* sorted_ids, int32_t* expert_ids,
                           int32_t* total_padded, int32_t* inv_sorted, int64_t max_pad, void* workspace,
                           int64_t workspace_bytes, moe_stream stream) {
    const char* who = "moe_route_align";
    REQUIRE(num_tokens >= 0, "%s: num_tokens %d is negative", who, num_tokens);
    REQUIRE(num_experts >= 1, "%s: num_experts %d < 1", who, num_experts);
    if (num_experts > 256)
        return fail(MOE_EUNSUPPORTED, "%s: num_experts=%d > 256", who, num_experts);
    REQUIRE(top_k >= 1 && top_k <= num_experts, "%s: top_k %d not in [1, num_experts=%d]", who, top_k,
            num_experts);
    const int64_t num_pairs = static_cast<int64_t>(num_tokens) * top_k;
    REQUIRE(num_pairs < INT32_MAX, "%s: num_tokens*top_k %lld out of range", who,
            static_cast<long long>(num_pairs));
    REQUIRE(valid_block_size(block_size), "%s: block_size %d not in {16,32,64,128}", who, block_size);
    const int64_t need = max_padded(num_pairs, num_experts, block_size);
    REQUIRE(max_pad >= need, "%s: max_pad %lld < required %lld", who, static_cast<long long>(max_pad),
            static_cast<long long>(need));
    REQUIRE(max_pad % block_size == 0, "%s: max_pad %lld is not a multiple of block_size %d", who,
            static_cast<long long>(max_pad), block_size);
    REQUIRE(max_pad < INT32_MAX, "%s: max_pad too large", who);
    const int64_t ws_need = moe_align_workspace_bytes(num_pairs, num_experts);
    REQUIRE(workspace_bytes >= ws_need, "%s: workspace_bytes %lld < required %lld", who,
            static_cast<long long>(workspace_bytes), static_cast<long long>(ws_need));
    if (num_tokens > 0) {
        REQUIRE_PTR(who, logits);
        REQUIRE_PTR(who, topk_ids);
        REQUIRE_PTR(who, topk_w);
        REQUIRE_PTR(who, inv_sorted);
    }
    REQUIRE_PTR(who, counts);
    REQUIRE_PTR(who, expert_offsets);
    REQUIRE_PTR(who, sorted_ids);
    REQUIRE_PTR(who, expert_ids);
    REQUIRE_PTR(who, total_padded);
    REQUIRE_PTR(who, workspace);
    if (num_tokens == 0)
        return launched(who, moe::launch_align(nullptr, 0, num_experts, block_size, counts, expert_offsets,
                                               sorted_ids, expert_ids, total_padded, inv_sorted,
                                               static_cast<int>(max_pad), static_cast<int32_t*>(workspace),
                                               static_cast<hipStream_t>(stream)));
    return launched(who, moe::launch_route_align(logits, num_tokens, num_experts, top_k, renormalize ? 1 : 0,
                                                 topk_ids, topk_w, block_size, counts, expert_offsets, sorted_ids,
                                                 expert_ids, total_padded, inv_sorted, static_cast<int>(max_pad),
                                                 static_cast<int32_t*>(workspace),
                                                 static_cast<hipStream_t>(stream)));
}

moe_status moe_grouped_gemm(int32_t op, const uint16_t* a, const moe_weight* w0, const moe_weight* w1,
                            uint16_t* c, const int32_t* sorted_ids, const int32_t* expert_ids,
                            const int32_t* expert_offsets, int64_t num_pairs, int32_t top_k,
                            int32_t num_experts, int32_t n, int32_t k, int32_t block_size, int64_t max_pad,
                            void* workspace, int64_t workspace_bytes, moe_stream stream) {
    const char* who = "moe_grouped_gemm";
    REQUIRE(op == MOE_OP_GATE_UP_SILU || op == MOE_OP_DOWN || op == MOE_OP_GATHER, "%s: unknown op %d", who, op);
    const bool gate_up = op == MOE_OP_GATE_UP_SILU;
    const bool by_token = op != MOE_OP_DOWN;  // a is the token-major x
    REQUIRE(num_pairs >= 0 && num_pairs < INT32_MAX, "%s: num_pairs out of range", who);
    REQUIRE(top_k >= 1, "%s: top_k %d < 1", who, top_k);
    REQUIRE(num_pairs % top_k == 0, "%s: num_pairs %lld is not a multiple of top_k %d", who,
            static_cast<long long>(num_pairs), top_k);
    REQUIRE(num_experts >= 1, "%s: num_experts %d < 1", who, num_experts);
    if (num_experts > 256) return fail(MOE_EUNSUPPORTED, "%s: num_experts=%d > 256", who, num_experts);
    REQUIRE(valid_block_size(block_size), "%s: block_size %d not in {16,32,64,128}", who, block_size);
    REQUIRE(n >= 8 && n % 8 == 0, "%s: n %d must be a positive multiple of 8", who, n);
    REQUIRE(k >= 8 && k % 8 == 0, "%s: k %d must be a positive multiple of 8", who, k);
    REQUIRE(max_pad >= max_padded(num_pairs, num_experts, block_size) && max_pad % block_size == 0 &&
                max_pad < INT32_MAX,
            "%s: max_pad %lld must be >= %lld and a multiple of block_size", who, static_cast<long long>(max_pad),
            static_cast<long long>(max_padded(num_pairs, num_experts, block_size)));
    REQUIRE(w0 != nullptr, "%s: w0 is NULL", who);
    if (gate_up) REQUIRE(w1 != nullptr, "%s: MOE_OP_GATE_UP_SILU needs w1 (up)", who);
    else REQUIRE(w1 == nullptr, "%s: op %d takes no w1", who, op);
    REQUIRE(w0->type == MOE_W_BF16 || w0->type == MOE_W_INT4_GPTQ, "%s: w0 has unsupported type %d", who,
            w0->type);
    if (w1) REQUIRE(w1->type == w0->type, "%s: w0 and w1 have different types", who);
    if (workspace != nullptr) {
        const int64_t need = moe_grouped_gemm_workspace_bytes();
        REQUIRE_PTR(who, workspace);
        REQUIRE(need > 0 && workspace_bytes >= need, "%s: workspace_bytes %lld < required %lld", who,
                static_cast<long long>(workspace_bytes), static_cast<long long>(need));
    }
    if (num_pairs == 0) return ok();
    REQUIRE_PTR(who, a);
    REQUIRE_PTR(who, c);
    REQUIRE_PTR(who, sorted_ids);
    REQUIRE_PTR(who, w0->data);
    if (w1) REQUIRE_PTR(who, w1->data);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int P = static_cast<int>(num_pairs);
    if (w0->type == MOE_W_BF16) {
        REQUIRE_PTR(who, expert_offsets);
        // the kernel addresses a's rows and each expert matrix with 32-bit byte offsets
        const int64_t a_rows = by_token ? num_pairs / top_k : max_pad;
        if (a_rows * k * 2 > INT64_C(0xffffffff) || static_cast<int64_t>(n) * k * 2 > INT64_C(0xffffffff))
            return fail(MOE_EUNSUPPORTED, "%s: bf16 a (%lld rows) or an expert matrix (%d x %d) exceeds 4 GiB", who,
                        static_cast<long long>(a_rows), n, k);
        return launched(who, moe::launch_gemm_bf16(op, a, static_cast<const uint16_t*>(w0->data),
                                                   w1 ? static_cast<const uint16_t*>(w1->data) : nullptr, c,
                                                   sorted_ids, expert_offsets, P, top_k, num_experts, n, k,
                                                   static_cast<int>(max_pad), workspace, workspace_bytes, s));
    }
    const int G = w0->group_size;
    REQUIRE(G == 32 || G == 64 || G == 128 || G == 256, "%s: group_size %d not in {32,64,128,256}", who, G);
    if (w1) REQUIRE(w1->group_size == G, "%s: w0 and w1 group sizes differ", who);
    REQUIRE(k % G == 0, "%s: k %d is not a multiple of group_size %d", who, k, G);
    REQUIRE(n % 64 == 0, "%s: int4 weights need n %% 64 == 0 (n = %d)", who, n);
    REQUIRE_PTR(who, expert_ids);
    REQUIRE_PTR(who, w0->scales);
    REQUIRE_PTR(who, w0->qzeros);
    if (w1) {
        REQUIRE_PTR(who, w1->scales);
        REQUIRE_PTR(who, w1->qzeros);
    }
    return launched(who, moe::launch_gemm_int4(
                             op, a, static_cast<const int32_t*>(w0->data), static_cast<const uint16_t*>(w0->scales),
                             w0->qzeros, w1 ? static_cast<const int32_t*>(w1->data) : nullptr,
                             w1 ? static_cast<const uint16_t*>(w1->scales) : nullptr,
                             w1 ? w1->qzeros : nullptr, G, c, sorted_ids, expert_ids, P, top_k, num_experts, n, k,
                             block_size, static_cast<int>(max_pad), s));
}

moe_status moe_lora_fold(const uint16_t* x, uint16_t* base, const uint64_t* a_table, const uint64_t* b_table,
                         const float* scale_table, int32_t n_tab, int32_t n_adapters, int32_t k_in, int32_t n_out,
                         int32_t max_rank, const int32_t* expert_offsets, int32_t num_experts, const int32_t* sorted_ids,
                         int64_t num_pairs, int32_t top_k, const int32_t* row_adapter, uint16_t* xa, int64_t cap,
                         int64_t row_offset, int64_t row_end, int64_t max_pad, int32_t x_gather,
                         moe_stream stream) {
    const char* who = "moe_lora_fold";
    REQUIRE(x_gather == 0 || x_gather == 1, "%s: x_gather %d not 0 or 1", who, x_gather);
    REQUIRE(num_experts >= 1, "%s: num_experts %d < 1", who, num_experts);
    if (num_experts > 256) return fail(MOE_EUNSUPPORTED, "%s: num_experts=%d > 256", who, num_experts);
    REQUIRE(n_tab >= 0 && n_tab <= num_experts, "%s: n_tab %d not in [0, num_experts=%d]", who, n_tab,
            num_experts);
    REQUIRE(n_adapters >= 1 && n_adapters <= 65536, "%s: n_adapters %d not in [1, 65536]", who, n_adapters);
    REQUIRE(k_in >= 8 && k_in % 8 == 0, "%s: k_in %d must be a positive multiple of 8", who, k_in);
    REQUIRE(n_out >= 8 && n_out % 8 == 0, "%s: n_out %d must be a positive multiple of 8", who, n_out);
    REQUIRE(max_rank >= 32 && max_rank <= 128 && max_rank % 32 == 0, "%s: max_rank %d not in {32,64,96,128}", who,
            max_rank);
    REQUIRE(top_k >= 1, "%s: top_k %d < 1", who, top_k);
    REQUIRE(num_pairs >= 0 && num_pairs < INT32_MAX && num_pairs % top_k == 0, "%s: bad num_pairs %lld", who,
            static_cast<long long>(num_pairs));
    REQUIRE(max_pad >= 0 && max_pad < INT32_MAX, "%s: bad max_pad", who);
    REQUIRE(row_offset >= 0 && row_end <= max_pad, "%s: window [%lld, %lld) outside [0, max_pad=%lld)", who,
            static_cast<long long>(row_offset), static_cast<long long>(row_end), static_cast<long long>(max_pad));
    REQUIRE(cap >= row_end - row_offset, "%s: cap %lld < window rows %lld", who, static_cast<long long>(cap),
            static_cast<long long>(row_end - row_offset));
    if (row_end <= row_offset || n_tab == 0 || num_pairs == 0) return ok();
    REQUIRE_PTR(who, x);
    REQUIRE_PTR(who, base);
    REQUIRE_PTR(who, a_table);
    REQUIRE_PTR(who, b_table);
    REQUIRE_PTR(who, scale_table);
    REQUIRE_PTR(who, expert_offsets);
    REQUIRE_PTR(who, sorted_ids);
    REQUIRE_PTR(who, xa);
    if (row_adapter) REQUIRE_PTR(who, row_adapter);
    return launched(who, moe::launch_lora_fold(x, base, a_table, b_table, scale_table, n_tab, n_adapters, k_in, n_out,
                                               max_rank,
                                               expert_offsets, num_experts, sorted_ids, static_cast<int>(num_pairs),
                                               top_k, row_adapter, xa, row_offset, row_end, x_gather,
                                               static_cast<hipStream_t>(stream)));
}

moe_status moe_grouped_gemm_gate_up_lora(const uint16_t* x, const moe_weight* w_gate, const moe_weight* w_up,
                                         uint16_t* hs, const int32_t* sorted_ids, const int32_t* expert_offsets,
                                         int64_t num_pairs, int32_t top_k, int32_t num_experts, int32_t n, int32_t k,
                                         int32_t block_size, int64_t max_pad, const uint64_t* a_gate,
                                         const uint64_t* b_gate, const float* s_gate, int32_t n_tab_gate,
                                         const uint64_t* a_up, const uint64_t* b_up, const float* s_up,
                                         int32_t n_tab_up, int32_t n_adapters, int32_t max_rank,
                                         const int32_t* row_adapter,
                                         uint16_t* xa, void* workspace, int64_t workspace_bytes,
                                         moe_stream stream) {
    const char* who = "moe_grouped_gemm_gate_up_lora";
    REQUIRE(num_pairs >= 0 && num_pairs < INT32_MAX, "%s: num_pairs out of range", who);
    REQUIRE(top_k >= 1 && num_pairs % top_k == 0, "%s: num_pairs %lld is not a multiple of top_k %d", who,
            static_cast<long long>(num_pairs), top_k);
    REQUIRE(num_experts >= 1, "%s: num_experts %d < 1", who, num_experts);
    if (num_experts > 256) return fail(MOE_EUNSUPPORTED, "%s: num_experts=%d > 256", who, num_experts);
    REQUIRE(valid_block_size(block_size), "%s: block_size %d not in {16,32,64,128}", who, block_size);
    REQUIRE(n >= 8 && n % 8 == 0, "%s: n %d must be a positive multiple of 8", who, n);
    REQUIRE(k >= 8 && k % 8 == 0, "%s: k %d must be a positive multiple of 8", who, k);
    REQUIRE(max_pad >= max_padded(num_pairs, num_experts, block_size) && max_pad % block_size == 0 &&
                max_pad < INT32_MAX,
            "%s: max_pad %lld must be >= %lld and a multiple of block_size", who, static_cast<long long>(max_pad),
            static_cast<long long>(max_padded(num_pairs, num_experts, block_size)));
    REQUIRE(w_gate != nullptr && w_up != nullptr, "%s: w_gate and w_up are required", who);
    if (w_gate->type != MOE_W_BF16 || w_up->type != MOE_W_BF16)
        return fail(MOE_EUNSUPPORTED, "%s: the fused gate/up LoRA takes bf16 weights only", who);
    REQUIRE(max_rank >= 32 && max_rank <= 128 && max_rank % 32 == 0, "%s: max_rank %d not in {32,64,96,128}", who,
            max_rank);
    REQUIRE(n_tab_gate >= 0 && n_tab_gate <= num_experts && n_tab_up >= 0 && n_tab_up <= num_experts,
            "%s: table lengths must be in [0, num_experts=%d]", who, num_experts);
    REQUIRE(n_adapters >= 1 && n_adapters <= 65536, "%s: n_adapters %d not in [1, 65536]", who, n_adapters);
    if (workspace != nullptr) {
        const int64_t need = moe_grouped_gemm_workspace_bytes();
        REQUIRE_PTR(who, workspace);
        REQUIRE(workspace_bytes >= need, "%s: workspace_bytes %lld < required %lld", who,
                static_cast<long long>(workspace_bytes), static_cast<long long>(need));
    }
    if (num_pairs == 0) return ok();
    REQUIRE_PTR(who, x);
    REQUIRE_PTR(who, hs);
    REQUIRE_PTR(who, sorted_ids);
    REQUIRE_PTR(who, expert_offsets);
    REQUIRE_PTR(who, w_gate->data);
    REQUIRE_PTR(who, w_up->data);
    REQUIRE_PTR(who, xa);
    if (n_tab_gate > 0) {
        REQUIRE_PTR(who, a_gate);
        REQUIRE_PTR(who, b_gate);
        REQUIRE_PTR(who, s_gate);
    }
    if (n_tab_up > 0) {
        REQUIRE_PTR(who, a_up);
        REQUIRE_PTR(who, b_up);
        REQUIRE_PTR(who, s_up);
    }
    if (row_adapter) REQUIRE_PTR(who, row_adapter);
    const int64_t a_rows = num_pairs / top_k;
    if (a_rows * k * 2 > INT64_C(0xffffffff) || static_cast<int64_t>(n) * k * 2 > INT64_C(0xffffffff))
        return fail(MOE_EUNSUPPORTED, "%s: x or an expert matrix exceeds 4 GiB", who);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int P = static_cast<int>(num_pairs);
    uint16_t* xa_up = xa + max_pad * max_rank;
    hipError_t err = moe::launch_lora_shrink(x, a_gate, b_gate, n_tab_gate, n_adapters, k, max_rank, expert_offsets,
                                             num_experts, sorted_ids, P, top_k, row_adapter, xa, 0, max_pad, 1, s);
    if (err == hipSuccess)
        err = moe::launch_lora_shrink(x, a_up, b_up, n_tab_up, n_adapters, k, max_rank, expert_offsets, num_experts,
                                      sorted_ids, P, top_k, row_adapter, xa_up, 0, max_pad, 1, s);
    if (err != hipSuccess) return launched(who, err);
    moe::GateUpLora lora{};
    lora.xa[0] = xa;
    lora.xa[1] = xa_up;
    lora.a_tab[0] = a_gate;
    lora.a_tab[1] = a_up;
    lora.b_tab[0] = b_gate;
    lora.b_tab[1] = b_up;
    lora.s_tab[0] = s_gate;
    lora.s_tab[1] = s_up;
    lora.n_tab[0] = n_tab_gate;
    lora.n_tab[1] = n_tab_up;
    lora.n_ad = n_adapters;
    lora.rank = max_rank;
    lora.row_adapter = row_adapter;
    return launched(who, moe::launch_gemm_bf16(moe::kOpGateUpSilu, x, static_cast<const uint16_t*>(w_gate->data),
                                               static_cast<const uint16_t*>(w_up->data), hs, sorted_ids,
                                               expert_offsets, P, top_k, num_experts, n, k,
                                               static_cast<int>(max_pad), workspace, workspace_bytes, s, &lora));
}

moe_status moe_grouped_gemm_down_lora(const uint16_t* hs, const moe_weight* w_down, uint16_t* ys,
                                      const int32_t* sorted_ids, const int32_t* expert_offsets, int64_t num_pairs,
                                      int32_t top_k, int32_t num_experts, int32_t n, int32_t k, int32_t block_size,
                                      int64_t max_pad, const uint64_t* a_table, const uint64_t* b_table,
                                      const float* scale_table, int32_t n_tab, int32_t n_adapters, int32_t max_rank,
                                      const int32_t* row_adapter, uint16_t* xa, void* workspace,
                                      int64_t workspace_bytes, moe_stream stream) {
    const char* who = "moe_grouped_gemm_down_lora";
    REQUIRE(num_pairs >= 0 && num_pairs < INT32_MAX, "%s: num_pairs out of range", who);
    REQUIRE(top_k >= 1 && num_pairs % top_k == 0, "%s: num_pairs %lld is not a multiple of top_k %d", who,
            static_cast<long long>(num_pairs), top_k);
    REQUIRE(num_experts >= 1, "%s: num_experts %d < 1", who, num_experts);
    if (num_experts > 256) return fail(MOE_EUNSUPPORTED, "%s: num_experts=%d > 256", who, num_experts);
    REQUIRE(valid_block_size(block_size), "%s: block_size %d not in {16,32,64,128}", who, block_size);
    REQUIRE(n >= 8 && n % 8 == 0, "%s: n %d must be a positive multiple of 8", who, n);
    REQUIRE(k >= 8 && k % 8 == 0, "%s: k %d must be a positive multiple of 8", who, k);
    REQUIRE(max_pad >= max_padded(num_pairs, num_experts, block_size) && max_pad % block_size == 0 &&
                max_pad < INT32_MAX,
            "%s: max_pad %lld must be >= %lld and a multiple of block_size", who, static_cast<long long>(max_pad),
            static_cast<long long>(max_padded(num_pairs, num_experts, block_size)));
    REQUIRE(w_down != nullptr, "%s: w_down is required", who);
    if (w_down->type != MOE_W_BF16)
        return fail(MOE_EUNSUPPORTED, "%s: the fused down LoRA takes bf16 weights only", who);
    REQUIRE(max_rank >= 32 && max_rank <= 128 && max_rank % 32 == 0, "%s: max_rank %d not in {32,64,96,128}", who,
            max_rank);
    REQUIRE(n_tab >= 0 && n_tab <= num_experts, "%s: n_tab %d not in [0, num_experts=%d]", who, n_tab, num_experts);
    REQUIRE(n_adapters >= 1 && n_adapters <= 65536, "%s: n_adapters %d not in [1, 65536]", who, n_adapters);
    if (workspace != nullptr) {
        const int64_t need = moe_grouped_gemm_workspace_bytes();
        REQUIRE_PTR(who, workspace);
        REQUIRE(workspace_bytes >= need, "%s: workspace_bytes %lld < required %lld", who,
                static_cast<long long>(workspace_bytes), static_cast<long long>(need));
    }
    if (num_pairs == 0) return ok();
    REQUIRE_PTR(who, hs);
    REQUIRE_PTR(who, ys);
    REQUIRE_PTR(who, sorted_ids);
    REQUIRE_PTR(who, expert_offsets);
    REQUIRE_PTR(who, w_down->data);
    REQUIRE_PTR(who, xa);
    if (n_tab > 0) {
        REQUIRE_PTR(who, a_table);
        REQUIRE_PTR(who, b_table);
        REQUIRE_PTR(who, scale_table);
    }
    if (row_adapter) REQUIRE_PTR(who, row_adapter);
    // the kernel addresses Hs rows and each expert matrix with 32-bit byte offsets
    if (max_pad * k * 2 > INT64_C(0xffffffff) || static_cast<int64_t>(n) * k * 2 > INT64_C(0xffffffff))
        return fail(MOE_EUNSUPPORTED, "%s: hs or an expert matrix exceeds 4 GiB", who);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const int P = static_cast<int>(num_pairs);
    hipError_t err = hipSuccess;
    if (n_tab > 0)
        err = moe::launch_lora_shrink(hs, a_table, b_table, n_tab, n_adapters, k, max_rank, expert_offsets,
                                      num_experts, sorted_ids, P, top_k, row_adapter, xa, 0, max_pad, 0, s);
    if (err != hipSuccess) return launched(who, err);
    moe::GateUpLora lora{};
    for (int i = 0; i < 2; ++i) {  // the one projection's tables in both slots (the two column halves)
        lora.xa[i] = xa;
        lora.a_tab[i] = a_table;
        lora.b_tab[i] = b_table;
        lora.s_tab[i] = scale_table;
        lora.n_tab[i] = n_tab;
    }
    lora.n_ad = n_adapters;
    lora.rank = max_rank;
    lora.row_adapter = row_adapter;
    return launched(who, moe::launch_gemm_bf16(moe::kOpDown, hs, static_cast<const uint16_t*>(w_down->data), nullptr,
                                               ys, sorted_ids, expert_offsets, P, top_k, num_experts, n, k,
                                               static_cast<int>(max_pad), workspace, workspace_bytes, s,
                                               n_tab > 0 ? &lora : nullptr));
}

moe_status moe_quantize_fp8(const uint16_t* x, int64_t rows, int32_t k, const int32_t* sorted_ids,
                            int64_t num_pairs, uint8_t* q, float* scale, moe_stream stream) {
    const char* who = "moe_quantize_fp8";
    REQUIRE(k >= 16 && k % 16 == 0, "%s: k %d must be a positive multiple of 16", who, k);
    REQUIRE(rows >= 0 && rows < INT32_MAX, "%s: rows %lld out of range", who, static_cast<long long>(rows));
    REQUIRE(num_pairs >= 0 && num_pairs < INT32_MAX, "%s: num_pairs out of range", who);
    if (rows == 0) return ok();
    REQUIRE_PTR(who, x);
    REQUIRE_PTR(who, q);
    REQUIRE_PTR(who, scale);
    if (sorted_ids) REQUIRE_PTR(who, sorted_ids);
    return launched(who, moe::launch_quantize_fp8(x, rows, k, sorted_ids, static_cast<int>(num_pairs), q, scale,
                                                  static_cast<hipStream_t>(stream)));
}

moe_status moe_grouped_gemm_fp8(int32_t op, const uint8_t* a, const float* a_scale, const moe_weight* w0,
                                const moe_weight* w1, uint16_t* c, const int32_t* sorted_ids,
                                const int32_t* expert_offsets, int64_t num_pairs, int32_t top_k,
                                int32_t num_experts, int32_t n, int32_t k, int32_t block_size, int64_t max_pad,
                                void* workspace, int64_t workspace_bytes, moe_stream stream) {
    const char* who = "moe_grouped_gemm_fp8";
    REQUIRE(op == MOE_OP_GATE_UP_SILU || op == MOE_OP_DOWN, "%s: op %d not GATE_UP_SILU or DOWN", who, op);
    const bool gate_up = op == MOE_OP_GATE_UP_SILU;
    REQUIRE(num_pairs >= 0 && num_pairs < INT32_MAX, "%s: num_pairs out of range", who);
    REQUIRE(top_k >= 1, "%s: top_k %d < 1", who, top_k);
    REQUIRE(num_pairs % top_k == 0, "%s: num_pairs %lld is not a multiple of top_k %d", who,
            static_cast<long long>(num_pairs), top_k);
    REQUIRE(num_experts >= 1, "%s: num_experts %d < 1", who, num_experts);
    if (num_experts > 256) return fail(MOE_EUNSUPPORTED, "%s: num_experts=%d > 256", who, num_experts);
    REQUIRE(valid_block_size(block_size), "%s: block_size %d not in {16,32,64,128}", who, block_size);
    REQUIRE(n >= 8 && n % 8 == 0, "%s: n %d must be a positive multiple of 8", who, n);
    REQUIRE(k >= 16 && k % 16 == 0, "%s: k %d must be a positive multiple of 16", who, k);
    REQUIRE(max_pad >= max_padded(num_pairs, num_experts, block_size) && max_pad % block_size == 0 &&
                max_pad < INT32_MAX,
            "%s: max_pad %lld must be >= %lld and a multiple of block_size", who, static_cast<long long>(max_pad),
            static_cast<long long>(max_padded(num_pairs, num_experts, block_size)));
    REQUIRE(w0 != nullptr, "%s: w0 is NULL", who);
    if (gate_up) REQUIRE(w1 != nullptr, "%s: MOE_OP_GATE_UP_SILU needs w1 (up)", who);
    else REQUIRE(w1 == nullptr, "%s: op %d takes no w1", who, op);
    REQUIRE(w0->type == MOE_W_FP8, "%s: w0 must be MOE_W_FP8 (type %d)", who, w0->type);
    if (w1) REQUIRE(w1->type == MOE_W_FP8, "%s: w1 must be MOE_W_FP8 (type %d)", who, w1->type);
    if (workspace != nullptr) {
        const int64_t need = moe_grouped_gemm_workspace_bytes();
        REQUIRE_PTR(who, workspace);
        REQUIRE(workspace_bytes >= need, "%s: workspace_bytes %lld < required %lld", who,
                static_cast<long long>(workspace_bytes), static_cast<long long>(need));
    }
    if (num_pairs == 0) return ok();
    REQUIRE_PTR(who, a);
    REQUIRE_PTR(who, a_scale);
    REQUIRE_PTR(who, c);
    REQUIRE_PTR(who, sorted_ids);
    REQUIRE_PTR(who, expert_offsets);
    REQUIRE_PTR(who, w0->data);
    REQUIRE_PTR(who, w0->scales);
    if (w1) {
        REQUIRE_PTR(who, w1->data);
        REQUIRE_PTR(who, w1->scales);
    }
    // the kernel addresses a's rows and each expert matrix with 32-bit byte offsets
    const int64_t a_rows = gate_up ? num_pairs / top_k : max_pad;
    if (a_rows * k > INT64_C(0xffffffff) || static_cast<int64_t>(n) * k > INT64_C(0xffffffff))
        return fail(MOE_EUNSUPPORTED, "%s: fp8 a (%lld rows) or an expert matrix (%d x %d) exceeds 4 GiB", who,
                    static_cast<long long>(a_rows), n, k);
    return launched(who, moe::launch_gemm_fp8(
                             gate_up, a, a_scale, static_cast<const uint8_t*>(w0->data),
                             static_cast<const float*>(w0->scales), w1 ? static_cast<const uint8_t*>(w1->data) : nullptr,
                             w1 ? static_cast<const float*>(w1->scales) : nullptr, c, sorted_ids, expert_offsets,
                             static_cast<int>(num_pairs), top_k, num_experts, n, k, static_cast<int>(max_pad),
                             workspace, workspace_bytes, static_cast<hipStream_t>(stream)));
}

moe_status moe_silu_mul(const uint16_t* gate, const uint16_t* up, uint16_t* out, const int32_t* sorted_ids,
                        int64_t num_pairs, int64_t rows, int32_t n, moe_stream stream) {
    const char* who = "moe_silu_mul";
    REQUIRE(n >= 8 && n % 8 == 0, "%s: n %d must be a positive multiple of 8", who, n);
    REQUIRE(rows >= 0 && rows < INT32_MAX, "%s: rows %lld out of range", who, static_cast<long long>(rows));
    REQUIRE(num_pairs >= 0 && num_pairs < INT32_MAX, "%s: num_pairs out of range", who);
    if (rows == 0) return ok();
    REQUIRE_PTR(who, gate);
    REQUIRE_PTR(who, up);
    REQUIRE_PTR(who, out);
    if (sorted_ids) REQUIRE_PTR(who, sorted_ids);
    return launched(who, moe::launch_silu_mul(gate, up, out, sorted_ids, static_cast<int>(num_pairs), rows, n,
                                              static_cast<hipStream_t>(stream)));
}

moe_status moe_lora_gather_fold(const uint16_t* x, int64_t x_rows, uint16_t* base, int64_t base_rows,
                                const int32_t* indices, int64_t n_slots, int32_t top_k, int32_t x_gather,
                                const int32_t* row_map, const int32_t* row_adapter, const uint64_t* a_table,
                                const uint64_t* b_table, const float* scale_table, int32_t n_tab, int32_t n_adapters,
                                int32_t k_in, int32_t n_out, int32_t max_rank, uint16_t* xa, moe_stream stream) {
    const char* who = "moe_lora_gather_fold";
    REQUIRE(top_k >= 1, "%s: top_k %d < 1", who, top_k);
    REQUIRE(n_slots >= 0 && n_slots < INT32_MAX && n_slots % top_k == 0,
            "%s: n_slots %lld must be in [0, 2^31) and a multiple of top_k=%d", who,
            static_cast<long long>(n_slots), top_k);
    REQUIRE(x_gather == 0 || x_gather == 1, "%s: x_gather %d not 0 or 1", who, x_gather);
    REQUIRE(n_tab >= 0 && n_tab <= 65536, "%s: n_tab %d not in [0, 65536]", who, n_tab);
    REQUIRE(n_adapters >= 1 && n_adapters <= 65536, "%s: n_adapters %d not in [1, 65536]", who, n_adapters);
    REQUIRE(k_in >= 8 && k_in % 8 == 0, "%s: k_in %d must be a positive multiple of 8", who, k_in);
    REQUIRE(n_out >= 8 && n_out % 8 == 0, "%s: n_out %d must be a positive multiple of 8", who, n_out);
    REQUIRE(max_rank >= 32 && max_rank <= 128 && max_rank % 32 == 0, "%s: max_rank %d not in {32,64,96,128}", who,
            max_rank);
    REQUIRE(x_rows >= 0 && base_rows >= 0, "%s: negative row count", who);
    const int64_t need_x = x_gather ? n_slots / top_k : (row_map ? 0 : n_slots);
    REQUIRE(x_rows >= need_x, "%s: x has %lld rows, needs %lld", who, static_cast<long long>(x_rows),
            static_cast<long long>(need_x));
    REQUIRE(row_map || base_rows >= n_slots, "%s: base has %lld rows < n_slots %lld (no row_map)", who,
            static_cast<long long>(base_rows), static_cast<long long>(n_slots));
    if (n_slots == 0 || n_tab == 0) return ok();
    REQUIRE_PTR(who, x);
    REQUIRE_PTR(who, base);
    REQUIRE_PTR(who, indices);
    REQUIRE_PTR(who, a_table);
    REQUIRE_PTR(who, b_table);
    REQUIRE_PTR(who, scale_table);
    REQUIRE_PTR(who, xa);
    if (row_map) REQUIRE_PTR(who, row_map);
    if (row_adapter) REQUIRE_PTR(who, row_adapter);
    return launched(who, moe::launch_lora_gather_fold(x, x_rows, base, base_rows, indices, n_slots, top_k, x_gather,
                                                      row_map, row_adapter, a_table, b_table, scale_table, n_tab,
                                                      n_adapters, k_in, n_out, max_rank, xa,
                                                      static_cast<hipStream_t>(stream)));
}

moe_status moe_combine(const uint16_t* ys, const int32_t* inv_sorted, const float* topk_w, uint16_t* out,
                       int32_t num_tokens, int32_t top_k, int32_t hidden, int64_t ys_rows, moe_stream stream) {
    const char* who = "moe_combine";
    REQUIRE(num_tokens >= 0, "%s: num_tokens %d is negative", who, num_tokens);
    REQUIRE(top_k >= 1, "%s: top_k %d < 1", who, top_k);
    REQUIRE(hidden >= 8 && hidden % 8 == 0, "%s: hidden %d must be a positive multiple of 8", who, hidden);
    REQUIRE(ys_rows >= 0, "%s: ys_rows is negative", who);
    if (num_tokens == 0) return ok();
    REQUIRE_PTR(who, ys);
    REQUIRE_PTR(who, topk_w);
    REQUIRE_PTR(who, out);
    if (inv_sorted) REQUIRE_PTR(who, inv_sorted);
    else REQUIRE(ys_rows >= static_cast<int64_t>(num_tokens) * top_k,
                 "%s: slot-major combine needs ys_rows >= num_tokens*top_k", who);
    return launched(who, moe::launch_combine(ys, inv_sorted, topk_w, out, num_tokens, top_k, hidden, ys_rows,
                                             static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------ ceiling probes (moe_probes.h)
moe_status moe_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t blocks, moe_stream stream) {
    const char* who = "moe_probe_stream_read";
    REQUIRE_PTR(who, src);
    REQUIRE_PTR(who, sink);
    REQUIRE(bytes > 0 && bytes % 16 == 0, "%s: bytes %lld must be a positive multiple of 16", who,
            static_cast<long long>(bytes));
    REQUIRE(blocks >= 1 && blocks <= (1 << 20), "%s: blocks %d not in [1, 2^20]", who, blocks);
    return launched(who, moe::launch_probe_stream_read(src, bytes, sink, blocks, static_cast<hipStream_t>(stream)));
}

moe_status moe_probe_mfma_bf16(int64_t iters, float* sink, int32_t blocks, moe_stream stream) {
    const char* who = "moe_probe_mfma_bf16";
    REQUIRE_PTR(who, sink);
    REQUIRE(iters >= 1, "%s: iters %lld < 1", who, static_cast<long long>(iters));
    REQUIRE(blocks >= 1 && blocks <= (1 << 20), "%s: blocks %d not in [1, 2^20]", who, blocks);
    return launched(who, moe::launch_probe_mfma_bf16(iters, sink, blocks, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
