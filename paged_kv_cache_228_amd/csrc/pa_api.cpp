// C-ABI front end of the paged decode attention library: argument checks,
// partition sizing and kernel launches. Declarations and the contract of each
// call are in include/pa.h.
#include "pa.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>

#include "pa_internal.h"

namespace {

thread_local char g_hip_msg[160] = "no HIP error recorded";

int hip_fail(hipError_t e)
{
    std::snprintf(g_hip_msg, sizeof g_hip_msg, "HIP error %d: %s", (int)e, hipGetErrorString(e));
    return PA_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Compute units of the current device (256 when there is none to ask).
int num_compute_units()
{
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
        return v;
    return 256;
}

// Shares per KV head (see pa_internal.h). An explicit partition_tokens asks
// for shares of about that many tokens, sized for the longest possible batch
// (num_seqs x max_blocks_per_seq blocks). Otherwise one wave per share fills
// the device once: compute units x decode waves per unit, split over the KV
// heads, and no share shorter than 8 blocks of that bound; for a bound of at
// most kTinyBound blocks, shares of one block but at most kMergeRound per
// sequence (the merge kernel's loads in flight per round). Never more shares
// than the bound has blocks.
constexpr long long kTinyBound = 64;
constexpr long long kMergeRound = 8;
long long shares_per_head(int num_seqs, int num_kv_heads, int head_dim, int max_blocks,
                          int partition_tokens, int fmt)
{
    const long long bound = (long long)num_seqs * max_blocks;
    if (bound <= 0) return 1;
    long long k;
    if (partition_tokens > 0) {
        k = (bound * pa::kBlockTokens + partition_tokens - 1) / partition_tokens;
    } else {
        const long long waves = (long long)num_compute_units() * pa::decode_waves_per_cu(head_dim, fmt);
        k = std::max(1LL, waves / num_kv_heads);
        if (bound <= kTinyBound) {
            // a tiny batch is all latency: shares of one block, so that no wave
            // walks two rows' segments one after the other, but no more than
            // kMergeRound per sequence, so that a row's partials are merged in
            // one round of loads
            k = std::min(k, std::min(bound, (long long)kMergeRound * num_seqs));
        } else {
            k = std::min(k, (bound + 7) / 8);
        }
    }
    return std::max(1LL, std::min(k, bound));
}

int check_decode_shape(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                       int block_size, int max_blocks_per_seq, int64_t num_blocks,
                       int partition_tokens)
{
    if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 || partition_tokens < 0)
        return PA_ERR_SHAPE;
    if (num_q_heads % num_kv_heads) return PA_ERR_SHAPE;
    if (partition_tokens % pa::kBlockTokens) return PA_ERR_SHAPE;
    if (block_size != pa::kBlockTokens) return PA_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    const int group = num_q_heads / num_kv_heads;
    if (group < 1 || group > pa::kMaxGroup) return PA_ERR_UNSUPPORTED;
    if (num_seqs > 65535 || num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;
    if ((long long)max_blocks_per_seq * pa::kBlockTokens > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
    // tile and cost prefix sums are int32; one workgroup per (share, KV head)
    if ((long long)num_seqs * (max_blocks_per_seq + pa::kMaxRowCost) > 0x7fffffffLL)
        return PA_ERR_UNSUPPORTED;
    for (int fmt = pa::kKvF16; fmt <= pa::kKvF8; ++fmt)
        if (shares_per_head(num_seqs, num_kv_heads, head_dim, max_blocks_per_seq, partition_tokens, fmt) *
                num_kv_heads > 0x7fffffffLL)
            return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

int decode_common(const void* q, const void* k, const void* v, const float* ks, const float* vs,
                  const int32_t* tables, const int32_t* ctx, float* out, int num_seqs,
                  int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                  int max_blocks_per_seq, int64_t num_blocks, float softmax_scale,
                  int partition_tokens, void* workspace, size_t workspace_bytes, void* stream,
                  int fmt)
{
    if (!q || !k || !v || !tables || !ctx || !out) return PA_ERR_NULL;
    if (fmt != pa::kKvF16 && (!ks || !vs)) return PA_ERR_NULL;
    int rc = check_decode_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                max_blocks_per_seq, num_blocks, partition_tokens);
    if (rc) return rc;
    if (!std::isfinite(softmax_scale)) return PA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PA_OK;

    const int shares = (int)shares_per_head(num_seqs, num_kv_heads, head_dim, max_blocks_per_seq,
                                            partition_tokens, fmt);
    const size_t need = pa::workspace_bytes(num_seqs, num_q_heads, head_dim, shares);
    if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PA_ERR_UNSUPPORTED;

    pa::DecodeArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.k_scale = ks;
    a.v_scale = vs;
    a.tables = tables;
    a.ctx = ctx;
    a.out = out;
    a.rows = static_cast<int32_t*>(workspace);
    a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                      pa::workspace_int_bytes(num_seqs, shares));
    a.num_blocks = num_blocks;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.max_blocks = max_blocks_per_seq;
    a.shares = shares;
    // batches of at most kTinyBound possible tiles per KV head keep the plain
    // split, whose one-tile shares then start no second row
    a.row_cost = (long long)num_seqs * max_blocks_per_seq <= kTinyBound ? 0 : pa::decode_row_cost(head_dim, fmt);
    a.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
    hipError_t e = pa::launch_decode(a, head_dim, num_q_heads / num_kv_heads, fmt,
                                     static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : hip_fail(e);
}

int append_common(const void* k_new, const void* v_new, void* k_cache, void* v_cache, float* ks,
                  float* vs, const int32_t* tables, const int32_t* positions, int num_seqs,
                  int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                  int64_t num_blocks, void* stream, bool int8)
{
    if (!k_new || !v_new || !k_cache || !v_cache || !tables || !positions) return PA_ERR_NULL;
    if (int8 && (!ks || !vs)) return PA_ERR_NULL;
    if (num_seqs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        max_blocks_per_seq <= 0 || num_blocks <= 0)
        return PA_ERR_SHAPE;
    if (block_size != pa::kBlockTokens) return PA_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (num_seqs > 65535 || num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
        return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PA_OK;
    pa::AppendArgs a;
    a.k_new = static_cast<const uint16_t*>(k_new);
    a.v_new = static_cast<const uint16_t*>(v_new);
    a.k = k_cache;
    a.v = v_cache;
    a.ks = ks;
    a.vs = vs;
    a.tables = tables;
    a.positions = positions;
    a.num_blocks = num_blocks;
    a.num_seqs = num_seqs;
    a.num_kv_heads = num_kv_heads;
    a.max_blocks = max_blocks_per_seq;
    hipError_t e = pa::launch_append(a, head_dim, int8, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : hip_fail(e);
}

int quantize_common(const void* k_f16, const void* v_f16, void* k_i8, void* v_i8, float* k_scale,
                    float* v_scale, const int32_t* block_ids, int64_t num_ids, int64_t num_blocks,
                    int num_kv_heads, int block_size, int head_dim, void* stream, bool fp8)
{
    if (!k_f16 || !v_f16 || !k_i8 || !v_i8 || !k_scale || !v_scale) return PA_ERR_NULL;
    if (num_blocks <= 0 || num_kv_heads <= 0 || block_size <= 0 || head_dim <= 0)
        return PA_ERR_SHAPE;
    if (block_ids && num_ids < 0) return PA_ERR_SHAPE;
    if (block_size != pa::kBlockTokens) return PA_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (!aligned16(k_f16) || !aligned16(v_f16) || (reinterpret_cast<uintptr_t>(k_i8) & 7u) ||
        (reinterpret_cast<uintptr_t>(v_i8) & 7u))
        return PA_ERR_UNSUPPORTED;
    pa::QuantArgs a;
    a.k = static_cast<const uint16_t*>(k_f16);
    a.v = static_cast<const uint16_t*>(v_f16);
    a.kc = static_cast<int8_t*>(k_i8);
    a.vc = static_cast<int8_t*>(v_i8);
    a.ks = k_scale;
    a.vs = v_scale;
    a.ids = block_ids;
    a.num_ids = block_ids ? num_ids : num_blocks;
    a.num_blocks = num_blocks;
    a.num_kv_heads = num_kv_heads;
    if ((a.num_ids * num_kv_heads * 2 + 3) / 4 > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
    hipError_t e = fp8 ? pa::launch_quantize_fp8(a, head_dim, static_cast<hipStream_t>(stream))
                       : pa::launch_quantize(a, head_dim, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : hip_fail(e);
}

}  // namespace

extern "C" {

const char* pa_error_string(int code)
{
    switch (code) {
        case PA_OK: return "success";
        case PA_ERR_NULL: return "a required pointer is NULL";
        case PA_ERR_SHAPE: return "inconsistent or non-positive sizes";
        case PA_ERR_UNSUPPORTED:
            return "unsupported configuration (block_size must be 16, head_dim 64 or 128, "
                   "1..8 query heads per KV head, 16-byte aligned buffers)";
        case PA_ERR_WORKSPACE: return "split-K workspace missing or too small";
        case PA_ERR_HIP: return g_hip_msg;
        case PA_ERR_FULL: return "no free KV block (or a reference count at its limit)";
        case PA_ERR_STATE: return "the block is not allocated";
        default: return "unknown error code";
    }
}

int pa_quantize_kv_int8(const void* k_f16, const void* v_f16, int8_t* k_i8, int8_t* v_i8,
                        float* k_scale, float* v_scale, const int32_t* block_ids,
                        int64_t num_ids, int64_t num_blocks, int num_kv_heads, int block_size,
                        int head_dim, void* stream)
{
    return quantize_common(k_f16, v_f16, k_i8, v_i8, k_scale, v_scale, block_ids, num_ids,
                           num_blocks, num_kv_heads, block_size, head_dim, stream, false);
}

int pa_quantize_kv_fp8(const void* k_f16, const void* v_f16, uint8_t* k_fp8, uint8_t* v_fp8,
                       float* k_scale, float* v_scale, const int32_t* block_ids,
                       int64_t num_ids, int64_t num_blocks, int num_kv_heads, int block_size,
                       int head_dim, void* stream)
{
    return quantize_common(k_f16, v_f16, k_fp8, v_fp8, k_scale, v_scale, block_ids, num_ids,
                           num_blocks, num_kv_heads, block_size, head_dim, stream, true);
}

int pa_decode_shares(int num_seqs, int num_kv_heads, int head_dim, int max_blocks_per_seq,
                     int block_size, int partition_tokens, int kv_format)
{
    if (num_seqs < 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 || block_size <= 0 ||
        partition_tokens < 0 || partition_tokens % pa::kBlockTokens)
        return PA_ERR_SHAPE;
    if (block_size != pa::kBlockTokens) return PA_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
    if (kv_format < pa::kKvF16 || kv_format > pa::kKvF8) return PA_ERR_UNSUPPORTED;
    if ((long long)num_seqs * (max_blocks_per_seq + pa::kMaxRowCost) > 0x7fffffffLL)
        return PA_ERR_UNSUPPORTED;
    return (int)std::min(shares_per_head(num_seqs, num_kv_heads, head_dim, max_blocks_per_seq,
                                         partition_tokens, kv_format),
                         0x7fffffffLL);
}

size_t pa_decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                 int max_blocks_per_seq, int block_size, int partition_tokens,
                                 int kv_format)
{
    if (kv_format < pa::kKvF16 || kv_format > pa::kKvF8) return 0;
    if (check_decode_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                           max_blocks_per_seq, 1, partition_tokens))
        return 0;
    const long long shares = shares_per_head(num_seqs, num_kv_heads, head_dim, max_blocks_per_seq,
                                             partition_tokens, kv_format);
    return pa::workspace_bytes(num_seqs, num_q_heads, head_dim, (int)shares);
}

int pa_paged_decode_f16(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* context_lens, float* out,
                        int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                        int block_size, int max_blocks_per_seq, int64_t num_blocks,
                        float softmax_scale, int partition_tokens, void* workspace,
                        size_t workspace_bytes, void* stream)
{
    return decode_common(q, k_cache, v_cache, nullptr, nullptr, block_tables, context_lens, out,
                         num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                         max_blocks_per_seq, num_blocks, softmax_scale, partition_tokens,
                         workspace, workspace_bytes, stream, pa::kKvF16);
}

int pa_paged_decode_int8(const void* q, const int8_t* k_cache, const int8_t* v_cache,
                         const float* k_scale, const float* v_scale,
                         const int32_t* block_tables, const int32_t* context_lens, float* out,
                         int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                         int block_size, int max_blocks_per_seq, int64_t num_blocks,
                         float softmax_scale, int partition_tokens, void* workspace,
                         size_t workspace_bytes, void* stream)
{
    return decode_common(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, out,
                         num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                         max_blocks_per_seq, num_blocks, softmax_scale, partition_tokens,
                         workspace, workspace_bytes, stream, pa::kKvI8);
}

int pa_paged_decode_int8_noalloc(const void* q, const int8_t* k_cache, const int8_t* v_cache,
                                 const float* k_scale, const float* v_scale,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 float* out, int num_seqs, int num_q_heads, int num_kv_heads,
                                 int head_dim, int block_size, int max_blocks_per_seq,
                                 int64_t num_blocks, float softmax_scale, int partition_tokens,
                                 void* stream)
{
    static_assert(PA_NOALLOC_SCRATCH_BYTES == pa::kNoAllocScratchBytes, "one stated maximum");
    // every host-side check of the workspace variant, and the size limit, before
    // any HIP call
    if (!q || !k_cache || !v_cache || !k_scale || !v_scale || !block_tables || !context_lens || !out)
        return PA_ERR_NULL;
    int rc = check_decode_shape(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                max_blocks_per_seq, num_blocks, partition_tokens);
    if (rc) return rc;
    if (!std::isfinite(softmax_scale)) return PA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
        return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PA_OK;
    const long long shares = shares_per_head(num_seqs, num_kv_heads, head_dim, max_blocks_per_seq,
                                             partition_tokens, pa::kKvI8);
    const size_t need = pa::workspace_bytes(num_seqs, num_q_heads, head_dim, (int)shares);
    if (need > pa::kNoAllocScratchBytes) return PA_ERR_WORKSPACE;
    void* scratch = nullptr;
    hipError_t e = pa::noalloc_scratch(&scratch);
    if (e != hipSuccess) return hip_fail(e);
    return decode_common(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, out,
                         num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                         max_blocks_per_seq, num_blocks, softmax_scale, partition_tokens, scratch,
                         pa::kNoAllocScratchBytes, stream, pa::kKvI8);
}

int pa_paged_decode_fp8(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                        const float* k_scale, const float* v_scale, const int32_t* block_tables,
                        const int32_t* context_lens, float* out, int num_seqs, int num_q_heads,
                        int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                        int64_t num_blocks, float softmax_scale, int partition_tokens,
                        void* workspace, size_t workspace_bytes, void* stream)
{
    return decode_common(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, out,
                         num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                         max_blocks_per_seq, num_blocks, softmax_scale, partition_tokens,
                         workspace, workspace_bytes, stream, pa::kKvF8);
}

int pa_copy_blocks(const void* src_pool, void* dst_pool, int64_t bytes_per_block,
                   const int32_t* src_ids, const int32_t* dst_ids, int64_t num_pairs,
                   int64_t num_blocks, void* stream)
{
    if (num_pairs < 0 || bytes_per_block <= 0 || num_blocks <= 0) return PA_ERR_SHAPE;
    if (num_pairs == 0) return PA_OK;
    if (!src_pool || !dst_pool || !src_ids || !dst_ids) return PA_ERR_NULL;
    if (num_pairs > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
    pa::CopyArgs a;
    a.src = static_cast<const char*>(src_pool);
    a.dst = static_cast<char*>(dst_pool);
    a.src_ids = src_ids;
    a.dst_ids = dst_ids;
    a.bytes_per_block = bytes_per_block;
    a.num_blocks = num_blocks;
    a.num_pairs = num_pairs;
    hipError_t e = pa::launch_copy_blocks(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : hip_fail(e);
}

int pa_hbm_read_probe(const void* src, int64_t bytes, uint32_t* sink, int workgroups, void* stream)
{
    if (!src || !sink) return PA_ERR_NULL;
    if (bytes <= 0 || workgroups <= 0) return PA_ERR_SHAPE;
    if (bytes % 16 || !aligned16(src)) return PA_ERR_UNSUPPORTED;
    pa::ProbeArgs a;
    a.src = src;
    a.words = bytes / 16;
    a.sink = sink;
    a.dst = nullptr;
    hipError_t e = pa::launch_read_probe(a, workgroups, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : hip_fail(e);
}

int pa_hbm_rw_probe(const void* src, int64_t bytes, void* dst, int workgroups, void* stream)
{
    if (!src || !dst) return PA_ERR_NULL;
    if (bytes <= 0 || workgroups <= 0) return PA_ERR_SHAPE;
    if (bytes % 16 || !aligned16(src) || (reinterpret_cast<uintptr_t>(dst) & 7u)) return PA_ERR_UNSUPPORTED;
    pa::ProbeArgs a;
    a.src = src;
    a.words = bytes / 16;
    a.sink = nullptr;
    a.dst = dst;
    hipError_t e = pa::launch_read_probe(a, workgroups, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : hip_fail(e);
}

int pa_evict_select(const int32_t* refcount, const int32_t* last_used, int64_t num_blocks,
                    int32_t current_tick, int64_t k, int32_t* out_ids, void* stream)
{
    if (!refcount || !last_used || (k > 0 && !out_ids)) return PA_ERR_NULL;
    if (num_blocks <= 0 || k < 0) return PA_ERR_SHAPE;
    if (num_blocks > 0x7fffffffLL || k > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
    if (((reinterpret_cast<uintptr_t>(refcount) | reinterpret_cast<uintptr_t>(last_used)) & 15u) ||
        (reinterpret_cast<uintptr_t>(out_ids) & 3u))
        return PA_ERR_UNSUPPORTED;
    pa::EvictArgs a;
    a.refcount = refcount;
    a.last_used = last_used;
    a.out = out_ids;
    a.num_blocks = num_blocks;
    a.k = k;
    a.tick = current_tick;
    hipError_t e = pa::launch_evict(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : hip_fail(e);
}

int pa_append_kv_f16(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                     const int32_t* block_tables, const int32_t* positions, int num_seqs,
                     int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                     int64_t num_blocks, void* stream)
{
    return append_common(k_new, v_new, k_cache, v_cache, nullptr, nullptr, block_tables, positions,
                         num_seqs, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                         num_blocks, stream, false);
}

int pa_append_kv_int8(const void* k_new, const void* v_new, int8_t* k_cache, int8_t* v_cache,
                      float* k_scale, float* v_scale, const int32_t* block_tables,
                      const int32_t* positions, int num_seqs, int num_kv_heads, int head_dim,
                      int block_size, int max_blocks_per_seq, int64_t num_blocks, void* stream)
{
    return append_common(k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_tables,
                         positions, num_seqs, num_kv_heads, head_dim, block_size,
                         max_blocks_per_seq, num_blocks, stream, true);
}

}  // extern "C"
