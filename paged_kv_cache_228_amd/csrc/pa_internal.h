// Internal interface between the C-ABI front end (pa_api.cpp) and the HIP
// kernels (pa_decode.hip, pa_decode_mfma.hip, pa_quantize.hip, pa_append.hip,
// pa_evict.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// KV cache formats of the decode: fp16, INT8 codes, FP8 (OCP E4M3) codes; the
// code formats carry one fp32 scale per (block, KV head) for K and for V.
enum KvFormat { kKvF16 = 0, kKvI8 = 1, kKvF8 = 2 };

constexpr int kBlockTokens = 16;   // tokens per physical KV block
constexpr int kMaxChunkBlocks = 256;  // block ids a decode wave stages in LDS at a time
constexpr int kMaxGroup = 8;       // query heads per KV head
constexpr int kPrepThreads = 1024; // the prefix-sum kernel's one workgroup

// Work decomposition of the decode: for every KV head, the tiles of all
// sequences in order (sequence-major, block-minor; T = sum of blocks per
// sequence) are cut into `shares` contiguous ranges of equal cost, where a
// sequence costs its tiles plus row_cost (pa_split.h; with row cost 0 share
// k is [k T / shares, (k + 1) T / shares)); one wave per (share, KV head).
// A (sequence, KV head) row lying inside one share is finished by that wave;
// a row cut by share boundaries leaves one partial per share, merged by a
// second kernel. The tile prefix sums of the rows come from the context
// lengths: up to kScanSeqs sequences, every decode wave scans them itself
// (and the first wave stores them for the merge); beyond that, a one-workgroup
// kernel runs first and stores them with the first row of every share.
constexpr int kScanSeqs = 256;
struct DecodeArgs {
    const void* q;          // fp16 [S][Hq][D]
    const void* k;          // fp16, int8 or E4M3 pool [NB][Hkv][16][D]
    const void* v;
    const float* k_scale;   // INT8 and FP8: [NB][Hkv]
    const float* v_scale;
    const int32_t* tables;  // [S][max_blocks]
    const int32_t* ctx;     // [S]
    float* out;             // fp32 [S][Hq][D]
    int32_t* rows;          // workspace ints, layout below
    float* part;            // workspace partials, layout below
    int64_t num_blocks;
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int max_blocks;         // table row length
    int shares;             // shares per KV head
    int row_cost;           // the work split's cost of starting a row, in tiles (pa_split.h)
    float scale_log2;       // softmax_scale * log2(e)
};

// Workspace, int32 part: tile prefix sums rows[S + 1]; cost prefix sums
// costs[S + 1] (pa_split.h); the row holding the first tile of each share
// [shares] (written only when S > kScanSeqs); padded to 256 bytes. Then
// fp32 partials: acc [shares][Hkv][2][G][D], then m and l, each
// [shares][Hkv][2][G]; slot 1 of a share holds a cut row whose first tile
// the share holds (the row is the share's last segment), slot 0 a cut row
// that began in an earlier share (the share's first segment).
inline size_t workspace_int_bytes(int S, int shares)
{
    return ((size_t)(2 * ((size_t)S + 1) + shares) * 4 + 255) & ~(size_t)255;
}
inline size_t workspace_bytes(int S, int Hq, int D, int shares)
{
    return workspace_int_bytes(S, shares) + (size_t)shares * 2 * Hq * (size_t)(D + 2) * 4;
}
// Offsets (in int32) of the cost prefix sums and of the share first rows.
__host__ __device__ inline int64_t ws_costs(int S) { return (int64_t)S + 1; }
__host__ __device__ inline int64_t ws_first_row(int S) { return 2 * ((int64_t)S + 1); }
// Largest row cost of the work split (decode_row_cost), for the size checks.
constexpr int kMaxRowCost = 16;

// pa_paged_decode_int8_noalloc's workspace: a static device array of this
// many bytes per GPU (PA_NOALLOC_SCRATCH_BYTES in pa.h), whose address on the
// current device noalloc_scratch() looks up once per device.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
hipError_t noalloc_scratch(void** ptr);

// Work split (prefix sums) -> decode waves -> merge of cut rows, all on `st`.
hipError_t launch_decode(const DecodeArgs& a, int head_dim, int group, int fmt, hipStream_t st);
hipError_t launch_decode_waves(const DecodeArgs& a, int head_dim, int group, int fmt, hipStream_t st);
// Decode waves each compute unit holds at once for this configuration.
int decode_waves_per_cu(int head_dim, int fmt);
// The work split's row cost, in tiles, for this configuration (0..kMaxRowCost).
int decode_row_cost(int head_dim, int fmt);

struct QuantArgs {
    const uint16_t* k;
    const uint16_t* v;
    int8_t* kc;             // INT8 codes, or FP8 (E4M3) codes as bytes
    int8_t* vc;
    float* ks;
    float* vs;
    const int32_t* ids;     // NULL = all blocks
    int64_t num_ids;        // tiles per tensor = num_ids * num_kv_heads
    int64_t num_blocks;
    int num_kv_heads;
};

hipError_t launch_quantize(const QuantArgs& a, int head_dim, hipStream_t st);
hipError_t launch_quantize_fp8(const QuantArgs& a, int head_dim, hipStream_t st);

// One new token per sequence into the paged cache (pa_append.hip).
struct AppendArgs {
    const uint16_t* k_new;    // fp16 [S][Hkv][D]
    const uint16_t* v_new;
    void* k;                  // fp16 or int8 pool [NB][Hkv][16][D]
    void* v;
    float* ks;                // INT8 only: [NB][Hkv]
    float* vs;
    const int32_t* tables;    // [S][max_blocks]
    const int32_t* positions; // [S]
    int64_t num_blocks;
    int num_seqs;
    int num_kv_heads;
    int max_blocks;
};

hipError_t launch_append(const AppendArgs& a, int head_dim, bool int8, hipStream_t st);

// Eviction choice over the physical blocks (pa_evict.hip).
struct EvictArgs {
    const int32_t* refcount;   // [num_blocks]
    const int32_t* last_used;  // [num_blocks]
    int32_t* out;              // [k]
    int64_t num_blocks;
    int64_t k;
    int32_t tick;
};

hipError_t launch_evict(const EvictArgs& a, hipStream_t st);

// Block copy for copy-on-write (pa_copy.hip).
struct CopyArgs {
    const char* src;
    char* dst;
    const int32_t* src_ids;  // [num_pairs]
    const int32_t* dst_ids;
    int64_t bytes_per_block;
    int64_t num_blocks;
    int64_t num_pairs;
};

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t st);

// HBM read-bandwidth probe (pa_probe.hip).
struct ProbeArgs {
    const void* src;  // 16-byte aligned
    int64_t words;    // 16-byte words to read
    uint32_t* sink;   // read probe: [workgroups]
    void* dst;        // read-and-write probe: [words] 8-byte words (NULL: read probe)
};

hipError_t launch_read_probe(const ProbeArgs& a, int workgroups, hipStream_t st);

}  // namespace pa
