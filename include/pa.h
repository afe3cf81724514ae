/*
 * pa.h - paged single-token decode attention for AMD MI355X (gfx950).
 *
 * A K/V cache is split into fixed 16-token physical blocks; each sequence
 * reaches its blocks through a block table, and one decode step attends a
 * single query token per sequence over its whole context (paged-attention-
 * runtime summary, "CORE CAPABILITIES" 1 "Block Manager" and 2 "CUDA Kernel":
 * fixed 16-token blocks, block-table indirection, online single-pass softmax,
 * fp32 accumulation; PagedKV-Fusion README, "Overview": per-(block, head)
 * quantized decode attention).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every pointer is a DEVICE pointer owned by the caller. The library never
 *    allocates, frees or synchronizes; each call enqueues its kernels on
 *    `stream` (a hipStream_t passed as void*, NULL = the null stream) and
 *    returns without waiting. Calls keep no state and may be issued from
 *    several host threads at once (pa_paged_decode_int8_noalloc aside: its
 *    workspace is one static device array per GPU, see there).
 *  - K/V pools: [num_blocks][num_kv_heads][block_size][head_dim], row-major;
 *    the 16 x head_dim tile of one (block, KV head) is contiguous. Token t of
 *    sequence s lives in block block_tables[s][t / 16] at slot t % 16
 *    (PagedAttention & KV-Cache glossary monograph, section 2.1).
 *  - block_size must be 16; head_dim 64 or 128; num_q_heads a multiple of
 *    num_kv_heads with num_q_heads / num_kv_heads between 1 and 8. Query head
 *    h reads KV head h / (num_q_heads / num_kv_heads) (consecutive GQA
 *    groups; paged-attention-runtime summary item 4, GQA expanded).
 *  - q: fp16 [num_seqs][num_q_heads][head_dim]; out: fp32, same shape.
 *    block_tables: int32 [num_seqs][max_blocks_per_seq]; context_lens: int32
 *    [num_seqs]. q, pools, codes, out and workspace must be 16-byte aligned.
 *  - Errors found on the host (NULL pointers, bad shapes, unsupported sizes,
 *    a workspace that is too small) return a negative code before anything
 *    is launched. A launch failure returns PA_ERR_HIP; pa_error_string then
 *    names the HIP error. Device-resident data is not validated (that would
 *    need a synchronization): a context length below 0 counts as 0 and one
 *    above max_blocks_per_seq * 16 is clamped to it; a block id outside
 *    [0, num_blocks) reads as a tile of zeros instead of faulting; a
 *    sequence with context length 0 gets an all-zero output row.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    PA_OK = 0,
    PA_ERR_NULL = -1,        /* a required pointer is NULL */
    PA_ERR_SHAPE = -2,       /* inconsistent or non-positive sizes */
    PA_ERR_UNSUPPORTED = -3, /* valid but not built: block_size, head_dim, group size, alignment */
    PA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required */
    PA_ERR_HIP = -5,         /* a HIP call failed; see pa_error_string */
    PA_ERR_FULL = -6,        /* block manager: no free block */
    PA_ERR_STATE = -7        /* block manager: the block is not allocated */
};

/* Static description of a return code. For PA_ERR_HIP it names the last HIP
 * error seen by the calling thread. Never NULL. */
const char* pa_error_string(int code);

/* Symmetric INT8 quantization with one fp32 scale per (block, KV head), for
 * K and for V separately (PagedKV-Fusion README, "Overview" and "Architecture":
 * per-block,head symmetric INT8; "Memory footprint (exact arithmetic)": two
 * fp32 scales per (block, head); glossary monograph section 5.1: code =
 * round(x / S)). For every listed physical block b and KV head h, over the
 * whole 16 x head_dim tile (unused slots included):
 *     amax = max |x|,  scale = amax / 127 (fp32, IEEE-rounded division),
 *     code = clamp(round_half_even(x / scale), -127, 127)  (x / scale an IEEE
 *     fp32 division), and scale 0 gives codes 0.
 *  k_f16, v_f16   in:  fp16 pools [num_blocks][num_kv_heads][16][head_dim]
 *  k_i8, v_i8     out: int8 code pools of the same shape
 *  k_scale,v_scale out: fp32 [num_blocks][num_kv_heads]
 *  block_ids      in:  int32 [num_ids] physical blocks to quantize, or NULL for
 *                      all num_blocks blocks; other blocks are left untouched.
 *                      Ids outside [0, num_blocks) are skipped on the device.
 * Returns PA_OK or a negative PA_ERR_* code. */
int pa_quantize_kv_int8(const void* k_f16, const void* v_f16, int8_t* k_i8, int8_t* v_i8,
                        float* k_scale, float* v_scale, const int32_t* block_ids,
                        int64_t num_ids, int64_t num_blocks, int num_kv_heads, int block_size,
                        int head_dim, void* stream);

/* The FP8 variant of pa_quantize_kv_int8 (monograph section 5.1: FP8 or INT8
 * codes with symmetric per-block scales; the format read as OCP 8-bit E4M3:
 * bias 7, largest finite 448, no infinities). Per (block, KV head) tile:
 *     amax = max |x|,  scale = amax / 448 (fp32, IEEE-rounded division),
 *     code = the E4M3 value nearest to x / scale (an IEEE fp32 division; ties
 *     to an even mantissa), and scale 0 gives codes 0.
 *  k_fp8, v_fp8   out: E4M3 code pools (bytes) [num_blocks][num_kv_heads][16][head_dim]
 * Other arguments, layouts and errors as pa_quantize_kv_int8. */
int pa_quantize_kv_fp8(const void* k_f16, const void* v_f16, uint8_t* k_fp8, uint8_t* v_fp8,
                       float* k_scale, float* v_scale, const int32_t* block_ids,
                       int64_t num_ids, int64_t num_blocks, int num_kv_heads, int block_size,
                       int head_dim, void* stream);

/* Work split of the decode calls. For every KV head the tiles of all
 * sequences, in sequence order, are cut into contiguous shares of equal
 * cost, one 64-lane wave each, where each sequence costs its tiles plus a
 * few tiles' worth for starting it (spread over its tiles; sequences of equal
 * length, up to 256 sequences, and batches of at most 64 possible blocks per
 * KV head are cut by tiles alone); a (sequence, KV head)
 * whose tiles fall in one share is finished by that wave, one cut by share
 * boundaries is completed by a merge kernel from the shares' partial results
 * (log-sum-exp combine).
 * partition_tokens: the wanted tokens per share for the longest possible
 * batch (num_seqs x max_blocks_per_seq x 16 tokens), a multiple of 16, or 0
 * to let the library size one wave per SIMD of the current device (two at
 * head_dim 64) over the KV heads (fewer for small batches: at least 8 blocks of that longest batch
 * per share, or, when it has at most 64 blocks, one block per share and at
 * most 8 shares per sequence). A share spans sequence boundaries, so this is not a
 * per-sequence context partition: a value of at least num_seqs x
 * max_blocks_per_seq x 16 gives one share per KV head, with which no row is
 * cut (no split-K; the merge kernel then only writes the rows of empty
 * contexts), while max_blocks_per_seq x 16 still gives num_seqs shares.
 * kv_format: 0 for pa_paged_decode_f16, 1 for pa_paged_decode_int8, 2
 * for pa_paged_decode_fp8 (other values are rejected). The sizing helpers
 * take num_kv_heads, head_dim and kv_format because the automatic share
 * count spreads the waves over the KV heads and the waves per SIMD depend on
 * the head dimension (and may depend on the format).
 *
 * pa_decode_shares returns the number of shares per KV head, or a negative
 * PA_ERR_* code for arguments the decode calls would reject.
 * pa_decode_workspace_bytes returns the workspace a decode call with these
 * arguments needs (tile prefix sums and partials; always more than 0), or 0
 * for arguments the decode calls would reject. Both depend on the current
 * device's compute-unit count when partition_tokens is 0. */
int pa_decode_shares(int num_seqs, int num_kv_heads, int head_dim, int max_blocks_per_seq,
                     int block_size, int partition_tokens, int kv_format);
size_t pa_decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                 int max_blocks_per_seq, int block_size, int partition_tokens,
                                 int kv_format);

/* Decode attention over an fp16 paged KV cache. For every sequence s and
 * query head h, with n = context_lens[s] and k_t, v_t the K/V rows of token t
 * reached through the block table:
 *     out[s][h] = sum_t softmax_t(softmax_scale * q[s][h] . k_t) * v_t
 * computed with a single-pass online softmax in fp32 (paged-attention-runtime
 * summary, "CORE CAPABILITIES" 2; glossary monograph section 5.2,
 * softmax(Q K^T / sqrt(d))). Two stream-ordered kernels, the decode waves
 * and the merge (see pa_decode_shares); above 256 sequences a third, the
 * work split (prefix sums of the context lengths), runs first. workspace: at least pa_decode_workspace_bytes(...) bytes
 * of device memory owned by the caller, overwritten by every call; calls that
 * share a workspace must not overlap. num_seqs may be 0 (nothing is
 * launched, workspace may be NULL). */
int pa_paged_decode_f16(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* context_lens, float* out,
                        int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                        int block_size, int max_blocks_per_seq, int64_t num_blocks,
                        float softmax_scale, int partition_tokens, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Same as pa_paged_decode_f16 over an INT8 cache produced by
 * pa_quantize_kv_int8: K and V elements are float(code) * scale of their
 * (block, KV head), dequantized in registers (PagedKV-Fusion README,
 * "Overview": per-(block, head) quantized decode attention).
 *  k_cache, v_cache: int8 [num_blocks][num_kv_heads][16][head_dim]
 *  k_scale, v_scale: fp32 [num_blocks][num_kv_heads] */
int pa_paged_decode_int8(const void* q, const int8_t* k_cache, const int8_t* v_cache,
                         const float* k_scale, const float* v_scale,
                         const int32_t* block_tables, const int32_t* context_lens, float* out,
                         int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                         int block_size, int max_blocks_per_seq, int64_t num_blocks,
                         float softmax_scale, int partition_tokens, void* workspace,
                         size_t workspace_bytes, void* stream);

/* pa_paged_decode_int8 for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the workspace taken from a
 * static device array of PA_NOALLOC_SCRATCH_BYTES bytes that the library holds
 * on every GPU it runs on until the process ends; the call itself allocates
 * nothing. All arguments are those of pa_paged_decode_int8 without the
 * workspace. Every call on one GPU shares that GPU's array: calls that overlap
 * on one GPU (other streams, other host threads) race and must be ordered by
 * the caller. Nothing in the array needs clearing between calls (each call
 * writes what it later reads). Returns PA_ERR_WORKSPACE, before anything is
 * launched, when the shape needs more workspace than the array holds
 * (pa_decode_workspace_bytes(..., kv_format 1) > PA_NOALLOC_SCRATCH_BYTES),
 * PA_ERR_HIP when the array's address cannot be looked up on the current
 * device, and otherwise what pa_paged_decode_int8 returns. */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int pa_paged_decode_int8_noalloc(const void* q, const int8_t* k_cache, const int8_t* v_cache,
                                 const float* k_scale, const float* v_scale,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 float* out, int num_seqs, int num_q_heads, int num_kv_heads,
                                 int head_dim, int block_size, int max_blocks_per_seq,
                                 int64_t num_blocks, float softmax_scale, int partition_tokens,
                                 void* stream);

/* Same as pa_paged_decode_int8 over an FP8 (OCP E4M3) cache produced by
 * pa_quantize_kv_fp8: K and V elements are e4m3(code) * scale of their
 * (block, KV head) (monograph section 5.1's FP8 variant).
 *  k_cache, v_cache: E4M3 codes (bytes) [num_blocks][num_kv_heads][16][head_dim]
 *  k_scale, v_scale: fp32 [num_blocks][num_kv_heads] */
int pa_paged_decode_fp8(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                        const float* k_scale, const float* v_scale, const int32_t* block_tables,
                        const int32_t* context_lens, float* out, int num_seqs, int num_q_heads,
                        int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                        int64_t num_blocks, float softmax_scale, int partition_tokens,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Choose the physical blocks to evict (PagedKV-Fusion README, "Overview",
 * component A: scoring plus a top-k over the paged blocks, the "bottom-k
 * eviction ids" of its sequence diagram). Scores follow the PagedAttention &
 * KV-Cache Memory Management monograph, section 4.3.1 (least reference count
 * plus age): over the allocated blocks (refcount > 0),
 *     score = 0.7 (max_refcnt - refcount[b]) + 0.3 (current_tick - last_used[b])
 * with max_refcnt the largest reference count among them; a higher score is a
 * better block to evict. out_ids receives the min(k, candidates) blocks with
 * the largest scores (equal scores: the smaller block id first) in ascending
 * id order, then -1 up to k. The order is computed exactly (integer keys, no
 * rounding).
 *  refcount, last_used: int32 [num_blocks] (device, 16-byte aligned);
 *  out_ids: int32 [k] (device)
 * One asynchronous single-workgroup kernel on `stream`; nothing is allocated.
 * Returns PA_OK (k == 0 launches nothing), PA_ERR_NULL, PA_ERR_SHAPE
 * (num_blocks <= 0, k < 0), PA_ERR_UNSUPPORTED (more than 2^31 - 1 blocks or
 * ids, misaligned buffers) or PA_ERR_HIP. */
int pa_evict_select(const int32_t* refcount, const int32_t* last_used, int64_t num_blocks,
                    int32_t current_tick, int64_t k, int32_t* out_ids, void* stream);

/* Append one new token per sequence to a paged cache (the step before a
 * decode). Token t = positions[s] of sequence s goes to physical block
 * block_tables[s][t / 16] at slot t mod 16 (glossary monograph, section 2.1;
 * PagedAttention article, "Kernel Mechanics": new K/V are written at
 * phys_block_id * B + token_offset). A negative position, a position past the
 * table row (t / 16 >= max_blocks_per_seq) or a table entry outside
 * [0, num_blocks) appends nothing for that sequence; other device data is not
 * validated.
 *  k_new, v_new: fp16 [num_seqs][num_kv_heads][head_dim], the new token's rows
 *  k_cache, v_cache: [num_blocks][num_kv_heads][16][head_dim], updated in place
 *  block_tables: int32 [num_seqs][max_blocks_per_seq]; positions: int32 [num_seqs]
 * All pointers are device pointers owned by the caller; every buffer starts on
 * a 16-byte boundary. Two sequences must not append into the same block in one
 * call. One asynchronous kernel on `stream`; nothing is allocated.
 * Returns PA_OK (also for num_seqs == 0), PA_ERR_NULL, PA_ERR_SHAPE,
 * PA_ERR_UNSUPPORTED (block_size != 16, head_dim not 64 or 128, more than
 * 65,535 sequences or KV heads, misaligned buffers) or PA_ERR_HIP.
 *
 * pa_append_kv_f16 copies the rows into the fp16 cache. */
int pa_append_kv_f16(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                     const int32_t* block_tables, const int32_t* positions, int num_seqs,
                     int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                     int64_t num_blocks, void* stream);

/* pa_append_kv_int8 appends to an INT8 cache with one fp32 scale per (block,
 * KV head) for K and one for V (the layout pa_quantize_kv_int8 writes). The
 * pages fix the quantizer (PagedKV-Fusion README, "Overview": symmetric INT8
 * per (block, head); glossary monograph, section 5.1: code = round(x / S))
 * but not how a codes-only cache takes a new token; the rule here keeps one
 * scale per tile for its live rows. With x the new row, o = t mod 16, s_old
 * the tile's scale and s_new = max|x| / 127 (IEEE fp32 division):
 *   o == 0:                the block's first token: scale = s_new, row 0 = q(x, s_new)
 *   o > 0, s_new <= s_old: row o = q(x, s_old), scale kept
 *   o > 0, s_new >  s_old: rows r < o re-quantized as q(code * s_old, s_new)
 *                          (fp32 product), row o = q(x, s_new), scale = s_new
 * q(v, s) = 0 if s == 0, else clamp(round-half-even(v / s), -127, 127) with
 * an IEEE fp32 division. Rows after o are not touched.
 *  k_scale, v_scale: fp32 [num_blocks][num_kv_heads], updated in place */
int pa_append_kv_int8(const void* k_new, const void* v_new, int8_t* k_cache, int8_t* v_cache,
                      float* k_scale, float* v_scale, const int32_t* block_tables,
                      const int32_t* positions, int num_seqs, int num_kv_heads, int head_dim,
                      int block_size, int max_blocks_per_seq, int64_t num_blocks, void* stream);

/* ---- Block manager (host) and block copy -------------------------------
 * paged-attention-runtime summary, "CORE CAPABILITIES" 1 (fixed 16-token
 * blocks, free-list allocator, reference counting, prefix sharing,
 * copy-on-write, fragmentation metrics); PagedAttention & KV-Cache Memory
 * Management glossary page (the prefix-sharing allocator). A manager owns
 * the bookkeeping of one pool of num_blocks physical blocks: a reference
 * count per block, an optional 64-bit prefix hash per block, a free list
 * that hands out the lowest free id first, and a map from prefix hash to the
 * live block holding it. It never touches device memory; every call is
 * host-only, thread-safe (one call at a time per manager) and returns
 * PA_OK, PA_ERR_NULL, PA_ERR_FULL or PA_ERR_STATE.
 *
 * pa_bm_create returns NULL for num_blocks <= 0 or > 2^31 - 1, block_size
 * <= 0, or no host memory; pa_bm_destroy frees it (NULL is ignored).
 * pa_bm_allocate: with prefix_hash non-NULL and cached, the cached block
 *   gains a reference (*cache_hit = 1); otherwise the lowest free block gets
 *   one reference (and the hash, if given): *cache_hit = 0; PA_ERR_FULL when
 *   none is free. cache_hit may be NULL.
 * pa_bm_share: one more reference to a live block (a fork).
 * pa_bm_release: one reference fewer; at zero the block is free again and
 *   its hash forgotten.
 * pa_bm_copy_on_write: a block about to be written. Held once: *out_block =
 *   block, *must_copy = 0. Shared: a fresh block (no hash) takes the
 *   caller's reference, *out_block = it, *must_copy = 1 -- copy the block's
 *   K/V (and scales) with pa_copy_blocks before writing; PA_ERR_FULL when
 *   none is free.
 * pa_bm_num_free: free blocks (or PA_ERR_NULL).
 * pa_bm_refcounts: the n = num_blocks reference counts into host out[]
 *   (PA_ERR_SHAPE for another n): the eviction choice's refcount input.
 * pa_internal_fragmentation: for a batch's context lengths (host array), the
 *   unused token slots of its blocks over all their slots,
 *   1 - sum(ctx) / (block_size * sum(ceil(ctx / block_size))); 0 for none. */
typedef struct pa_block_manager pa_block_manager;
pa_block_manager* pa_bm_create(int64_t num_blocks, int block_size);
void pa_bm_destroy(pa_block_manager* m);
int pa_bm_allocate(pa_block_manager* m, const uint64_t* prefix_hash, int32_t* block, int* cache_hit);
int pa_bm_share(pa_block_manager* m, int32_t block);
int pa_bm_release(pa_block_manager* m, int32_t block);
int pa_bm_copy_on_write(pa_block_manager* m, int32_t block, int32_t* out_block, int* must_copy);
int64_t pa_bm_num_free(pa_block_manager* m);
int pa_bm_refcounts(pa_block_manager* m, int32_t* out, int64_t n);
double pa_internal_fragmentation(const int32_t* context_lens, int num_seqs, int block_size);

/* Copy whole blocks on the device (the data half of copy-on-write): for each
 * i, block dst_ids[i] of dst_pool receives the bytes_per_block bytes of
 * block src_ids[i] of src_pool (pools laid out as [num_blocks][bytes_per_block];
 * call once per K/V pool and once per scale array). Pairs naming a block
 * outside [0, num_blocks) are skipped; destinations must be distinct and
 * not sources of other pairs. Device pointers; one asynchronous kernel on
 * `stream`. Returns PA_OK (num_pairs == 0 launches nothing), PA_ERR_NULL,
 * PA_ERR_SHAPE, PA_ERR_UNSUPPORTED or PA_ERR_HIP. */
int pa_copy_blocks(const void* src_pool, void* dst_pool, int64_t bytes_per_block,
                   const int32_t* src_ids, const int32_t* dst_ids, int64_t num_pairs,
                   int64_t num_blocks, void* stream);

/* Measurement utility: the HBM read bandwidth a plain streaming read reaches
 * on this device, the practical ceiling next to which the decode's achieved
 * GB/s is read (the decode's bytes are HBM reads; nothing on the pages fixes
 * the ceiling). Reads the `bytes` bytes at device pointer `src` once, with
 * 16-byte non-temporal loads spread over `workgroups` workgroups of 256 lanes
 * (grid-stride over 32 KiB chunks), and writes the XOR of the 32-bit words
 * each workgroup read to sink[workgroup] (device memory, `workgroups`
 * entries), so the result depends on every byte. One asynchronous kernel on
 * `stream`. Returns PA_OK, PA_ERR_NULL, PA_ERR_SHAPE (bytes or workgroups
 * <= 0), PA_ERR_UNSUPPORTED (bytes not a multiple of 16, or src not 16-byte
 * aligned) or PA_ERR_HIP. */
int pa_hbm_read_probe(const void* src, int64_t bytes, uint32_t* sink, int workgroups, void* stream);

/* Measurement utility: the same streaming read, also writing half as many
 * bytes (the INT8 quantizer's mix of two bytes read per byte written), so
 * the quantizer's achieved GB/s can be read next to what the device reaches
 * for that mix. 16-byte word i of `src` (device, `bytes` bytes) becomes
 * 8-byte word i of `dst` (device, bytes / 2 bytes, 8-byte aligned): its low
 * 8 bytes XOR its high 8 bytes. Non-temporal loads and stores, `workgroups`
 * workgroups of 256 lanes. One asynchronous kernel on `stream`. Returns
 * PA_OK, PA_ERR_NULL, PA_ERR_SHAPE (bytes or workgroups <= 0),
 * PA_ERR_UNSUPPORTED (bytes not a multiple of 16, src not 16-byte or dst not
 * 8-byte aligned) or PA_ERR_HIP. */
int pa_hbm_rw_probe(const void* src, int64_t bytes, void* dst, int workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
