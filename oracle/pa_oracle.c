/*
 * CPU oracle for paged single-token decode attention, fp16 and INT8 KV.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it. It shares no code, header or constant with the HIP
 * library; both sides read the same seeded inputs and nothing else.
 *
 * It is the plain definition, written for a reader to check by eye:
 * scalar fp32 arithmetic, no blocking, no fusion, two-pass softmax, OpenMP
 * only over independent (sequence, query head) pairs. Build it with
 * -O2 -fopenmp -ffp-contract=off and without -ffast-math.
 *
 * Sources (the pages, by title and section):
 *  - PagedKV-Fusion README, "Overview" component table: per-(block, head)
 *    quantized decode attention; "Architecture" flowchart: per-block,head
 *    symmetric INT8, online softmax, GQA; "Memory footprint (exact
 *    arithmetic)": one fp32 scale for K and one for V per (block, head).
 *  - paged-attention-runtime summary, "CORE CAPABILITIES" 1 and 2: fixed
 *    16-token blocks, block-table indirection, fp32 accumulation; item 4,
 *    GQA expanded to the query heads.
 *  - PagedAttention & KV-Cache Memory Management (glossary monograph),
 *    section 2.1: physical block = table[t / B], offset = t mod B;
 *    section 5.1: symmetric scaling Q = round(K / S); section 5.2:
 *    A = softmax(Q K^T / sqrt(d)).
 *
 * Readings the pages leave open (each one stated where it is used):
 *  - pool layout [num_blocks][num_kv_heads][block_size][head_dim];
 *  - query head h reads KV head h / (H_q / H_kv) (consecutive groups);
 *  - scale = amax / 127 in fp32; code = clamp(round-half-even(x / scale),
 *    -127, 127) with an IEEE fp32 division; amax = 0 gives scale 0, codes 0;
 *  - INT8 dequantization is float(code) * scale, one fp32 multiply;
 *  - context length 0 gives an all-zero output row;
 *  - appending to an INT8 cache re-scales the tile when the new row raises
 *    its scale (pa_ref_append_kv_int8 states the rule).
 *
 * Parity status: every function here is pinned by the CPU tests (dense
 * fp64 attention on contiguous K/V, invariants, closed forms, exact
 * rational checks of the quantizer, all 65,536 fp16 bit patterns; the
 * appends through decode against dense attention, whole-tile quantization
 * and exact rational re-scaling).
 */
#include <fenv.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { REF_OK = 0, REF_ERR_ARG = -1, REF_ERR_TABLE = -2, REF_ERR_NOMEM = -3 };

/* IEEE 754 binary16 -> binary32, straight from the format's definition:
 * exponent field 0 is subnormal (m * 2^-24), 31 is Inf/NaN, otherwise
 * (1024 + m) * 2^(e - 25). ldexpf is exact for all of these values. */
float pa_ref_half_to_float(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    float v;
    if (e == 0)
        v = ldexpf((float)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexpf((float)(1024 + m), e - 25);
    return sign ? -v : v;
}

void pa_ref_half_to_float_array(const uint16_t* h, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = pa_ref_half_to_float(h[i]);
}

/* Host threads the OpenMP loops use from now on (n <= 0 leaves it as it is);
 * for timing the oracle on fewer cores. */
void pa_ref_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int pa_ref_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Symmetric per-(block, head) INT8 quantization of one pool.                */
/* For each listed physical block b and each KV head h, over the whole       */
/* block_size x head_dim tile (dead slots included; they hold 0):            */
/*   amax  = max |x|                                                         */
/*   scale = amax / 127            (fp32, IEEE division)                     */
/*   code  = clamp(rint(x / scale), -127, 127), rint = round half to even    */
/* scales[b * H + h] receives the scale. Unlisted blocks are left untouched. */
int pa_ref_quantize_kv_int8(const uint16_t* x, int8_t* codes, float* scales,
                            const int32_t* block_ids, int64_t num_ids, int64_t num_blocks,
                            int num_kv_heads, int block_size, int head_dim)
{
    if (!x || !codes || !scales || num_blocks <= 0 || num_kv_heads <= 0 || block_size <= 0 ||
        head_dim <= 0)
        return REF_ERR_ARG;
    int64_t count = block_ids ? num_ids : num_blocks;
    for (int64_t i = 0; i < count; ++i) {
        int64_t b = block_ids ? block_ids[i] : i;
        if (b < 0 || b >= num_blocks) return REF_ERR_TABLE;
    }
    const int64_t tile = (int64_t)block_size * head_dim;
    int ret = REF_OK;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        int64_t b = block_ids ? block_ids[i] : i;
        if (fegetround() != FE_TONEAREST) fesetround(FE_TONEAREST);
        for (int h = 0; h < num_kv_heads; ++h) {
            const int64_t base = (b * num_kv_heads + h) * tile;
            float amax = 0.0f;
            for (int64_t e = 0; e < tile; ++e) {
                float a = fabsf(pa_ref_half_to_float(x[base + e]));
                if (a > amax) amax = a;
            }
            float scale = amax / 127.0f;
            scales[b * num_kv_heads + h] = scale;
            for (int64_t e = 0; e < tile; ++e) {
                int c = 0;
                if (scale != 0.0f) {
                    float r = nearbyintf(pa_ref_half_to_float(x[base + e]) / scale);
                    if (r > 127.0f) r = 127.0f;
                    if (r < -127.0f) r = -127.0f;
                    c = (r == r) ? (int)r : 0; /* NaN input: undefined, write 0 */
                }
                codes[base + e] = (int8_t)c;
            }
        }
    }
    return ret;
}

/* ------------------------------------------------------------------------ */
/* FP8 (OCP E4M3) per-(block, head) quantization.                            */
/* The monograph's section 5.1 quantizes K and V with symmetric scales to    */
/* FP8 or INT8 (Q_K = round(K / S_K)) and keeps one scale per block; the FP8 */
/* format is not named there, and the reading here is OCP 8-bit E4M3: sign, */
/* 4 exponent bits (bias 7), 3 mantissa bits, no infinities, S.1111.111 NaN, */
/* largest finite 448. Per (block, head) tile, like the INT8 quantizer:      */
/*   amax  = max |x|;  scale = amax / 448      (fp32, IEEE division)          */
/*   code  = E4M3(x / scale)                   (IEEE division, then the      */
/*           nearest E4M3 value, ties to an even mantissa, beyond 448 kept   */
/*           at 448)                                                          */
/* scale 0 gives code 0. A code decodes to fp32 exactly.                     */

/* E4M3 code -> value (exact in fp32). */
float pa_ref_e4m3_to_float(uint8_t c)
{
    int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    float v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexpf((float)m, -9);          /* subnormal: m * 2^-9 */
    else
        v = ldexpf((float)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

/* fp32 -> E4M3, round to nearest (ties to even), saturating at +-448.
 * The step between neighbouring E4M3 values at |y| is 2^(max(E, -6) - 3),
 * E = floor(log2 |y|); |y| / step is exact, rint rounds it half to even. */
uint8_t pa_ref_float_to_e4m3(float y)
{
    if (y != y) return 0x7F;
    uint8_t sign = signbit(y) ? 0x80 : 0;
    float a = fabsf(y);
    if (a == 0.0f) return sign;
    int E;
    frexpf(a, &E); /* a = f 2^E, f in [0.5, 1): floor(log2 a) = E - 1 */
    E -= 1;
    if (E < -6) E = -6;
    float steps = nearbyintf(ldexpf(a, 3 - E)); /* multiples of the step */
    float q = ldexpf(steps, E - 3);
    if (q > 448.0f) q = 448.0f;
    /* encode q: subnormal below 2^-6 */
    if (q < 0.015625f) return sign | (uint8_t)(int)ldexpf(q, 9);
    int e2;
    float f = frexpf(q, &e2); /* q = f 2^e2, f in [0.5, 1) */
    int m = (int)ldexpf(f, 4) - 8; /* q = (1 + m/8) 2^(e2-1) */
    return sign | (uint8_t)(((e2 - 1 + 7) << 3) | m);
}

int pa_ref_quantize_kv_fp8(const uint16_t* x, uint8_t* codes, float* scales,
                           const int32_t* block_ids, int64_t num_ids, int64_t num_blocks,
                           int num_kv_heads, int block_size, int head_dim)
{
    if (!x || !codes || !scales || num_blocks <= 0 || num_kv_heads <= 0 || block_size <= 0 ||
        head_dim <= 0)
        return REF_ERR_ARG;
    int64_t count = block_ids ? num_ids : num_blocks;
    for (int64_t i = 0; i < count; ++i) {
        int64_t b = block_ids ? block_ids[i] : i;
        if (b < 0 || b >= num_blocks) return REF_ERR_TABLE;
    }
    const int64_t tile = (int64_t)block_size * head_dim;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        int64_t b = block_ids ? block_ids[i] : i;
        if (fegetround() != FE_TONEAREST) fesetround(FE_TONEAREST);
        for (int h = 0; h < num_kv_heads; ++h) {
            const int64_t base = (b * num_kv_heads + h) * tile;
            float amax = 0.0f;
            for (int64_t e = 0; e < tile; ++e) {
                float a = fabsf(pa_ref_half_to_float(x[base + e]));
                if (a > amax) amax = a;
            }
            float scale = amax / 448.0f;
            scales[b * num_kv_heads + h] = scale;
            for (int64_t e = 0; e < tile; ++e)
                codes[base + e] = scale != 0.0f ? pa_ref_float_to_e4m3(pa_ref_half_to_float(x[base + e]) / scale)
                                                : 0;
        }
    }
    return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* Single-query attention for one (sequence, query head) over gathered rows. */
/*   s_t = softmax_scale * sum_j q_j k_tj                                    */
/*   m   = max_t s_t,  p_t = exp(s_t - m),  l = sum_t p_t                    */
/*   out_j = (sum_t p_t v_tj) / l                                            */
/* Two passes over the scores: the plain definition of softmax(q K^T/sqrt d)V*/
static void attend(const float* q, const float* K, const float* V, int n, int d,
                   float softmax_scale, float* out, float* weights, float* scores)
{
    if (n <= 0) {
        for (int j = 0; j < d; ++j) out[j] = 0.0f;
        return;
    }
    for (int t = 0; t < n; ++t) {
        float dot = 0.0f;
        for (int j = 0; j < d; ++j) dot += q[j] * K[(int64_t)t * d + j];
        scores[t] = softmax_scale * dot;
    }
    float m = scores[0];
    for (int t = 1; t < n; ++t)
        if (scores[t] > m) m = scores[t];
    float l = 0.0f;
    for (int t = 0; t < n; ++t) {
        scores[t] = expf(scores[t] - m);
        l += scores[t];
    }
    for (int j = 0; j < d; ++j) {
        float acc = 0.0f;
        for (int t = 0; t < n; ++t) acc += scores[t] * V[(int64_t)t * d + j];
        out[j] = acc / l;
    }
    if (weights)
        for (int t = 0; t < n; ++t) weights[t] = scores[t] / l;
}

/* Shared argument check: shapes, and every table entry a sequence reads must
 * name a block of the pool. */
static int check_args(const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                      int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                      int max_blocks_per_seq, int64_t num_blocks)
{
    if (!block_tables || !context_lens || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
        head_dim <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0)
        return REF_ERR_ARG;
    if (num_q_heads % num_kv_heads) return REF_ERR_ARG;
    for (int s = 0; s < num_seqs; ++s) {
        int n = context_lens[s];
        if (n < 0 || n > max_blocks_per_seq * block_size) return REF_ERR_ARG;
        int nb = (n + block_size - 1) / block_size;
        for (int i = 0; i < nb; ++i) {
            int32_t b = block_tables[(int64_t)s * max_blocks_per_seq + i];
            if (b < 0 || b >= num_blocks) return REF_ERR_TABLE;
        }
    }
    return REF_OK;
}

/* Gather one sequence's K and V for one KV head through the block table:
 * token t lives in block table[s][t / B] at slot t mod B (glossary
 * monograph, section 2.1). fp16 pools when k16 != NULL, INT8 otherwise
 * (dequantized as float(code) * scale of that (block, head)). */
static void gather(int s, int kvh, int n, const int32_t* block_tables, int max_blocks_per_seq,
                   int num_kv_heads, int block_size, int head_dim, const uint16_t* k16,
                   const uint16_t* v16, const int8_t* k8, const int8_t* v8, const uint8_t* kf8,
                   const uint8_t* vf8, const float* ks, const float* vs, float* K, float* V)
{
    for (int t = 0; t < n; ++t) {
        int64_t b = block_tables[(int64_t)s * max_blocks_per_seq + t / block_size];
        int o = t % block_size;
        int64_t row = ((b * num_kv_heads + kvh) * block_size + o) * head_dim;
        for (int j = 0; j < head_dim; ++j) {
            if (k16) {
                K[(int64_t)t * head_dim + j] = pa_ref_half_to_float(k16[row + j]);
                V[(int64_t)t * head_dim + j] = pa_ref_half_to_float(v16[row + j]);
            } else if (kf8) {
                float sk = ks[b * num_kv_heads + kvh];
                float sv = vs[b * num_kv_heads + kvh];
                K[(int64_t)t * head_dim + j] = pa_ref_e4m3_to_float(kf8[row + j]) * sk;
                V[(int64_t)t * head_dim + j] = pa_ref_e4m3_to_float(vf8[row + j]) * sv;
            } else {
                float sk = ks[b * num_kv_heads + kvh];
                float sv = vs[b * num_kv_heads + kvh];
                K[(int64_t)t * head_dim + j] = (float)k8[row + j] * sk;
                V[(int64_t)t * head_dim + j] = (float)v8[row + j] * sv;
            }
        }
    }
}

static int decode_common(const uint16_t* q, const uint16_t* k16, const uint16_t* v16,
                         const int8_t* k8, const int8_t* v8, const uint8_t* kf8,
                         const uint8_t* vf8, const float* ks, const float* vs,
                         const int32_t* block_tables, const int32_t* context_lens, float* out,
                         int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                         int block_size, int max_blocks_per_seq, int64_t num_blocks,
                         float softmax_scale, const int32_t* seq_ids, int num_seq_ids,
                         float* weights, int weights_stride)
{
    if (!q || !out) return REF_ERR_ARG;
    int rc = check_args(block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads,
                        head_dim, block_size, max_blocks_per_seq, num_blocks);
    if (rc) return rc;
    const int count = seq_ids ? num_seq_ids : num_seqs;
    for (int i = 0; i < count; ++i) {
        int s = seq_ids ? seq_ids[i] : i;
        if (s < 0 || s >= num_seqs) return REF_ERR_ARG;
        if (weights && context_lens[s] > weights_stride) return REF_ERR_ARG;
    }
    const int group = num_q_heads / num_kv_heads;
    const int64_t pairs = (int64_t)count * num_q_heads;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t pi = 0; pi < pairs; ++pi) {
        int s = seq_ids ? seq_ids[pi / num_q_heads] : (int)(pi / num_q_heads);
        int h = (int)(pi % num_q_heads);
        int kvh = h / group; /* consecutive GQA groups */
        int n = context_lens[s];
        size_t rows = (size_t)(n > 0 ? n : 1);
        float* K = (float*)malloc(rows * head_dim * sizeof(float));
        float* V = (float*)malloc(rows * head_dim * sizeof(float));
        float* sc = (float*)malloc(rows * sizeof(float));
        float* qf = (float*)malloc((size_t)head_dim * sizeof(float));
        if (!K || !V || !sc || !qf) {
#pragma omp atomic write
            failed = 1;
        } else {
            const int64_t qrow = ((int64_t)s * num_q_heads + h) * head_dim;
            for (int j = 0; j < head_dim; ++j) qf[j] = pa_ref_half_to_float(q[qrow + j]);
            gather(s, kvh, n, block_tables, max_blocks_per_seq, num_kv_heads, block_size,
                   head_dim, k16, v16, k8, v8, kf8, vf8, ks, vs, K, V);
            float* w = weights ? weights + ((int64_t)s * num_q_heads + h) * weights_stride : NULL;
            attend(qf, K, V, n, head_dim, softmax_scale, out + qrow, w, sc);
        }
        free(K);
        free(V);
        free(sc);
        free(qf);
    }
    return failed ? REF_ERR_NOMEM : REF_OK;
}

/* fp16 KV: q [S][H_q][d] fp16, pools [NB][H_kv][B][d] fp16, out [S][H_q][d] fp32.
 * seq_ids (optional) restricts the work to the listed sequences; weights
 * (optional, [S][H_q][weights_stride]) receives the normalised softmax
 * weights p_t / l of each computed row. */
int pa_ref_paged_decode_f16(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                            const int32_t* block_tables, const int32_t* context_lens, float* out,
                            int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                            int block_size, int max_blocks_per_seq, int64_t num_blocks,
                            float softmax_scale, const int32_t* seq_ids, int num_seq_ids,
                            float* weights, int weights_stride)
{
    if (!k_pool || !v_pool) return REF_ERR_ARG;
    return decode_common(q, k_pool, v_pool, NULL, NULL, NULL, NULL, NULL, NULL, block_tables, context_lens,
                         out, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                         max_blocks_per_seq, num_blocks, softmax_scale, seq_ids, num_seq_ids,
                         weights, weights_stride);
}

/* INT8 KV: codes [NB][H_kv][B][d] int8 with scales [NB][H_kv] fp32 for K and
 * for V; every K/V element is dequantized as float(code) * scale first, then
 * the same attention as the fp16 path runs on the dequantized rows. */
int pa_ref_paged_decode_int8(const uint16_t* q, const int8_t* k_codes, const int8_t* v_codes,
                             const float* k_scale, const float* v_scale,
                             const int32_t* block_tables, const int32_t* context_lens, float* out,
                             int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                             int block_size, int max_blocks_per_seq, int64_t num_blocks,
                             float softmax_scale, const int32_t* seq_ids, int num_seq_ids,
                             float* weights, int weights_stride)
{
    if (!k_codes || !v_codes || !k_scale || !v_scale) return REF_ERR_ARG;
    return decode_common(q, NULL, NULL, k_codes, v_codes, NULL, NULL, k_scale, v_scale, block_tables,
                         context_lens, out, num_seqs, num_q_heads, num_kv_heads, head_dim,
                         block_size, max_blocks_per_seq, num_blocks, softmax_scale, seq_ids,
                         num_seq_ids, weights, weights_stride);
}

/* FP8 KV: E4M3 codes [NB][H_kv][B][d] with scales [NB][H_kv] fp32 for K and
 * for V; every element is decoded exactly and multiplied by its scale (one
 * fp32 multiply), then the same attention runs. */
int pa_ref_paged_decode_fp8(const uint16_t* q, const uint8_t* k_codes, const uint8_t* v_codes,
                            const float* k_scale, const float* v_scale,
                            const int32_t* block_tables, const int32_t* context_lens, float* out,
                            int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                            int block_size, int max_blocks_per_seq, int64_t num_blocks,
                            float softmax_scale, const int32_t* seq_ids, int num_seq_ids,
                            float* weights, int weights_stride)
{
    if (!k_codes || !v_codes || !k_scale || !v_scale) return REF_ERR_ARG;
    return decode_common(q, NULL, NULL, NULL, NULL, k_codes, v_codes, k_scale, v_scale,
                         block_tables, context_lens, out, num_seqs, num_q_heads, num_kv_heads,
                         head_dim, block_size, max_blocks_per_seq, num_blocks, softmax_scale,
                         seq_ids, num_seq_ids, weights, weights_stride);
}

/* ------------------------------------------------------------------------ */
/* Append: one new token per sequence into the paged cache.                   */
/* Token t = positions[s] of sequence s goes to block                        */
/* b = block_tables[s][t / block_size] at slot o = t mod block_size           */
/* (glossary monograph, section 2.1; PagedAttention article, "Kernel          */
/* Mechanics": the new K/V are written into the block at                      */
/* phys_block_id * B + token_offset). A negative position, a position past   */
/* the table row, or a table entry outside the pool appends nothing.          */
/* k_new, v_new: fp16 [num_seqs][num_kv_heads][head_dim].                     */

/* The append slot of sequence s, or -1 when it appends nothing. */
static int64_t append_block(const int32_t* block_tables, const int32_t* positions, int s,
                            int block_size, int max_blocks_per_seq, int64_t num_blocks, int* slot)
{
    int t = positions[s];
    if (t < 0 || t / block_size >= max_blocks_per_seq) return -1;
    int64_t b = block_tables[(int64_t)s * max_blocks_per_seq + t / block_size];
    if (b < 0 || b >= num_blocks) return -1;
    *slot = t % block_size;
    return b;
}

int pa_ref_append_kv_f16(const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_pool,
                         uint16_t* v_pool, const int32_t* block_tables, const int32_t* positions,
                         int num_seqs, int num_kv_heads, int block_size, int head_dim,
                         int max_blocks_per_seq, int64_t num_blocks)
{
    if (!k_new || !v_new || !k_pool || !v_pool || !block_tables || !positions || num_seqs < 0 ||
        num_kv_heads <= 0 || block_size <= 0 || head_dim <= 0 || max_blocks_per_seq <= 0 ||
        num_blocks <= 0)
        return REF_ERR_ARG;
    for (int s = 0; s < num_seqs; ++s) {
        int o;
        int64_t b = append_block(block_tables, positions, s, block_size, max_blocks_per_seq,
                                 num_blocks, &o);
        if (b < 0) continue;
        for (int h = 0; h < num_kv_heads; ++h) {
            int64_t dst = ((b * num_kv_heads + h) * block_size + o) * head_dim;
            int64_t src = ((int64_t)s * num_kv_heads + h) * head_dim;
            for (int j = 0; j < head_dim; ++j) {
                k_pool[dst + j] = k_new[src + j];
                v_pool[dst + j] = v_new[src + j];
            }
        }
    }
    return REF_OK;
}

/* The quantizer of pa_ref_quantize_kv_int8 for one value at a given scale:
 * 0 when the scale is 0, else clamp(rint(v / scale), -127, 127). */
static int8_t quantize_one(float v, float scale)
{
    if (scale == 0.0f) return 0;
    float r = nearbyintf(v / scale);
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    return (int8_t)((r == r) ? (int)r : 0);
}

/* INT8 append. The pages define the per-(block, head) symmetric quantizer
 * (PagedKV-Fusion README, "Overview"; glossary monograph, section 5.1) but
 * not how a cache that holds only codes takes a new token; the reading used
 * here keeps the tile quantized with one scale for its live rows:
 *   x = the new row (head_dim values), s_old = the tile's scale,
 *   s_new = amax(x) / 127 (fp32, IEEE division);
 *   o == 0: the block's first token (no live row yet): scale = s_new,
 *           row 0 = q(x, s_new);
 *   o > 0, s_new <= s_old: row o = q(x, s_old), scale kept;
 *   o > 0, s_new >  s_old: the tile grows to s_new: each live row r < o is
 *           dequantized (code * s_old, one fp32 multiply) and quantized
 *           again, c = q(code * s_old, s_new); row o = q(x, s_new);
 *           scale = s_new.
 * Rows after o are not touched. The same rule runs for K and for V, each
 * with its own scale. */
static void append_tile_int8(const uint16_t* x, int8_t* tile, float* scale, int o, int head_dim)
{
    float amax = 0.0f;
    for (int j = 0; j < head_dim; ++j) {
        float a = fabsf(pa_ref_half_to_float(x[j]));
        if (a > amax) amax = a;
    }
    float s_new = amax / 127.0f;
    float s_old = *scale;
    float s = s_new;
    if (o > 0 && s_new <= s_old) {
        s = s_old;
    } else if (o > 0) {
        for (int r = 0; r < o; ++r)
            for (int j = 0; j < head_dim; ++j) {
                float v = (float)tile[(int64_t)r * head_dim + j] * s_old;
                tile[(int64_t)r * head_dim + j] = quantize_one(v, s_new);
            }
    }
    for (int j = 0; j < head_dim; ++j)
        tile[(int64_t)o * head_dim + j] = quantize_one(pa_ref_half_to_float(x[j]), s);
    *scale = s;
}

int pa_ref_append_kv_int8(const uint16_t* k_new, const uint16_t* v_new, int8_t* k_codes,
                          int8_t* v_codes, float* k_scale, float* v_scale,
                          const int32_t* block_tables, const int32_t* positions, int num_seqs,
                          int num_kv_heads, int block_size, int head_dim, int max_blocks_per_seq,
                          int64_t num_blocks)
{
    if (!k_new || !v_new || !k_codes || !v_codes || !k_scale || !v_scale || !block_tables ||
        !positions || num_seqs < 0 || num_kv_heads <= 0 || block_size <= 0 || head_dim <= 0 ||
        max_blocks_per_seq <= 0 || num_blocks <= 0)
        return REF_ERR_ARG;
    if (fegetround() != FE_TONEAREST) fesetround(FE_TONEAREST);
    for (int s = 0; s < num_seqs; ++s) {
        int o;
        int64_t b = append_block(block_tables, positions, s, block_size, max_blocks_per_seq,
                                 num_blocks, &o);
        if (b < 0) continue;
        for (int h = 0; h < num_kv_heads; ++h) {
            int64_t tile = (b * num_kv_heads + h) * block_size * (int64_t)head_dim;
            int64_t src = ((int64_t)s * num_kv_heads + h) * head_dim;
            append_tile_int8(k_new + src, k_codes + tile, k_scale + b * num_kv_heads + h, o,
                             head_dim);
            append_tile_int8(v_new + src, v_codes + tile, v_scale + b * num_kv_heads + h, o,
                             head_dim);
        }
    }
    return REF_OK;
}
