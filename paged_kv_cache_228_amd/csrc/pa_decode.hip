// Paged single-token decode attention for gfx950 (MI355X): the context-
// partition kernel and the split-K merge kernel.
//
// What is computed (paged-attention-runtime summary, "CORE CAPABILITIES" 2:
// block-table indirection, online single-pass softmax, wave-level reductions,
// vectorized loads, fp32 accumulation; PagedKV-Fusion README, "Overview":
// per-(block, head) INT8 decode attention with GQA): for sequence s and query
// head h, out = sum_t softmax_t(scale * q.k_t) v_t over the sequence's tokens,
// K/V reached through the block table (glossary monograph, section 2.1).
//
// Work decomposition: one workgroup of four waves per (sequence, KV head,
// context partition). The workgroup stages the partition's block ids in LDS;
// wave w takes the partition's blocks w, w+4, ... and keeps its own online
// softmax state (m, l, acc) for all G query heads of the KV head, so each K/V
// tile is read from HBM once per decode step. The four waves' states are
// merged through LDS; with more than one partition the partition's state goes
// to the workspace and a second kernel merges the partitions (log-sum-exp
// combine). Scores live in the log2 domain (scale * log2 e folded into one
// multiply) so the exponentials are single v_exp_f32 instructions.
//
// Register layout of one (block, KV head) tile, 16 rows x D elements:
// a wave reads it with 16-byte loads, lane + 64*l reading chunk lane + 64*l
// of the row-major tile, so every load instruction moves 1 KiB of contiguous
// bytes. R = D / (elements per chunk) lanes share a token row; lane owns the
// dims [ (lane % R) * EPC, +EPC ) of rows lane / R + l * (64 / R). Dot
// products reduce across the R lanes of a row with DPP row permutations.
#include "pa_internal.h"

namespace pa {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr uint32_t kRsrcWord3 = 0x00020000u;  // gfx9 raw buffer: 32-bit data format

// Element i of a 4-dword vector (i a compile-time constant after unrolling).
// Written as a select chain: subscripting an array of ext-vector values with
// a loop index inside nested unrolled loops lost elements with this compiler.
__device__ __forceinline__ uint32_t word(const u32x4& v, int i)
{
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of R consecutive lanes (R = 4, 8 or 16) using
// row-local DPP: swap neighbours, swap pairs, mirror halves of 8, mirror
// halves of 16. Every lane of a group ends with the identical total.
template <int R>
__device__ __forceinline__ float group_sum(float x)
{
    static_assert(R == 4 || R == 8 || R == 16, "group of 4, 8 or 16 lanes");
    x += dpp<0xB1>(x);  // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);  // quad_perm [2,3,0,1]
    if constexpr (R >= 8) x += dpp<0x141>(x);   // row_half_mirror
    if constexpr (R >= 16) x += dpp<0x140>(x);  // row_mirror
    return x;
}

// Reductions across the groups: over lanes that share lane % R.
template <int R>
__device__ __forceinline__ float xgroup_sum(float x)
{
#pragma unroll
    for (int m = R; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
    return x;
}

template <int R>
__device__ __forceinline__ float xgroup_max(float x)
{
#pragma unroll
    for (int m = R; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
    return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Four signed INT8 codes (one dword) to two pairs of exact fp16 values.
// Flipping each sign bit gives c + 128 in [1, 255]; placing that byte as the
// low mantissa bits under the fp16 pattern 0x64xx gives 1024 + c + 128, and
// subtracting 1152 leaves c exactly.
__device__ __forceinline__ void codes_to_h2(uint32_t w, h2_t& lo, h2_t& hi)
{
    const uint32_t u = w ^ 0x80808080u;
    const h2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    lo = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - bias;
    hi = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - bias;
}

template <int D, bool I8>
struct Cfg {
    static constexpr int EB = I8 ? 1 : 2;           // bytes per element
    static constexpr int EPC = 16 / EB;             // elements per 16-byte chunk
    static constexpr int NP = EPC / 2;              // fp16 pairs per chunk
    static constexpr int R = D / EPC;               // lanes per token row
    static constexpr int RPL = 64 / R;              // rows per wave load
    static constexpr int L = kBlockTokens / RPL;    // loads per tile
    static constexpr int TILE = kBlockTokens * D * EB;  // bytes per (block, head) tile
    static_assert(L >= 1 && RPL * L == kBlockTokens, "tile must split into whole loads");
};

template <int D, bool I8>
struct Tile {
    u32x4 k[Cfg<D, I8>::L];
    u32x4 v[Cfg<D, I8>::L];
    float ksc, vsc;  // INT8 scales of this (block, head); 1 for fp16
    int tok0;        // first token position of the block in its sequence
};

// Issue the loads of one tile. bytes == 0 (no block, or an id outside the
// pool) makes every buffer load return zeros without touching memory.
template <int D, bool I8>
__device__ __forceinline__ void load_tile(Tile<D, I8>& t, const DecodeArgs& a, int bid, bool valid,
                                          int kvh, int tok0, int lane)
{
    using C = Cfg<D, I8>;
    const bool in_pool = valid && (uint64_t)(int64_t)bid < (uint64_t)a.num_blocks;
    const int64_t b = in_pool ? bid : 0;
    const int64_t off = (b * a.num_kv_heads + kvh) * (int64_t)C::TILE;
    const int bytes = in_pool ? C::TILE : 0;
    rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(static_cast<const char*>(a.k) + off), (short)0, bytes, kRsrcWord3);
    rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(static_cast<const char*>(a.v) + off), (short)0, bytes, kRsrcWord3);
#pragma unroll
    for (int l = 0; l < C::L; ++l)
        t.k[l] = __builtin_amdgcn_raw_buffer_load_b128(rk, (lane + 64 * l) * 16, 0, 0);
#pragma unroll
    for (int l = 0; l < C::L; ++l)
        t.v[l] = __builtin_amdgcn_raw_buffer_load_b128(rv, (lane + 64 * l) * 16, 0, 0);
    if constexpr (I8) {
        const int64_t si = b * a.num_kv_heads + kvh;
        t.ksc = in_pool ? a.k_scale[si] : 0.0f;
        t.vsc = in_pool ? a.v_scale[si] : 0.0f;
    } else {
        t.ksc = 1.0f;
        t.vsc = 1.0f;
    }
    t.tok0 = tok0;
}

template <int D, int G, bool I8>
struct State {
    float m[G];                       // running max of log2-domain scores (wave-uniform)
    float l[G];                       // this lane's share of the softmax denominator
    float acc[G][Cfg<D, I8>::EPC];    // this lane's share of sum p * v for its dims
};

template <int D, int G, bool I8>
__device__ __forceinline__ void process_tile(State<D, G, I8>& st, Tile<D, I8>& t,
                                             const h2_t (&q)[G][Cfg<D, I8>::NP], int ctx,
                                             float scale_log2, int row0)
{
    using C = Cfg<D, I8>;
    float sc[C::L][G];
    const float sl = scale_log2 * t.ksc;
#pragma unroll
    for (int l = 0; l < C::L; ++l) {
        h2_t kh[C::NP];
        if constexpr (I8) {
#pragma unroll
            for (int w = 0; w < 4; ++w) codes_to_h2(word(t.k[l], w), kh[2 * w], kh[2 * w + 1]);
        } else {
#pragma unroll
            for (int w = 0; w < 4; ++w) kh[w] = __builtin_bit_cast(h2_t, word(t.k[l], w));
        }
#pragma unroll
        for (int i = 0; i < G; ++i) {
            float part = 0.0f;
#pragma unroll
            for (int n = 0; n < C::NP; ++n) part = __builtin_amdgcn_fdot2(q[i][n], kh[n], part, false);
            sc[l][i] = group_sum<C::R>(part) * sl;
        }
    }
    if (t.tok0 + kBlockTokens > ctx) {  // last block of the sequence: mask the tail rows
#pragma unroll
        for (int l = 0; l < C::L; ++l) {
            if (t.tok0 + row0 + l * C::RPL >= ctx) {
#pragma unroll
                for (int i = 0; i < G; ++i) sc[l][i] = -INFINITY;
                t.v[l] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
    float p[C::L][G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        float tmax = sc[0][i];
#pragma unroll
        for (int l = 1; l < C::L; ++l) tmax = fmaxf(tmax, sc[l][i]);
        tmax = xgroup_max<C::R>(tmax);
        const float mn = fmaxf(st.m[i], tmax);
        if (mn > st.m[i]) {
            const float alpha = fast_exp2(st.m[i] - mn);
            st.l[i] *= alpha;
#pragma unroll
            for (int e = 0; e < C::EPC; ++e) st.acc[i][e] *= alpha;
            st.m[i] = mn;
        }
#pragma unroll
        for (int l = 0; l < C::L; ++l) {
            p[l][i] = fast_exp2(sc[l][i] - st.m[i]);
            st.l[i] += p[l][i];
        }
    }
#pragma unroll
    for (int l = 0; l < C::L; ++l) {
        h2_t vh[C::NP];
        if constexpr (I8) {
#pragma unroll
            for (int w = 0; w < 4; ++w) codes_to_h2(word(t.v[l], w), vh[2 * w], vh[2 * w + 1]);
        } else {
#pragma unroll
            for (int w = 0; w < 4; ++w) vh[w] = __builtin_bit_cast(h2_t, word(t.v[l], w));
        }
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const float pw = p[l][i] * t.vsc;
#pragma unroll
            for (int n = 0; n < C::NP; ++n) {
                st.acc[i][2 * n] = __builtin_fmaf(pw, (float)vh[n].x, st.acc[i][2 * n]);
                st.acc[i][2 * n + 1] = __builtin_fmaf(pw, (float)vh[n].y, st.acc[i][2 * n + 1]);
            }
        }
    }
}

template <int D, int G, bool I8>
__global__ __launch_bounds__(kThreads) void decode_partition_kernel(DecodeArgs a)
{
    using C = Cfg<D, I8>;
    const int p = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int hq0 = kvh * G;

    int ctx = a.ctx[s];
    ctx = ctx < 0 ? 0 : (ctx > a.max_blocks * kBlockTokens ? a.max_blocks * kBlockTokens : ctx);
    if (ctx == 0) {  // empty context: the first partition writes a zero row
        if (p == 0)
            for (int e = threadIdx.x; e < G * D; e += kThreads)
                a.out[((int64_t)s * a.num_q_heads + hq0) * D + e] = 0.0f;
        return;
    }
    const int nblk = (ctx + kBlockTokens - 1) / kBlockTokens;
    const int b0 = p * a.part_blocks;
    if (b0 >= nblk) return;
    const int nloc = min(nblk - b0, a.part_blocks);
    const int nparts = (nblk + a.part_blocks - 1) / a.part_blocks;

    __shared__ int ids[kMaxPartitionBlocks];
    __shared__ float red_m[kWaves][G];
    __shared__ float red_l[kWaves][G];
    __shared__ float red_acc[kWaves][G][D];

    if ((int)threadIdx.x < nloc) ids[threadIdx.x] = a.tables[(int64_t)s * a.max_blocks + b0 + threadIdx.x];

    // query rows of the G heads, the lane's dims only, as fp16 pairs
    const int chunk = lane % C::R;
    const int row0 = lane / C::R;
    h2_t q[G][C::NP];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const u32x4* qp = reinterpret_cast<const u32x4*>(
            static_cast<const _Float16*>(a.q) + ((int64_t)s * a.num_q_heads + hq0 + i) * D +
            chunk * C::EPC);
#pragma unroll
        for (int c = 0; c < C::EPC / 8; ++c) {
            const u32x4 w = qp[c];
#pragma unroll
            for (int k = 0; k < 4; ++k) q[i][4 * c + k] = __builtin_bit_cast(h2_t, word(w, k));
        }
    }
    State<D, G, I8> st;
#pragma unroll
    for (int i = 0; i < G; ++i) {
        st.m[i] = -INFINITY;
        st.l[i] = 0.0f;
#pragma unroll
        for (int e = 0; e < C::EPC; ++e) st.acc[i][e] = 0.0f;
    }
    __syncthreads();

    // software pipeline: the next tile's loads are in flight while the
    // current tile is processed; past the end the loads are zero-sized
    if (wave < nloc) {
        Tile<D, I8> ta, tb;
        int j = wave;
        load_tile<D, I8>(ta, a, uniform(ids[j]), true, kvh, (b0 + j) * kBlockTokens, lane);
        while (true) {
            int jn = j + kWaves;
            load_tile<D, I8>(tb, a, uniform(ids[jn < nloc ? jn : j]), jn < nloc, kvh,
                             (b0 + jn) * kBlockTokens, lane);
            process_tile<D, G, I8>(st, ta, q, ctx, a.scale_log2, row0);
            j = jn;
            if (j >= nloc) break;
            jn = j + kWaves;
            load_tile<D, I8>(ta, a, uniform(ids[jn < nloc ? jn : j]), jn < nloc, kvh,
                             (b0 + jn) * kBlockTokens, lane);
            process_tile<D, G, I8>(st, tb, q, ctx, a.scale_log2, row0);
            j = jn;
            if (j >= nloc) break;
        }
    }

    // wave epilogue: fold the row groups together
#pragma unroll
    for (int i = 0; i < G; ++i) {
        st.l[i] = xgroup_sum<C::R>(st.l[i]);
#pragma unroll
        for (int e = 0; e < C::EPC; ++e) st.acc[i][e] = xgroup_sum<C::R>(st.acc[i][e]);
    }
    if (lane < C::R) {
#pragma unroll
        for (int i = 0; i < G; ++i)
#pragma unroll
            for (int e = 0; e < C::EPC; ++e) red_acc[wave][i][chunk * C::EPC + e] = st.acc[i][e];
    }
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < G; ++i) {
            red_m[wave][i] = st.m[i];
            red_l[wave][i] = st.l[i];
        }
    }
    __syncthreads();

    // workgroup epilogue: merge the four waves, then write the output row or
    // this partition's partial state
    for (int e = threadIdx.x; e < G * D; e += kThreads) {
        const int i = e / D, j = e % D;
        float M = red_m[0][i];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, red_m[w][i]);
        float Lsum = 0.0f, A = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = fast_exp2(red_m[w][i] - M);
            Lsum += red_l[w][i] * f;
            A += red_acc[w][i][j] * f;
        }
        const int64_t row = (int64_t)s * a.num_q_heads + hq0 + i;
        if (nparts == 1) {
            a.out[row * D + j] = A / Lsum;
        } else {
            const int64_t slot = row * a.max_parts + p;
            a.ws[slot * D + j] = A;
            if (j == 0) {
                const int64_t n = (int64_t)a.num_seqs * a.num_q_heads * a.max_parts;
                a.ws[n * D + slot] = M;
                a.ws[n * (D + 1) + slot] = Lsum;
            }
        }
    }
}

// Split-K merge: out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,
// M = max_p m_p. One wave per (sequence, query head).
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a)
{
    const int h = blockIdx.x, s = blockIdx.y;
    const int lane = threadIdx.x;
    int ctx = a.ctx[s];
    ctx = ctx < 0 ? 0 : (ctx > a.max_blocks * kBlockTokens ? a.max_blocks * kBlockTokens : ctx);
    const int nblk = (ctx + kBlockTokens - 1) / kBlockTokens;
    const int nparts = (nblk + a.part_blocks - 1) / a.part_blocks;
    if (nparts <= 1) return;  // written by the partition kernel

    const int64_t row = (int64_t)s * a.num_q_heads + h;
    const int64_t n = (int64_t)a.num_seqs * a.num_q_heads * a.max_parts;
    const float* acc = a.ws + row * a.max_parts * D;
    const float* ms = a.ws + n * D + row * a.max_parts;
    const float* ls = a.ws + n * (D + 1) + row * a.max_parts;

    float M = -INFINITY;
    for (int i = lane; i < nparts; i += 64) M = fmaxf(M, ms[i]);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
    float Lsum = 0.0f;
    for (int i = lane; i < nparts; i += 64) Lsum += ls[i] * fast_exp2(ms[i] - M);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) Lsum += __shfl_xor(Lsum, m, 64);

    __shared__ float wts[64];
    float o[D / 64];
#pragma unroll
    for (int k = 0; k < D / 64; ++k) o[k] = 0.0f;
    for (int base = 0; base < nparts; base += 64) {
        const int i = base + lane;
        wts[lane] = i < nparts ? fast_exp2(ms[i] - M) : 0.0f;
        __syncthreads();
        const int cnt = min(64, nparts - base);
        for (int k2 = 0; k2 < cnt; ++k2) {
            const float w = wts[k2];
#pragma unroll
            for (int k = 0; k < D / 64; ++k) o[k] += w * acc[(int64_t)(base + k2) * D + k * 64 + lane];
        }
        __syncthreads();
    }
    const float inv = 1.0f / Lsum;
#pragma unroll
    for (int k = 0; k < D / 64; ++k) a.out[row * D + k * 64 + lane] = o[k] * inv;
}

template <int D, int G, bool I8>
hipError_t launch_valu(const DecodeArgs& a, hipStream_t st)
{
    const dim3 grid(a.max_parts, a.num_kv_heads, a.num_seqs);
    hipLaunchKernelGGL((decode_partition_kernel<D, G, I8>), grid, dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <int D, bool I8>
hipError_t launch_valu_d(const DecodeArgs& a, int group, hipStream_t st)
{
    switch (group) {
        case 1: return launch_valu<D, 1, I8>(a, st);
        case 2: return launch_valu<D, 2, I8>(a, st);
        case 3: return launch_valu<D, 3, I8>(a, st);
        case 4: return launch_valu<D, 4, I8>(a, st);
        case 5: return launch_valu<D, 5, I8>(a, st);
        case 6: return launch_valu<D, 6, I8>(a, st);
        case 7: return launch_valu<D, 7, I8>(a, st);
        case 8: return launch_valu<D, 8, I8>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Partition kernel on the vector ALUs (one four-wave workgroup per
// partition, every lane reducing its own dims); kept for comparison with the
// matrix-core kernel.
hipError_t launch_decode_partitions_valu(const DecodeArgs& a, int head_dim, int group, bool int8,
                                         hipStream_t st)
{
    if (head_dim == 64) return int8 ? launch_valu_d<64, true>(a, group, st) : launch_valu_d<64, false>(a, group, st);
    if (head_dim == 128) return int8 ? launch_valu_d<128, true>(a, group, st) : launch_valu_d<128, false>(a, group, st);
    return hipErrorInvalidValue;
}

hipError_t launch_decode_merge(const DecodeArgs& a, int head_dim, hipStream_t st)
{
    const dim3 grid(a.num_q_heads, a.num_seqs);
    if (head_dim == 64) hipLaunchKernelGGL(decode_merge_kernel<64>, grid, dim3(64), 0, st, a);
    else if (head_dim == 128) hipLaunchKernelGGL(decode_merge_kernel<128>, grid, dim3(64), 0, st, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int head_dim, int group, bool int8, hipStream_t st)
{
#ifdef PA_DECODE_VALU
    hipError_t e = launch_decode_partitions_valu(a, head_dim, group, int8, st);
#else
    hipError_t e = launch_decode_partitions_mfma(a, head_dim, group, int8, st);
#endif
    if (e != hipSuccess || a.max_parts <= 1) return e;
    return launch_decode_merge(a, head_dim, st);
}

}  // namespace pa
