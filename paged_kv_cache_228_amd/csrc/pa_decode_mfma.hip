// Paged single-token decode attention for gfx950 (MI355X) on the matrix
// cores: the GQA query group of one KV head is one small dense Q.K^T tile.
//
// What is computed (paged-attention-runtime summary, "CORE CAPABILITIES" 2:
// block-table indirection, online single-pass softmax, fp32 accumulation;
// PagedKV-Fusion README, "Overview": per-(block, head) INT8 decode attention
// with GQA; glossary monograph, section 2.1 for the table lookup and
// section 5.2 for softmax(Q K^T / sqrt d) V): for sequence s and query head
// h, out = sum_t softmax_t(scale * q.k_t) v_t over the sequence's tokens.
//
// Work decomposition: one wave (the whole workgroup) per (sequence, KV head,
// context partition). The wave stages the partition's block ids in LDS and
// streams the partition's (block, head) tiles through a ring of register
// buffers, so several tiles' loads are in flight while one is computed.
//
// Per 16-token tile, with the G <= 16 query heads of the KV head padded to
// the 16 columns of a 16x16 MFMA tile:
//   S^T[token][head] = K[token][:] . Q^T[:][head]     v_mfma_f32_16x16x32_f16
//   O[head][dim]    += P[head][token] . V[token][dim]  v_mfma_f32_16x16x16_f16
// The lane map of the first product's result (lane = head + 16 * g holds
// tokens 4g .. 4g+3) is exactly the lane map the second product wants for
// its P operand, so scores never move between lanes. P goes to the matrix
// core as two fp16 halves (hi + lo, about 20 significant bits); K and V enter
// as fp16 (INT8 codes convert to fp16 exactly). Accumulation is fp32.
//
// Online softmax with a lazy reference: scores are kept in the log2 domain;
// the running reference max m of each head is only raised when a tile holds a
// score more than kLazy above it, so p = 2^(s - m) <= 2^kLazy and the rescale
// of the accumulators is rare. The result is the same softmax: every partial
// sum carries the same reference, and the merge divides it out.
#include "pa_internal.h"

namespace pa {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr uint32_t kRsrcWord3 = 0x00020000u;  // gfx9 raw buffer descriptor, 32-bit format
constexpr float kLazy = 8.0f;                 // log2 headroom before the reference max moves
constexpr float kPScale = 64.0f;              // P enters the matrix core as p * 2^6 (<= 2^14)
constexpr float kPUnscale = 1.0f / 64.0f;
#ifndef PA_KV_AUX
#define PA_KV_AUX 0
#endif
// Grid order: the KV heads of one (sequence, partition) are neighbours in
// dispatch order, so the head tiles of each physical block (adjacent in the
// pool) are read at about the same time.
#ifndef PA_HEAD_FAST
#define PA_HEAD_FAST 1
#endif
#ifndef PA_WG_HEADS
#define PA_WG_HEADS 0
#endif
constexpr int kKvAux = PA_KV_AUX;  // cache-policy bits of the K/V tile loads

__device__ __forceinline__ uint32_t word(const u32x4& v, int i)
{
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}
__device__ __forceinline__ uint32_t word(const u32x2& v, int i) { return i == 0 ? v.x : v.y; }
__device__ __forceinline__ uint32_t word(const uint32_t& v, int) { return v; }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}

// Sum / max over the four lanes that share l % 16 (lanes l, l^16, l^32, l^48).
// Outside the per-tile fast path only, so the LDS-routed shuffle is cheap
// enough. (The permlane16/32 swap builtins were tried here; with both
// operands the same value this compiler folded the pair of results into one.)
__device__ __forceinline__ float sum_over_groups(float x)
{
    x += __shfl_xor(x, 16, 64);
    return x + __shfl_xor(x, 32, 64);
}

__device__ __forceinline__ float max_over_groups(float x)
{
    x = fmaxf(x, __shfl_xor(x, 16, 64));
    return fmaxf(x, __shfl_xor(x, 32, 64));
}

// Value of lane `src` (a lane index in [0, 64)).
__device__ __forceinline__ float from_lane(float x, int src)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, x)));
}

// Four signed INT8 codes (one dword) to two pairs of exact fp16 values:
// flipping the sign bit gives c + 128; under the fp16 pattern 0x64xx that
// byte reads 1024 + c + 128, and subtracting 1152 leaves c.
__device__ __forceinline__ void codes_to_h2(uint32_t w, h2_t& lo, h2_t& hi)
{
    const uint32_t u = w ^ 0x80808080u;
    const h2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    lo = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - bias;
    hi = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - bias;
}

// Byte b of code words w0 and w1 (already sign-flipped) as an exact fp16 pair.
__device__ __forceinline__ h2_t code_pair(uint32_t u0, uint32_t u1, int b)
{
    const uint32_t sel = (uint32_t)b | 0x0C00u | ((uint32_t)(4 + b) << 16) | 0x0C000000u;
    const uint32_t two = __builtin_amdgcn_perm(u1, u0, sel) | 0x64006400u;
    const h2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    return __builtin_bit_cast(h2_t, two) - bias;
}

// Half h (0/1) of fp16 words w0 and w1 as a pair.
__device__ __forceinline__ h2_t half_pair(uint32_t w0, uint32_t w1, int h)
{
    return __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(w1, w0, h ? 0x07060302u : 0x05040100u));
}

template <int D, bool I8>
struct MCfg {
    static constexpr int EB = I8 ? 1 : 2;      // bytes per element
    static constexpr int ROW = D * EB;         // bytes per token row of a tile
    static constexpr int TILE = 16 * ROW;      // bytes per (block, head) tile
    static constexpr int NQK = D / 32;         // 16x16x32 MFMAs for Q.K^T
    static constexpr int KLD = I8 ? (NQK + 1) / 2 : NQK;  // 16-byte K loads per lane
    static constexpr int DPL = D / 16;         // V dims per lane
    static constexpr int VB = DPL * EB;        // V bytes per lane per token
};

template <int VB> struct VChunk;
template <> struct VChunk<16> { typedef u32x4 type; };
template <> struct VChunk<8> { typedef u32x2 type; };
template <> struct VChunk<4> { typedef uint32_t type; };

template <int VB>
__device__ __forceinline__ typename VChunk<VB>::type vload(rsrc_t r, int off)
{
    if constexpr (VB == 16) return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kKvAux);
    else if constexpr (VB == 8) return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kKvAux);
    else return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kKvAux);
}

template <int D, bool I8>
struct MTile {
    using C = MCfg<D, I8>;
    u32x4 k[C::KLD];
    typename VChunk<C::VB>::type v[4];
    float ksc, vsc;  // INT8 scales of the (block, head); unused for fp16
};

// Issue every load of one tile. valid == false (past the partition) or an id
// outside the pool gives a zero-byte descriptor: the loads return zeros and
// touch no memory.
template <int D, bool I8>
__device__ __forceinline__ void mload(MTile<D, I8>& t, const DecodeArgs& a, rsrc_t scales_k,
                                      rsrc_t scales_v, int bid, bool valid, int kvh, int lane)
{
    using C = MCfg<D, I8>;
    const bool in_pool = valid && (uint64_t)(int64_t)bid < (uint64_t)a.num_blocks;
    const int64_t b = in_pool ? bid : 0;
    const int64_t off = (b * a.num_kv_heads + kvh) * (int64_t)C::TILE;
    const int bytes = in_pool ? C::TILE : 0;
    const rsrc_t rk = make_rsrc(static_cast<const char*>(a.k) + off, bytes);
    const rsrc_t rv = make_rsrc(static_cast<const char*>(a.v) + off, bytes);
    const int g = lane >> 4, n = lane & 15;
#pragma unroll
    for (int c = 0; c < C::KLD; ++c) {
        // fp16: chunk 4c+g of token n (dims 8(4c+g) ..); int8: chunk g+4c (dims 16(g+4c) ..)
        const int chunk = I8 ? (g + 4 * c) : (4 * c + g);
        t.k[c] = __builtin_amdgcn_raw_buffer_load_b128(rk, n * C::ROW + 16 * chunk, 0, kKvAux);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) t.v[ks] = vload<C::VB>(rv, (4 * g + ks) * C::ROW + n * C::VB);
    if constexpr (I8) {
        const int si = (int)(b * a.num_kv_heads + kvh) * 4;
        t.ksc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(scales_k, in_pool ? si : -4, 0, 0));
        t.vsc = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(scales_v, in_pool ? si : -4, 0, 0));
    }
}

template <int D, bool I8>
struct MState {
    using C = MCfg<D, I8>;
    f4_t acc[C::DPL];  // O[heads 4g..4g+3][dim DPL*n + nb] x 2^6
    float m;           // reference max of head n (log2 domain)
    float l;           // this lane's share of head n's softmax denominator
};

template <int D, bool I8>
__device__ __forceinline__ void mprocess(MState<D, I8>& st, MTile<D, I8>& t,
                                         const h8_t (&qb)[MCfg<D, I8>::NQK], int valid,
                                         float scale_log2, int lane)
{
    using C = MCfg<D, I8>;
    const int g = lane >> 4;

    // S^T = K . Q^T
    f4_t s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < C::NQK; ++c) {
        h8_t ka;
        if constexpr (I8) {
            const u32x4& w = t.k[c >> 1];
            h2_t p0, p1, p2, p3;
            codes_to_h2(word(w, 2 * (c & 1)), p0, p1);
            codes_to_h2(word(w, 2 * (c & 1) + 1), p2, p3);
            ka = h8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
        } else {
            ka = __builtin_bit_cast(h8_t, t.k[c]);
        }
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qb[c], s, 0, 0, 0);
    }
    const float sl = I8 ? scale_log2 * t.ksc : scale_log2;
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = s[i] * sl;
    if (valid < 16) {  // tail of the sequence: mask scores and zero the V rows
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * g + i >= valid) {
                sc[i] = -INFINITY;
                if constexpr (C::VB == 16) t.v[i] = u32x4{0u, 0u, 0u, 0u};
                else if constexpr (C::VB == 8) t.v[i] = u32x2{0u, 0u};
                else t.v[i] = 0u;
            }
    }

    // lazy online softmax
    const float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    if (__builtin_amdgcn_ballot_w64(mx > st.m + kLazy) != 0) {
        const float mn = fmaxf(st.m, max_over_groups(mx));
        const float alpha = __builtin_amdgcn_exp2f(st.m - mn);  // 0 on the first tile
        st.l *= alpha;
        st.m = mn;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float ai = from_lane(alpha, 4 * g + i);  // alpha of head 4g+i
#pragma unroll
            for (int nb = 0; nb < C::DPL; ++nb) st.acc[nb][i] *= ai;
        }
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(sc[i] - st.m);
        st.l += p[i];
    }
    // P x 2^6 (<= 2^14) as fp16 hi + lo
    float ps[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ps[i] = p[i] * kPScale;
    const h2_t hi01 = __builtin_bit_cast(h2_t, __builtin_amdgcn_cvt_pkrtz(ps[0], ps[1]));
    const h2_t hi23 = __builtin_bit_cast(h2_t, __builtin_amdgcn_cvt_pkrtz(ps[2], ps[3]));
    const h2_t lo01 = __builtin_bit_cast(h2_t, __builtin_amdgcn_cvt_pkrtz(
                                                   ps[0] - (float)hi01.x, ps[1] - (float)hi01.y));
    const h2_t lo23 = __builtin_bit_cast(h2_t, __builtin_amdgcn_cvt_pkrtz(
                                                   ps[2] - (float)hi23.x, ps[3] - (float)hi23.y));
    const h4_t pa_hi = {hi01.x, hi01.y, hi23.x, hi23.y};
    const h4_t pa_lo = {lo01.x, lo01.y, lo23.x, lo23.y};

    // O += P . V, one 16x16x16 product per dim slot nb of the lane
    if constexpr (I8) {
        uint32_t u[4][C::VB / 4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int w = 0; w < C::VB / 4; ++w) u[ks][w] = word(t.v[ks], w) ^ 0x80808080u;
#pragma unroll
        for (int nb = 0; nb < C::DPL; ++nb) {
            const h2_t b01 = code_pair(u[0][nb >> 2], u[1][nb >> 2], nb & 3);
            const h2_t b23 = code_pair(u[2][nb >> 2], u[3][nb >> 2], nb & 3);
            const h4_t vb = {b01.x, b01.y, b23.x, b23.y};
            // the tile's own product in fresh accumulators, then scaled by
            // the tile's V scale into the running sum (P never carries vsc,
            // so its fp16 range does not depend on the data's scale)
            f4_t tacc = __builtin_amdgcn_mfma_f32_16x16x16f16(pa_hi, vb, f4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
            tacc = __builtin_amdgcn_mfma_f32_16x16x16f16(pa_lo, vb, tacc, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) st.acc[nb][i] = __builtin_fmaf(t.vsc, tacc[i], st.acc[nb][i]);
        }
    } else {
#pragma unroll
        for (int nb = 0; nb < C::DPL; ++nb) {
            const h2_t b01 = half_pair(word(t.v[0], nb >> 1), word(t.v[1], nb >> 1), nb & 1);
            const h2_t b23 = half_pair(word(t.v[2], nb >> 1), word(t.v[3], nb >> 1), nb & 1);
            const h4_t vb = {b01.x, b01.y, b23.x, b23.y};
            st.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa_hi, vb, st.acc[nb], 0, 0, 0);
            st.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa_lo, vb, st.acc[nb], 0, 0, 0);
        }
    }
}

template <int D, bool I8, int NBUF>
__global__ __launch_bounds__(PA_WG_HEADS ? 512 : 64) void decode_mfma_kernel(DecodeArgs a, int group)
{
    using C = MCfg<D, I8>;
    const int p = PA_WG_HEADS ? blockIdx.x : (PA_HEAD_FAST ? blockIdx.y : blockIdx.x);
    const int kvh = PA_WG_HEADS ? uniform(threadIdx.x >> 6) : (PA_HEAD_FAST ? blockIdx.x : blockIdx.y);
    const int s = PA_WG_HEADS ? blockIdx.y : blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, n = lane & 15;
    const int hq0 = kvh * group;

    int ctx = a.ctx[s];
    ctx = ctx < 0 ? 0 : (ctx > a.max_blocks * kBlockTokens ? a.max_blocks * kBlockTokens : ctx);
    if (ctx == 0) {  // empty context: the first partition writes the zero rows
        if (p == 0)
            for (int e = lane; e < group * D; e += 64) a.out[((int64_t)s * a.num_q_heads + hq0) * D + e] = 0.0f;
        return;
    }
    const int nblk = (ctx + kBlockTokens - 1) / kBlockTokens;
    const int b0 = p * a.part_blocks;
    if (b0 >= nblk) return;
    const int nloc = min(nblk - b0, a.part_blocks);
    const int nparts = (nblk + a.part_blocks - 1) / a.part_blocks;

    __shared__ int ids[kMaxPartitionBlocks];
    for (int i = PA_WG_HEADS ? (int)threadIdx.x : lane; i < nloc; i += PA_WG_HEADS ? (int)blockDim.x : 64)
        ids[i] = a.tables[(int64_t)s * a.max_blocks + b0 + i];

    // Q^T as the B operand of the 16x16x32 products: lane (g, n) holds head n,
    // the same 8 dims its K chunk covers; heads past the group are zero.
    h8_t qb[C::NQK];
    {
        const _Float16* qrow = static_cast<const _Float16*>(a.q) + ((int64_t)s * a.num_q_heads + hq0 + n) * D;
#pragma unroll
        for (int c = 0; c < C::NQK; ++c) {
            const int d0 = I8 ? 16 * (g + 4 * (c >> 1)) + 8 * (c & 1) : 8 * (4 * c + g);
            if (n < group)
                qb[c] = __builtin_bit_cast(h8_t, *reinterpret_cast<const u32x4*>(qrow + d0));
            else
                qb[c] = h8_t{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }
    MState<D, I8> st;
#pragma unroll
    for (int nb = 0; nb < C::DPL; ++nb) st.acc[nb] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
    st.m = -INFINITY;
    st.l = 0.0f;

    const rsrc_t rks = make_rsrc(a.k_scale, I8 ? (int)min<int64_t>(a.num_blocks * a.num_kv_heads * 4, 0x7fffffff) : 0);
    const rsrc_t rvs = make_rsrc(a.v_scale, I8 ? (int)min<int64_t>(a.num_blocks * a.num_kv_heads * 4, 0x7fffffff) : 0);
    __syncthreads();

    // ring of NBUF tiles: tile j sits in buf[j % NBUF]; tile j + NBUF - 1 is
    // loaded while tile j is processed
    MTile<D, I8> buf[NBUF];
#pragma unroll
    for (int b = 0; b < NBUF - 1; ++b)
        mload<D, I8>(buf[b], a, rks, rvs, uniform(ids[b < nloc ? b : 0]), b < nloc, kvh, lane);
    for (int base = 0; base < nloc; base += NBUF) {
#pragma unroll
        for (int b = 0; b < NBUF; ++b) {
            const int j = base + b;
            if (j >= nloc) break;
            const int jn = j + NBUF - 1;
            mload<D, I8>(buf[(b + NBUF - 1) % NBUF], a, rks, rvs, uniform(ids[jn < nloc ? jn : 0]),
                         jn < nloc, kvh, lane);
            const int valid = ctx - (b0 + j) * kBlockTokens;
            mprocess<D, I8>(st, buf[b], qb, valid, a.scale_log2, lane);
        }
    }

    // epilogue: the denominator of head n, summed over the four lane groups
    const float lsum = sum_over_groups(st.l);
    const int64_t row0 = (int64_t)s * a.num_q_heads + hq0;
    if (nparts == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int hd = 4 * g + i;
            const float inv = kPUnscale / from_lane(lsum, hd & 15);
            if (hd < group) {
                float* o = a.out + (row0 + hd) * D + n * C::DPL;
#pragma unroll
                for (int nb = 0; nb < C::DPL; ++nb) o[nb] = st.acc[nb][i] * inv;
            }
        }
    } else {
        const int64_t nslots = (int64_t)a.num_seqs * a.num_q_heads * a.max_parts;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int hd = 4 * g + i;
            if (hd < group) {
                float* o = a.ws + ((row0 + hd) * a.max_parts + p) * D + n * C::DPL;
#pragma unroll
                for (int nb = 0; nb < C::DPL; ++nb) o[nb] = st.acc[nb][i] * kPUnscale;
            }
        }
        if (g == 0 && n < group) {
            const int64_t slot = (row0 + n) * a.max_parts + p;
            a.ws[nslots * D + slot] = st.m;
            a.ws[nslots * (D + 1) + slot] = lsum;
        }
    }
}

}  // namespace

// Ring depths: tiles of one wave in flight (loads) plus the one being computed.
#ifndef PA_RING_F16
#define PA_RING_F16 2
#endif
#ifndef PA_RING_I8
#define PA_RING_I8 3
#endif

hipError_t launch_decode_partitions_mfma(const DecodeArgs& a, int head_dim, int group, bool int8,
                                         hipStream_t st)
{
    const dim3 grid = PA_WG_HEADS ? dim3(a.max_parts, a.num_seqs)
                      : (PA_HEAD_FAST ? dim3(a.num_kv_heads, a.max_parts, a.num_seqs)
                                      : dim3(a.max_parts, a.num_kv_heads, a.num_seqs));
    const dim3 block(PA_WG_HEADS ? 64 * a.num_kv_heads : 64);
    if (head_dim == 128) {
        if (int8) hipLaunchKernelGGL((decode_mfma_kernel<128, true, PA_RING_I8>), grid, block, 0, st, a, group);
        else hipLaunchKernelGGL((decode_mfma_kernel<128, false, PA_RING_F16>), grid, block, 0, st, a, group);
    } else if (head_dim == 64) {
        if (int8) hipLaunchKernelGGL((decode_mfma_kernel<64, true, PA_RING_I8>), grid, block, 0, st, a, group);
        else hipLaunchKernelGGL((decode_mfma_kernel<64, false, PA_RING_F16>), grid, block, 0, st, a, group);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pa
