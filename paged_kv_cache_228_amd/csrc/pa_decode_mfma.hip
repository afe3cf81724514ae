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
// Work decomposition: one wave (the whole workgroup) per (share, KV head):
// a share is a contiguous range of the head's tiles over all sequences
// (pa_split.h). The wave stages a chunk of block ids in LDS and streams the
// (block, head) tiles in slots of SLOT consecutive blocks through a two-slot
// register ring: one slot's loads are in flight while the other is computed.
//
// Three cache formats, one kernel template (F): fp16; INT8 codes with one
// fp32 scale per (block, head) for K and for V; FP8 (OCP E4M3) codes with
// the same scales (monograph section 5.1's FP8 variant). INT8 scores run on
// the int8 matrix cores; FP8 tiles are widened to fp16 in registers (the
// hardware's E4M3 -> fp16 conversion) and take the fp16 path.
//
// Per 16-token tile, with the G <= 8 query heads of the KV head in the 16
// columns of the MFMA tile:
//   S^T[token][col] = K[token][:] . Q^T[:][col]        v_mfma_f32_16x16x32_f16
// and per pair of tiles (32 tokens)
//   O[row][dim]    += P[row][token] . V[token][dim]    v_mfma_f32_16x16x32_f16
// The lane map of the first product's result (lane = column + 16 * g holds
// tokens 4g .. 4g+3) is the lane map the second product wants for its P
// operand (lane = row + 16 * g holds k = 8g .. 8g+7, here tokens 4g .. 4g+3
// of the pair's first tile, then of its second), so scores never move between
// lanes. Columns 0..7 of Q^T hold the group's heads and columns 8..15 the
// same heads again, so rows h and h + 8 of P carry the fp16 hi and lo halves
// of head h's weights (about 20 significant bits together) and one product
// covers both; the two output rows are added once at the end. V enters as
// fp16 (INT8 and E4M3 codes convert to fp16 exactly), K as fp16 or, for INT8,
// as raw codes. Accumulation is fp32.
//
// Online softmax with a lazy reference: scores are kept in the log2 domain;
// the running reference max m of each head is only raised when a slot holds a
// score more than kLazy above it, so p = 2^(s - m) <= 2^kLazy and the rescale
// of the accumulators is rare. The result is the same softmax: every partial
// sum carries the same reference, and the merge divides it out.
#include <type_traits>

#include "pa_internal.h"
#include "pa_split.h"

namespace pa {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr uint32_t kRsrcWord3 = 0x00020000u;  // gfx9 raw buffer descriptor, 32-bit format
constexpr float kLazy = 8.0f;                 // log2 headroom before the reference max moves
constexpr float kPScale = 64.0f;              // P enters the matrix core as p * 2^6 (<= 2^14, INT8 <= 2^15)
constexpr float kPUnscale = 1.0f / 64.0f;

// Cache-policy bits of the K/V tile loads: non-temporal (2) for tiles read
// once; the default policy (0) for blocks the neighbouring rows of the batch
// also reference (a shared prefix), which other waves of the same die read
// at about the same time.
#ifndef PA_KV_AUX
#define PA_KV_AUX 2
#endif
constexpr int kKvAuxShared = 0;

// Launch shape per (head_dim, format), chosen by graph-timed sweeps over the
// mixed prefix-sharing batch, the uniform 32 x 1,024 and 64 x 2,048-token
// batches, ragged batches of 300 and 1,000 sequences and the Qwen2-shaped
// layers:
//   SLOT  blocks per ring slot (even); two slots form the ring, one slot's
//         loads in flight while the other is computed. Two everywhere:
//         4-tile fp16 slots (32 KiB in flight per wave) were 0.4 % slower on
//         the mixed batch and 4 % slower on 32 x 1,024 tokens, and deeper
//         one-byte slots slower still.
//   MINW  waves per SIMD the register allocation leaves room for: fp16 and
//         FP8 at d = 128 need more than 256 registers and get one (FP8 with
//         256 spilled once it read shared blocks with their own policy); INT8
//         at d = 128 and every d = 64 kernel fit 256 (the d = 64 ones under
//         190).
//   WAVES waves launched per SIMD. One at d = 128: a second wave per SIMD
//         ended later than the first, and one wave holding twice the tiles
//         finished sooner. Two at d = 64, whose tiles are half the size: the
//         one-byte decodes of the mixed batch at d = 64 took 98 instead of
//         118 us, fp16 160 instead of 166 us.
template <int D, int F>
struct Launch {
    static constexpr int SLOT = 2;
    static constexpr int MINW = (D == 128 && F != kKvI8) ? 1 : 2;
    static constexpr int WAVES = D == 64 ? 2 : 1;
};

// Element i of a 4-dword vector (i a compile-time constant after unrolling).
// Written as a select chain: subscripting an array of ext-vector values with
// a loop index inside nested unrolled loops lost elements with this compiler.
__device__ __forceinline__ uint32_t word(const u32x4& v, int i)
{
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}
__device__ __forceinline__ uint32_t word(const u32x2& v, int i) { return i == 0 ? v.x : v.y; }
__device__ __forceinline__ uint32_t word(const uint32_t& v, int) { return v; }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// The lane's index, computed where it is used: the output and partial
// addresses of emit() are then formed there instead of being hoisted to the
// kernel's start and kept in registers across the hot loop (which spilled).
__device__ __forceinline__ int lane_here()
{
    int v;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
    return v;
}

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}

// Sum / max over the four lanes that share l % 16 (lanes l, l^16, l^32, l^48).
// Outside the per-slot fast path only, so the LDS-routed shuffle is cheap
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

// Half h (0/1) of fp16 words w0 and w1 as a pair.
__device__ __forceinline__ uint32_t half_pair(uint32_t w0, uint32_t w1, int h)
{
    return __builtin_amdgcn_perm(w1, w0, h ? 0x07060302u : 0x05040100u);
}

// E4M3 codes B, B+1 (B = 0 or 2) of word w as an fp16 pair: the hardware's
// scaled conversion with scale 1, exact (every E4M3 value is an fp16 value).
template <int B>
__device__ __forceinline__ uint32_t e4m3_pair(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, B != 0));
}

// Code b of words w0 and w1 as an fp16 pair.
__device__ __forceinline__ uint32_t e4m3_pair2(uint32_t w0, uint32_t w1, int b)
{
    const uint32_t sel = (uint32_t)b | ((uint32_t)(4 + b) << 8) | 0x0C0C0000u;
    return e4m3_pair<0>(__builtin_amdgcn_perm(w1, w0, sel));
}

template <int D, int F>
struct MCfg {
    static constexpr bool I8 = F == kKvI8;     // int8 codes on the int8 matrix cores
    static constexpr bool SCALED = F != kKvF16;  // per-(block, head) K and V scales
    static constexpr int EB = I8 ? 1 : 2;      // bytes per element in registers and LDS
    static constexpr int SEB = F == kKvF16 ? 2 : 1;  // bytes per element in the pool
    static constexpr int ROW = D * EB;         // bytes per token row of a register tile
    static constexpr int TILE = 16 * ROW;      // bytes per register tile
    static constexpr int STILE = 16 * D * SEB; // bytes per (block, head) tile in the pool
    static constexpr int NQK = D / 32;         // 16x16x32 MFMAs for Q.K^T per tile
    static constexpr int KLD = I8 ? (NQK + 1) / 2 : NQK;  // 16-byte K registers per lane
    static constexpr int DPL = D / 16;         // V dims per lane
    static constexpr int VB = DPL * EB;        // V register bytes per lane per token
    static constexpr int SVB = DPL * SEB;      // V pool bytes per lane per token
};

template <int VB> struct VChunk;
template <> struct VChunk<16> { typedef u32x4 type; };
template <> struct VChunk<8> { typedef u32x2 type; };
template <> struct VChunk<4> { typedef uint32_t type; };

template <int VB, int AUX>
__device__ __forceinline__ typename VChunk<VB>::type vload(rsrc_t r, int off)
{
    if constexpr (VB == 16) return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
    else if constexpr (VB == 8) return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX);
    else return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX);
}

// A tile as loaded: K in tile order (FP8: 8 codes per register pair), V as
// four token rows of this lane's dims, both in the pool's element size.
template <int D, int F>
struct MTile {
    using C = MCfg<D, F>;
    typename std::conditional<F == kKvF8, u32x2, u32x4>::type k[C::KLD];
    typename VChunk<C::SVB>::type v[4];
};

// Issue every load of one tile (and, for INT8, of its K and V scales).
// valid == false (past the chunk) or bid < 0 (an id outside the pool, marked
// when staged) gives a zero-byte descriptor: the loads return zeros and touch
// no memory, and the scales are 0.
template <int D, int F>
__device__ __forceinline__ void mscales(const DecodeArgs& a, int bid, bool valid, int kvh, float& ksc,
                                        float& vsc)
{
    if constexpr (MCfg<D, F>::SCALED) {  // uniform addresses: one scalar load each
        const bool in_pool = valid && bid >= 0;
        const int64_t si = (in_pool ? (int64_t)bid : 0) * a.num_kv_heads + kvh;
        ksc = in_pool ? a.k_scale[si] : 0.0f;
        vsc = in_pool ? a.v_scale[si] : 0.0f;
    }
}

// The tile's vector loads, with cache-policy bits AUX (its scales: mscales).
template <int D, int F, int AUX>
__device__ __forceinline__ void mload(MTile<D, F>& t, const DecodeArgs& a, int bid, bool valid,
                                      int kvh, int lane)
{
    using C = MCfg<D, F>;
    const bool in_pool = valid && bid >= 0;
    const int64_t b = in_pool ? bid : 0;
    const int64_t off = (b * a.num_kv_heads + kvh) * (int64_t)C::STILE;
    const int bytes = in_pool ? C::STILE : 0;
    const rsrc_t rk = make_rsrc(static_cast<const char*>(a.k) + off, bytes);
    const rsrc_t rv = make_rsrc(static_cast<const char*>(a.v) + off, bytes);
    const int g = lane >> 4, n = lane & 15;
    // K in the tile's own order: instruction c reads bytes [1024c, 1024c + 1024)
    // (FP8: [512c, 512c + 512), the codes of the fp16 layout's elements)
#pragma unroll
    for (int c = 0; c < C::KLD; ++c) {
        if constexpr (F == kKvF8)
            t.k[c] = __builtin_amdgcn_raw_buffer_load_b64(rk, 512 * c + 8 * lane, 0, AUX);
        else
            t.k[c] = __builtin_amdgcn_raw_buffer_load_b128(rk, 1024 * c + 16 * lane, 0, AUX);
    }
    // V: token 4g+ks, this lane's DPL dims (n * DPL ..)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) t.v[ks] = vload<C::SVB, AUX>(rv, (4 * g + ks) * D * C::SEB + n * C::SVB);
}

// K reaches the matrix cores through LDS. A load in operand order (lane =
// token) would make each 64-lane load instruction touch sixteen 128-byte lines
// and use half of each, which costs the vector memory path about twice the
// time of reading the same bytes in order; so K is read in order (eight whole
// lines per instruction), written to a per-wave LDS tile and read back in
// operand order. The 16-byte chunk q of row r sits at chunk q ^ f(r), an XOR
// swizzle for which both the in-order writes and the operand-order reads hit
// distinct LDS banks (whether the hardware serves 8 lanes per 128 bytes or
// 16 lanes per 256 bytes per pass).
template <int D, int F>
struct KSwz {
    using C = MCfg<D, F>;
    static_assert(C::ROW == 256 || C::ROW == 128 || C::ROW == 64, "row of 64, 128 or 256 bytes");
    static constexpr int KREG = C::TILE / 1024;  // 16-byte registers per lane per tile
    __device__ static int f(int r)
    {
        if constexpr (C::ROW == 256) return r & 15;
        else if constexpr (C::ROW == 128) return ((r >> 1) & 3) | (((r ^ (r >> 3)) & 1) << 2);
        else return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1);
    }
    // index (in 16-byte units) of chunk q of row r in an LDS tile
    __device__ static int at(int r, int q) { return r * (C::ROW / 16) + (q ^ f(r)); }
};

// Rearrange the K registers of one tile from tile order to operand order
// through the wave's LDS tile `kl`: afterwards k[c] holds, for lane (g, n),
// token n's 16-byte chunk 4c+g (fp16) or g+4c (INT8).
template <int D, int F, int KL>
__device__ __forceinline__ void k_to_operand(u32x4 (&k)[KL], u32x4* kl, int lane)
{
    using C = MCfg<D, F>;
    static_assert(KL == C::KLD, "K registers of one tile");
    using S = KSwz<D, F>;
    static_assert(S::KREG == C::KLD, "one 16-byte register per 1024 bytes of K");
    const int g = lane >> 4, n = lane & 15;
#pragma unroll
    for (int c = 0; c < C::KLD; ++c) {
        const int o = 1024 * c + 16 * lane;
        kl[S::at(o / C::ROW, (o % C::ROW) / 16)] = k[c];
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int c = 0; c < C::KLD; ++c) k[c] = kl[S::at(n, C::I8 ? (g + 4 * c) : (4 * c + g))];
    __builtin_amdgcn_wave_barrier();
}

template <int D, int F>
struct MState {
    using C = MCfg<D, F>;
    f4_t acc[C::DPL];  // rows 4g..4g+3 of O x 2^6 (row h: hi part of head h, row h+8: lo part)
    float m;           // reference max of head n (log2 domain)
    float l;           // this lane's share of head n's softmax denominator
    float vr;          // scaled formats: reference V scale of acc (uniform; 0 until a nonzero scale)
    float vinv;        // 1 / vr (0 while vr is 0), recomputed only when vr moves
};

// The query operand of S^T = K . Q^T (B operand; lane (g, n) serves column n,
// i.e. head n mod 8, over the same dims as its K chunk).
//  fp16 K: q as fp16, 8 dims per 16x16x32 product.
//  INT8 K: the codes go to v_mfma_i32_16x16x64_i8 unconverted, so q is split
//  per head into three int8 parts with a power-of-two step sigma
//  (max |q| / sigma in [32, 64)): q = sigma (a1 + a2 2^-7 + a3 2^-14) + r,
//  |r| <= sigma 2^-15, so every q element of at least max |q| / 1024 is exact
//  and the rest are off by less than 2^-20 max |q|. The three integer dot
//  products are exact; they are recombined in fp32.
template <int D, bool I8>
struct QOp;
template <int D>
struct QOp<D, false> {
    h8_t b[MCfg<D, false>::NQK];
};
template <int D>
struct QOp<D, true> {
    u32x4 part[3][MCfg<D, true>::KLD];  // a1, a2, a3: 16 int8 per register
    float sigma;                        // this lane's head's step
};

// Scores of one tile, S^T = K . Q^T (K registers in operand order), times
// `sl` (softmax scale x log2 e, x the tile's K scale for INT8).
template <int D, int F>
__device__ __forceinline__ f4_t tile_scores(const u32x4 (&kop)[MCfg<D, F>::KLD],
                                            const QOp<D, MCfg<D, F>::I8>& qo, float sl)
{
    using C = MCfg<D, F>;
    if constexpr (C::I8) {
        i32x4 s1 = {0, 0, 0, 0}, s2 = {0, 0, 0, 0}, s3 = {0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < C::KLD; ++c) {
            const i32x4 k = __builtin_bit_cast(i32x4, kop[c]);
            s1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(k, __builtin_bit_cast(i32x4, qo.part[0][c]), s1, 0, 0, 0);
            s2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(k, __builtin_bit_cast(i32x4, qo.part[1][c]), s2, 0, 0, 0);
            s3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(k, __builtin_bit_cast(i32x4, qo.part[2][c]), s3, 0, 0, 0);
        }
        // |s1|, |s2|, |s3| <= 127 * 64 * D, so s2 * 2^7 + s3 stays in int32
        const float f = sl * qo.sigma;
        f4_t r;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r[i] = __builtin_fmaf((float)(s2[i] * 128 + s3[i]), 1.0f / 16384.0f, (float)s1[i]) * f;
        return r;
    } else {
        f4_t s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < C::NQK; ++c)
            s = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, kop[c]), qo.b[c], s, 0, 0, 0);
        return s * sl;
    }
}

// The raw fp16 query registers of lane (g, n): head qh's dims the lane serves.
template <int D, bool I8>
struct QRaw {
    u32x4 w[I8 ? 2 * MCfg<D, I8>::KLD : MCfg<D, I8>::NQK];
};

// Issue the query loads of lane (g, n) for head qh (zeros past the group).
template <int D, bool I8>
__device__ __forceinline__ void fetch_q(QRaw<D, I8>& qr, const _Float16* qrow, bool live, int g)
{
    using C = MCfg<D, I8>;
    const u32x4 z = {0u, 0u, 0u, 0u};
    if constexpr (I8) {
        // dims 64c + 16g .. +15: the chunk g + 4c of this lane's K codes
#pragma unroll
        for (int c = 0; c < C::KLD; ++c)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                qr.w[2 * c + h] = live ? *reinterpret_cast<const u32x4*>(qrow + 64 * c + 16 * g + 8 * h) : z;
    } else {
#pragma unroll
        for (int c = 0; c < C::NQK; ++c)
            qr.w[c] = live ? *reinterpret_cast<const u32x4*>(qrow + 8 * (4 * c + g)) : z;
    }
}

// Build the query operand from the raw registers.
template <int D, bool I8>
__device__ __forceinline__ void make_q(QOp<D, I8>& qo, const QRaw<D, I8>& qr)
{
    using C = MCfg<D, I8>;
    if constexpr (I8) {
        float qf[C::KLD][16];
        float mloc = 0.0f;
#pragma unroll
        for (int c = 0; c < C::KLD; ++c)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const h8_t v = __builtin_bit_cast(h8_t, qr.w[2 * c + h]);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    qf[c][8 * h + i] = (float)v[i];
                    mloc = fmaxf(mloc, fabsf(qf[c][8 * h + i]));
                }
            }
        const float mh = max_over_groups(mloc);  // the four lanes of column n hold all of head n's dims
        const int e = mh > 0.0f ? __builtin_amdgcn_frexp_expf(mh) : 0;  // mh = f 2^e, f in [0.5, 1)
        const float inv = __builtin_ldexpf(1.0f, 6 - e);
        qo.sigma = __builtin_ldexpf(1.0f, e - 6);
#pragma unroll
        for (int c = 0; c < C::KLD; ++c) {
            uint32_t w[3][4] = {};
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float y = qf[c][i] * inv;  // |y| < 64, exact
                const float a1 = __builtin_rintf(y);
                const float r1 = (y - a1) * 128.0f;
                const float a2 = __builtin_rintf(r1);
                const float a3 = __builtin_rintf((r1 - a2) * 128.0f);
                w[0][i >> 2] |= ((uint32_t)(int)a1 & 0xFFu) << (8 * (i & 3));
                w[1][i >> 2] |= ((uint32_t)(int)a2 & 0xFFu) << (8 * (i & 3));
                w[2][i >> 2] |= ((uint32_t)(int)a3 & 0xFFu) << (8 * (i & 3));
            }
#pragma unroll
            for (int jj = 0; jj < 3; ++jj) qo.part[jj][c] = u32x4{w[jj][0], w[jj][1], w[jj][2], w[jj][3]};
        }
    } else {
#pragma unroll
        for (int c = 0; c < C::NQK; ++c) qo.b[c] = __builtin_bit_cast(h8_t, qr.w[c]);
    }
}

// The four V operand words of a pair of INT8 tiles for code byte B of word
// x0..x3 (tile a's tokens 4g..4g+3) and y0..y3 (tile b's): each word is
// the fp16 pair of two consecutive tokens' codes. The conversion takes the
// byte straight from its word, sign-extended (sub-dword operand select), so
// no byte moves and no bias is needed; every int8 value is an fp16 value.
// All low halves are written before any high half (which keeps the partial
// register writes apart), and the trailing wait states cover the partial
// writes' forwarding to the matrix core that reads the words.
template <int B>
__device__ __forceinline__ u32x4 i8_vwords(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3, uint32_t y0,
                                           uint32_t y1, uint32_t y2, uint32_t y3)
{
    static_assert(B >= 0 && B < 4, "a byte of a word");
    uint32_t w0, w1, w2, w3;
#define PA_SDWA_CVT(DST, SRC, HALF, KEEP) \
    "v_cvt_f16_i16_sdwa " DST ", sext(" SRC ") dst_sel:" HALF " dst_unused:" KEEP " src0_sel:BYTE_%12\n\t"
    asm(PA_SDWA_CVT("%0", "%4", "WORD_0", "UNUSED_PAD") PA_SDWA_CVT("%1", "%6", "WORD_0", "UNUSED_PAD")
        PA_SDWA_CVT("%2", "%8", "WORD_0", "UNUSED_PAD") PA_SDWA_CVT("%3", "%10", "WORD_0", "UNUSED_PAD")
        PA_SDWA_CVT("%0", "%5", "WORD_1", "UNUSED_PRESERVE") PA_SDWA_CVT("%1", "%7", "WORD_1", "UNUSED_PRESERVE")
        PA_SDWA_CVT("%2", "%9", "WORD_1", "UNUSED_PRESERVE") PA_SDWA_CVT("%3", "%11", "WORD_1", "UNUSED_PRESERVE")
        "s_nop 1"
        : "=&v"(w0), "=&v"(w1), "=&v"(w2), "=&v"(w3)
        : "v"(x0), "v"(x1), "v"(x2), "v"(x3), "v"(y0), "v"(y1), "v"(y2), "v"(y3), "i"(B));
#undef PA_SDWA_CVT
    return u32x4{w0, w1, w2, w3};
}

// i8_vwords for a byte index known after unrolling.
__device__ __forceinline__ u32x4 i8_vwords_at(int b, uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                              uint32_t y0, uint32_t y1, uint32_t y2, uint32_t y3)
{
    switch (b) {
    case 0: return i8_vwords<0>(x0, x1, x2, x3, y0, y1, y2, y3);
    case 1: return i8_vwords<1>(x0, x1, x2, x3, y0, y1, y2, y3);
    case 2: return i8_vwords<2>(x0, x1, x2, x3, y0, y1, y2, y3);
    default: return i8_vwords<3>(x0, x1, x2, x3, y0, y1, y2, y3);
    }
}

// The V operand word of tile t for dim slot nb and tokens 4g+2h, 4g+2h+1
// (fp16 and FP8; INT8 tiles take i8_vwords).
template <int D, int F>
__device__ __forceinline__ uint32_t v_word(const MTile<D, F>& t, int nb, int h)
{
    static_assert(F != kKvI8, "INT8 V words come from i8_vwords");
    if constexpr (F == kKvF8) {
        return e4m3_pair2(word(t.v[2 * h], nb >> 2), word(t.v[2 * h + 1], nb >> 2), nb & 3);
    } else {
        return half_pair(word(t.v[2 * h], nb >> 1), word(t.v[2 * h + 1], nb >> 1), nb & 1);
    }
}

// One slot: SLOT consecutive tiles of the partition. With TAIL, only the first
// `valid0` token rows are live (none when valid0 <= 0); without, all are.
template <int D, int F, int SLOT, bool TAIL>
__device__ __forceinline__ void mprocess(MState<D, F>& st, const MTile<D, F> (&t)[SLOT],
                                         const QOp<D, MCfg<D, F>::I8>& qo, int valid0,
                                         float scale_log2, const float (&ksc)[SLOT],
                                         const float (&vsc)[SLOT], int lane, float lo_sel,
                                         u32x4* kl)
{
    using C = MCfg<D, F>;
    const int g = lane >> 4;
    float sc[SLOT][4];
#pragma unroll
    for (int u = 0; u < SLOT; ++u) {
        u32x4 kop[C::KLD];
#pragma unroll
        for (int c = 0; c < C::KLD; ++c) {
            if constexpr (F == kKvF8) {  // 8 codes -> 8 fp16
                const uint32_t w0 = t[u].k[c].x, w1 = t[u].k[c].y;
                kop[c] = u32x4{e4m3_pair<0>(w0), e4m3_pair<2>(w0), e4m3_pair<0>(w1), e4m3_pair<2>(w1)};
            } else {
                kop[c] = t[u].k[c];
            }
        }
        k_to_operand<D, F, C::KLD>(kop, kl + u * (C::TILE / 16), lane);
        const f4_t s = tile_scores<D, F>(kop, qo, C::SCALED ? scale_log2 * ksc[u] : scale_log2);
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[u][i] = s[i];
    }
    // dead rows (past the sequence's end or the partition's) get score -inf
    // and a zero V row (their stored slots may hold anything, NaN included);
    // V rows are masked where the P.V operands are built, so the tile
    // registers themselves are only ever read
    uint32_t vmask[SLOT][2];
    if constexpr (TAIL) {
#pragma unroll
        for (int u = 0; u < SLOT; ++u) {
            const int vu = valid0 - 16 * u;  // live rows of tile u (may be <= 0)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * g + i >= vu) sc[u][i] = -INFINITY;
#pragma unroll
            for (int h = 0; h < 2; ++h)
                vmask[u][h] = (4 * g + 2 * h < vu ? 0x0000FFFFu : 0u) |
                              (4 * g + 2 * h + 1 < vu ? 0xFFFF0000u : 0u);
        }
    }

    // lazy online softmax over the whole slot
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < SLOT; ++u)
        mx = fmaxf(mx, fmaxf(fmaxf(sc[u][0], sc[u][1]), fmaxf(sc[u][2], sc[u][3])));
    if (__builtin_amdgcn_ballot_w64(mx > st.m + kLazy) != 0) {
        const float mn = fmaxf(st.m, max_over_groups(mx));
        const float alpha = __builtin_amdgcn_exp2f(st.m - mn);  // 0 on the first slot
        st.l *= alpha;
        st.m = mn;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float ai = from_lane(alpha, 4 * g + i);  // alpha of row 4g+i's head
#pragma unroll
            for (int nb = 0; nb < C::DPL; ++nb) st.acc[nb][i] *= ai;
        }
    }

    // Scaled formats: a lazy reference V scale, like the reference max. Each tile's
    // weights are multiplied by its V scale over the reference (<= 2, so P
    // keeps its fp16 range) and the products accumulate at the reference
    // scale; the reference only moves, rescaling the accumulators, when a
    // tile's scale exceeds twice it (on the first nonzero scale, and rarely
    // after).
    float vrel[SLOT];
#pragma unroll
    for (int u = 0; u < SLOT; ++u) vrel[u] = 1.0f;
    if constexpr (C::SCALED) {
        float vmax = vsc[0];
#pragma unroll
        for (int u = 1; u < SLOT; ++u) vmax = fmaxf(vmax, vsc[u]);
        if (vmax > 2.0f * st.vr) {
            const float f = st.vr / vmax;  // 0 while the reference is 0: acc is still 0
#pragma unroll
            for (int nb = 0; nb < C::DPL; ++nb) st.acc[nb] *= f;
            st.vr = vmax;
            st.vinv = 1.0f / vmax;  // vmax > 0 here
        }
        const float inv = st.vinv;
#pragma unroll
        for (int u = 0; u < SLOT; ++u) vrel[u] = vsc[u] * inv;
    }

#pragma unroll
    for (int pr = 0; pr < SLOT / 2; ++pr) {
        // P of the pair (x 2^6, x the tile's relative V scale: <= 2^15): rows
        // 0..7 (lo_sel 0) take its round-toward-zero fp16 value, rows 8..15
        // (lo_sel 1) what that rounding dropped
        uint32_t pw[4];
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
            const int u = 2 * pr + uu;
            float ps[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = __builtin_amdgcn_exp2f(sc[u][i] - st.m);
                st.l += p;
                ps[i] = p * (kPScale * vrel[u]);
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const float a = ps[2 * hh], b = ps[2 * hh + 1];
                const h2_t hi = __builtin_bit_cast(h2_t, __builtin_amdgcn_cvt_pkrtz(a, b));
                pw[2 * uu + hh] = __builtin_bit_cast(
                    uint32_t, __builtin_amdgcn_cvt_pkrtz(__builtin_fmaf(-lo_sel, (float)hi.x, a),
                                                         __builtin_fmaf(-lo_sel, (float)hi.y, b)));
            }
        }
        const h8_t pa = __builtin_bit_cast(h8_t, u32x4{pw[0], pw[1], pw[2], pw[3]});
        const MTile<D, F>& ta = t[2 * pr];
        const MTile<D, F>& tb = t[2 * pr + 1];
#pragma unroll
        for (int nb = 0; nb < C::DPL; ++nb) {
            u32x4 vw;
            if constexpr (F == kKvI8) {
                const int w = nb >> 2;
                vw = i8_vwords_at(nb & 3, word(ta.v[0], w), word(ta.v[1], w), word(ta.v[2], w), word(ta.v[3], w),
                                  word(tb.v[0], w), word(tb.v[1], w), word(tb.v[2], w), word(tb.v[3], w));
            } else {
                vw = u32x4{v_word<D, F>(ta, nb, 0), v_word<D, F>(ta, nb, 1), v_word<D, F>(tb, nb, 0),
                           v_word<D, F>(tb, nb, 1)};
            }
            if constexpr (TAIL)
                vw &= u32x4{vmask[2 * pr][0], vmask[2 * pr][1], vmask[2 * pr + 1][0], vmask[2 * pr + 1][1]};
            st.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, __builtin_bit_cast(h8_t, vw), st.acc[nb],
                                                                0, 0, 0);
        }
    }
}

// A slot, with the tail masking compiled in only where it can be needed.
template <int D, int F, int SLOT>
__device__ __forceinline__ void mslot(MState<D, F>& st, const MTile<D, F> (&t)[SLOT],
                                      const QOp<D, MCfg<D, F>::I8>& qo, int valid0,
                                      float scale_log2, const float (&ksc)[SLOT],
                                      const float (&vsc)[SLOT], int lane, float lo_sel, u32x4* kl)
{
    if (valid0 >= 16 * SLOT)
        mprocess<D, F, SLOT, false>(st, t, qo, valid0, scale_log2, ksc, vsc, lane, lo_sel, kl);
    else
        mprocess<D, F, SLOT, true>(st, t, qo, valid0, scale_log2, ksc, vsc, lane, lo_sel, kl);
}

// The end of one (sequence, KV head) segment of a share. If the segment is
// the row's whole context its query heads' outputs are written; otherwise its
// partial (acc, m, l) goes to slot `slot` of the share for the merge kernel
// (1: the row started in this share, which holds its first tile; 0: the row
// started in an earlier share).
template <int D, int F>
__device__ __forceinline__ void emit(MState<D, F>& st, const DecodeArgs& a, int s, int kvh, int group,
                                     int share, bool cut, int slot)
{
    using C = MCfg<D, F>;
    const int lane = lane_here();
    const int g = lane >> 4, n = lane & 15;
    // fold the lo rows (8..15, lane groups 2 and 3) onto the hi rows (0..7,
    // lane groups 0 and 1); the denominator of head n, summed over the four
    // lane groups
#pragma unroll
    for (int nb = 0; nb < C::DPL; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) st.acc[nb][i] += __shfl_xor(st.acc[nb][i], 32, 64);
    const float lsum = sum_over_groups(st.l);
    const float unscale = C::SCALED ? kPUnscale * st.vr : kPUnscale;  // back to the data's scale
    if (!cut) {
        const int64_t row0 = (int64_t)s * a.num_q_heads + (int64_t)kvh * group;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int hd = 4 * g + i;  // rows of lane groups 0 and 1 only
            const float inv = unscale / from_lane(lsum, hd & 7);
            if (g < 2 && hd < group) {
                float* o = a.out + (row0 + hd) * D + n * C::DPL;
#pragma unroll
                for (int nb = 0; nb < C::DPL; ++nb) o[nb] = st.acc[nb][i] * inv;
            }
        }
        return;
    }
    const int64_t nslot = (int64_t)a.shares * a.num_kv_heads * 2 * group;  // (share, head, slot, q) entries
    const int64_t base = (((int64_t)share * a.num_kv_heads + kvh) * 2 + slot) * group;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int hd = 4 * g + i;
        if (g < 2 && hd < group) {
            float* o = a.part + (base + hd) * D + n * C::DPL;
#pragma unroll
            for (int nb = 0; nb < C::DPL; ++nb) o[nb] = st.acc[nb][i] * unscale;
        }
    }
    if (g == 0 && n < group) {
        a.part[nslot * D + base + n] = st.m;
        a.part[nslot * (D + 1) + base + n] = lsum;
    }
}

// This wave's place in the work split (pa_split.h): its share's tile range
// [p0, p1) of the KV head's T tiles and the row s0 holding tile p0, whose
// first tile is rs0. The share's ends come from the cost line: b = k Q / K
// lies in one row's cost range, and p is that row's first tile plus the
// tile whose interval holds b. Up to kScanSeqs sequences the wave scans the
// context lengths itself (four per lane) into tile and cost prefix sums, and
// the grid's first wave stores them for the merge kernel; beyond that the
// prep kernel has stored them, with the row holding every share's first tile.
struct ShareLoc {
    int64_t p0, p1;
    int s0, rs0;
};
__device__ __forceinline__ ShareLoc locate_share(const DecodeArgs& a, int share, int lane)
{
    static_assert(kScanSeqs == 4 * 64, "four sequences per lane");
    const int S = a.num_seqs;
    const int64_t K = a.shares;
    const int32_t* costs = a.rows + ws_costs(S);
    ShareLoc r;
    if (S > kScanSeqs) {
        const int64_t T = a.rows[S], Q = costs[S];
        const int64_t b0 = share_start(share, Q, K), b1 = share_start(share + 1, Q, K);
        // the tile whose cost interval holds b, through the row the prep
        // kernel found for it
        auto tile_at = [&](int row, int64_t b) {
            const int64_t c0 = costs[row], rt = a.rows[row];
            const int64_t nb = a.rows[row + 1] - rt;
            return rt + tile_at_cost(b - c0, nb, costs[row + 1] - c0);
        };
        r.p0 = r.p1 = T;
        r.s0 = r.rs0 = 0;
        if (Q == 0) return r;  // no sequence has a tile (and the prep kernel stored no rows)
        const int32_t* first_row = a.rows + ws_first_row(S);
        r.s0 = first_row[share];
        r.p0 = tile_at(r.s0, b0);
        if (share + 1 < K) r.p1 = tile_at(first_row[share + 1], b1);
        r.rs0 = a.rows[r.s0];
        return r;
    }
    int nb[4], ex[4], exc[4];
    // the four loads unconditional (a lane past the batch reads the last
    // sequence) and in flight together: one memory round trip
    int x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = a.ctx[min(64 * u + lane, S - 1)];
    asm volatile("" ::"v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]));
#pragma unroll
    for (int u = 0; u < 4; ++u) nb[u] = 64 * u + lane < S ? clamp_blocks(x[u], a.max_blocks) : 0;
    // exclusive tile prefix sums (a 64-lane scan per 64 rows)
    int carry = 0;
    uint64_t live[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        int x = nb[u];
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(x, d, 64);
            if (lane >= d) x += y;
        }
        ex[u] = carry + x - nb[u];
        carry += __builtin_amdgcn_readlane(x, 63);
        live[u] = __builtin_amdgcn_ballot_w64(nb[u] > 0);
    }
    // The row cost, unless every non-empty row has as many tiles as the first:
    // rows of equal length take the plain split (cost 0), which cuts them the
    // same way wherever its shares fall on row boundaries, with less
    // arithmetic here.
    int nb_first = 0;
#pragma unroll
    for (int u = 3; u >= 0; --u)
        if (live[u] != 0) nb_first = __builtin_amdgcn_readlane(nb[u], __builtin_ctzll(live[u]));
    bool equal = true;
#pragma unroll
    for (int u = 0; u < 4; ++u) equal = equal && __builtin_amdgcn_ballot_w64(nb[u] > 0 && nb[u] != nb_first) == 0;
    const int c = equal ? 0 : a.row_cost;
    r.s0 = 0;
    r.rs0 = 0;
    if (c == 0) {  // tiles and costs coincide: share k is [k T / K, (k + 1) T / K)
        if (blockIdx.x == 0) {
            int32_t* costs_w = a.rows + ws_costs(S);
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (64 * u + lane < S) a.rows[64 * u + lane] = costs_w[64 * u + lane] = ex[u];
            if (lane == 0) a.rows[S] = costs_w[S] = carry;
        }
        const int64_t T = uniform(carry);
        r.p0 = div_floor(share * T, K);
        r.p1 = div_floor((share + 1) * T, K);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint64_t hit = __builtin_amdgcn_ballot_w64(nb[u] > 0 && ex[u] <= r.p0 && r.p0 < ex[u] + nb[u]);
            if (hit != 0) {
                const int l = __builtin_ctzll(hit);
                r.s0 = 64 * u + l;
                r.rs0 = __builtin_amdgcn_readlane(ex[u], l);
            }
        }
        return r;
    }
    // the cost prefix adds c per non-empty row before, counted from the ballots
    int rows_before = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(live[u] >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)live[u], 0));
        exc[u] = ex[u] + c * (rows_before + before);
        rows_before += __builtin_popcountll(live[u]);
    }
    if (blockIdx.x == 0) {
        int32_t* costs_w = a.rows + ws_costs(S);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (64 * u + lane < S) {
                a.rows[64 * u + lane] = ex[u];
                costs_w[64 * u + lane] = exc[u];
            }
        if (lane == 0) {
            a.rows[S] = carry;
            costs_w[S] = carry + c * rows_before;
        }
    }
    const int64_t T = uniform(carry), Q = T + (int64_t)c * uniform(rows_before);
    // the tiles whose cost intervals hold b0 and b1 (when below Q), each
    // through the one row with exc <= b < exc + nb + c, found in one pass
    const int64_t b0 = share_start(share, Q, K), b1 = share_start(share + 1, Q, K);
    r.p0 = T;
    r.p1 = T;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const bool has = nb[u] > 0;
        const uint64_t hit0 = __builtin_amdgcn_ballot_w64(has && exc[u] <= b0 && b0 < exc[u] + nb[u] + c);
        const uint64_t hit1 = __builtin_amdgcn_ballot_w64(has && exc[u] <= b1 && b1 < exc[u] + nb[u] + c);
        if (hit0 != 0) {
            const int l = __builtin_ctzll(hit0);
            const int n = __builtin_amdgcn_readlane(nb[u], l);
            r.s0 = 64 * u + l;
            r.rs0 = __builtin_amdgcn_readlane(ex[u], l);
            r.p0 = r.rs0 + tile_at_cost(b0 - __builtin_amdgcn_readlane(exc[u], l), n, n + c);
        }
        if (hit1 != 0) {
            const int l = __builtin_ctzll(hit1);
            const int n = __builtin_amdgcn_readlane(nb[u], l);
            r.p1 = __builtin_amdgcn_readlane(ex[u], l) +
                   tile_at_cost(b1 - __builtin_amdgcn_readlane(exc[u], l), n, n + c);
        }
    }
    return r;
}

// One wave per (share, KV head): consecutive workgroups take consecutive KV
// heads of one share, so the head tiles of each physical block (adjacent in
// the pool) are read at about the same time, each head by the same compute
// die throughout.
template <int D, int F, int SLOT, int MINW>
__global__ __launch_bounds__(64, MINW) void decode_mfma_kernel(const int32_t* ctx, int32_t* rows, int num_seqs,
                                                               int max_blocks, int num_kv_heads, int shares,
                                                               int row_cost, int group, DecodeArgs args)
{
    // the leading arguments (the same values as args' fields) are preloaded
    // into registers, so the work split's loads wait for no argument load
    DecodeArgs a = args;
    a.ctx = ctx;
    a.rows = rows;
    a.num_seqs = num_seqs;
    a.max_blocks = max_blocks;
    a.num_kv_heads = num_kv_heads;
    a.shares = shares;
    a.row_cost = row_cost;
    static_assert(SLOT >= 2 && SLOT % 2 == 0, "slots hold pairs of tiles");
    constexpr bool KI8 = MCfg<D, F>::I8;  // K codes on the int8 matrix cores
    const int kvh = blockIdx.x % a.num_kv_heads;
    const int share = blockIdx.x / a.num_kv_heads;
    const int lane = threadIdx.x;
    const int g = lane >> 4, n = lane & 15;
    const ShareLoc loc = locate_share(a, share, lane);
    const int64_t p0 = loc.p0, p1 = loc.p1;
    if (p0 >= p1) return;

    // the current chunk's block ids (ids outside the pool as -1), staged in
    // LDS and read back as a broadcast per tile
    __shared__ int mbid[kMaxChunkBlocks];
    __shared__ u32x4 kl[SLOT * MCfg<D, F>::TILE / 16];  // K of one slot on its way to operand order
    // lane (g, n) serves head n mod 8 of the group; columns 8..15 repeat the
    // group so that rows 8..15 of P can carry the lo halves
    const int qh = n & 7;
    const float lo_sel = n >= 8 ? 1.0f : 0.0f;
    constexpr int kIdRegs = kMaxChunkBlocks / 64;

    // Segment order: a share's first segment usually starts inside its row;
    // every later one starts at a row's first block. The later ones go first,
    // the first one last, so the rows starting in this share are read from
    // their first block at the start of the decode -- where sequences that
    // share a prefix keep their common blocks, now read by all of them at
    // about the same time, which the caches absorb.
    auto nblk = [&](int r) { return clamp_blocks(a.ctx[r], a.max_blocks); };  // tiles of row r
    auto next_row = [&](int r) {  // the next row with tiles (exists while tiles remain)
        do {
            ++r;
        } while (r < a.num_seqs - 1 && nblk(r) == 0);
        return r;
    };
    const int s0 = loc.s0;  // the row holding tile p0
    const int j0 = (int)(p0 - loc.rs0);
    const int nseg0 = (int)min((int64_t)(nblk(s0) - j0), p1 - p0);
    const bool deferred = j0 > 0 && p0 + nseg0 < p1;  // the first segment waits for the others
    int ws = deferred ? next_row(s0) : s0;  // the main walk's next segment
    int wj = deferred ? 0 : j0;
    int64_t wpos = deferred ? p0 + nseg0 : p0;
    bool pending = deferred;
    struct Seg {
        int s, j, nseg;
    };
    auto take_segment = [&](Seg& sg) {
        if (wpos < p1) {
            sg = Seg{ws, wj, (int)min((int64_t)(nblk(ws) - wj), p1 - wpos)};
            wpos += sg.nseg;
            if (wpos < p1) {
                ws = next_row(ws);
                wj = 0;
            }
            return true;
        }
        if (pending) {
            sg = Seg{s0, j0, nseg0};
            pending = false;
            return true;
        }
        return false;
    };

    // A chunk is up to kMaxChunkBlocks blocks of one segment. The next
    // chunk's table entries (and, when it starts a row, that row's query) are
    // loaded while the current chunk is computed, so switching chunks or rows
    // does not wait on memory.
    // The chunk's table entries, and for its first 64 blocks the entries the
    // rows before and after hold at the same positions (-2 where there is no
    // such row): equal ids mark blocks shared with a neighbouring row.
    auto fetch_ids = [&](const Seg& sg, int c0, int (&tb)[kIdRegs], int& tp, int& tn) {
        const int nloc = min(sg.nseg - c0, kMaxChunkBlocks);
        const int64_t at = (int64_t)sg.s * a.max_blocks + sg.j + c0;
#pragma unroll
        for (int r = 0; r < kIdRegs; ++r) {
            const int i = lane + 64 * r;
            tb[r] = i < nloc ? a.tables[at + i] : -1;
        }
        tp = lane < nloc && sg.s > 0 ? a.tables[at - a.max_blocks + lane] : -2;
        tn = lane < nloc && sg.s + 1 < a.num_seqs ? a.tables[at + a.max_blocks + lane] : -2;
    };
    auto q_row = [&](int row) {
        return static_cast<const _Float16*>(a.q) + ((int64_t)row * a.num_q_heads + kvh * group + qh) * D;
    };
    Seg cg;
    take_segment(cg);  // the share holds at least one tile
    int cc0 = 0;
    int tb[kIdRegs], tp, tn;
    QRaw<D, KI8> qraw;
    fetch_ids(cg, 0, tb, tp, tn);
    fetch_q<D, KI8>(qraw, q_row(cg.s), qh < group, g);
    QOp<D, KI8> qo;
    MState<D, F> st;
    while (true) {
        const int nloc = min(cg.nseg - cc0, kMaxChunkBlocks);
        // The run of blocks at the chunk's start that a neighbouring row also
        // references (within its first 64) is read with the default cache
        // policy, the rest non-temporally. Only the policy depends on the
        // neighbours, never the order of the arithmetic.
        const uint64_t same = __builtin_amdgcn_ballot_w64(lane < nloc && tb[0] >= 0 && (tb[0] == tp || tb[0] == tn));
        const int shared_len = ~same == 0 ? 64 : (int)__builtin_ctzll(~same);
        const int jb = cg.j + cc0;  // first block of the chunk within the row
        const bool seg_first = cc0 == 0;
        const bool seg_last = cc0 + kMaxChunkBlocks >= cg.nseg;
        int ctx = a.ctx[cg.s];
        ctx = ctx < 0 ? 0 : (ctx > a.max_blocks * kBlockTokens ? a.max_blocks * kBlockTokens : ctx);
        // live token rows of the chunk, counted from its first block
        const int live = min(ctx, (jb + nloc) * kBlockTokens) - jb * kBlockTokens;

        __syncthreads();  // the previous chunk is done with mbid
#pragma unroll
        for (int r = 0; r < kIdRegs; ++r) {
            const int i = lane + 64 * r;
            if (i < nloc) mbid[i] = (uint64_t)(int64_t)tb[r] < (uint64_t)a.num_blocks ? tb[r] : -1;
        }
        __syncthreads();

        // Two-slot ring: one slot is computed while the other's loads are in
        // flight. Tiles past the chunk load nothing (zero-byte descriptors)
        // and all their rows are dead; the loop takes two slots a step, and a
        // second slot wholly past the chunk is not computed.
        MTile<D, F> ring[2][SLOT];
        float ks[2][SLOT], vs[2][SLOT];
        // a slot's ids are read from LDS one slot ahead of its loads
        auto read_ids = [&](int (&e)[SLOT], int j0_) {
#pragma unroll
            for (int u = 0; u < SLOT; ++u) e[u] = mbid[j0_ + u < nloc ? j0_ + u : 0];
        };
        // issue the loads of ring slot r (blocks j0_ .. j0_ + SLOT - 1 of the
        // chunk) with cache policy AUX (an instruction field)
        auto load_slot = [&](auto aux, int r, const int (&e)[SLOT], int j0_) {
            constexpr int AUX = decltype(aux)::value;
#pragma unroll
            for (int u = 0; u < SLOT; ++u) {
                const int bid = uniform(e[u]);
                const bool valid = j0_ + u < nloc;
                mscales<D, F>(a, bid, valid, kvh, ks[r][u], vs[r][u]);
                mload<D, F, AUX>(ring[r][u], a, bid, valid, kvh, lane);
            }
        };
        // Slots before `split` (the chunk's shared run, rounded down to whole
        // slots) are loaded with the default policy, the rest non-temporally.
        // The policy is fixed per loop (a shared phase, one step that crosses
        // into the private blocks, a private phase), never chosen by a branch
        // inside the loop body: such a branch made the compiler wait for every
        // load in flight, the next slot's included, before computing a slot.
        const std::integral_constant<int, kKvAuxShared> shp{};
        const std::integral_constant<int, PA_KV_AUX> prv{};
        const int split = min(shared_len, nloc) / SLOT * SLOT;
        int e0[SLOT], e1[SLOT];
        read_ids(e0, 0);
        read_ids(e1, SLOT);
        if (split > 0)
            load_slot(shp, 0, e0, 0);
        else
            load_slot(prv, 0, e0, 0);

        if (seg_first) {  // a new row: its query operand and a fresh state
            make_q<D, KI8>(qo, qraw);
#pragma unroll
            for (int nb = 0; nb < MCfg<D, F>::DPL; ++nb) st.acc[nb] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
            st.m = -INFINITY;
            st.l = 0.0f;
            st.vr = 0.0f;
            st.vinv = 0.0f;
        }
        // the next chunk: prefetch its ids (and a new row's query)
        Seg ng = cg;
        int nc0 = cc0 + kMaxChunkBlocks;
        bool have_next = true;
        if (seg_last) {
            have_next = take_segment(ng);
            nc0 = 0;
        }
        if (have_next) {
            fetch_ids(ng, nc0, tb, tp, tn);
            if (nc0 == 0) fetch_q<D, KI8>(qraw, q_row(ng.s), qh < group, g);
        }

        // one step of the ring: slot jj + SLOT's loads (policy pb) go out,
        // slot jj is computed, slot jj + 2 SLOT's loads (policy pa) go out,
        // slot jj + SLOT is computed
        auto step = [&](int jj, auto pb, auto pa) {
            read_ids(e0, jj + 2 * SLOT);
            load_slot(pb, 1, e1, jj + SLOT);
            __builtin_amdgcn_sched_barrier(0);
            mslot<D, F, SLOT>(st, ring[0], qo, live - jj * kBlockTokens, a.scale_log2, ks[0], vs[0], lane,
                               lo_sel, kl);
            __builtin_amdgcn_sched_barrier(0);
            read_ids(e1, jj + 3 * SLOT);
            load_slot(pa, 0, e0, jj + 2 * SLOT);
            __builtin_amdgcn_sched_barrier(0);
            if (jj + SLOT < nloc)  // a slot wholly past the chunk changes nothing
                mslot<D, F, SLOT>(st, ring[1], qo, live - (jj + SLOT) * kBlockTokens, a.scale_log2, ks[1],
                                   vs[1], lane, lo_sel, kl);
            __builtin_amdgcn_sched_barrier(0);
        };
        int jj = 0;
        for (; jj < nloc && jj + 2 * SLOT < split; jj += 2 * SLOT) step(jj, shp, shp);
        if (jj < nloc && jj + SLOT < split) {  // split == jj + 2 SLOT
            step(jj, shp, prv);
            jj += 2 * SLOT;
        }
        for (; jj < nloc; jj += 2 * SLOT) step(jj, prv, prv);

        if (seg_last) {
            const int nb = nblk(cg.s);
            // slot 1: a segment from its row's first block (the row goes on
            // past this share: it is the share's last segment, and this share
            // holds the row's first tile); slot 0: one from inside its row
            // (the share's first segment)
            emit<D, F>(st, a, cg.s, kvh, group, share, cg.j > 0 || cg.j + cg.nseg < nb, cg.j == 0 ? 1 : 0);
        }
        if (!have_next) break;
        cg = ng;
        cc0 = nc0;
    }
}

template <int D, int F>
hipError_t launch_waves(const DecodeArgs& a, int group, hipStream_t st)
{
    const int64_t waves = (int64_t)a.shares * a.num_kv_heads;
    hipLaunchKernelGGL((decode_mfma_kernel<D, F, Launch<D, F>::SLOT, Launch<D, F>::MINW>), dim3((unsigned)waves),
                       dim3(64), 0, st, a.ctx,
                       a.rows, a.num_seqs, a.max_blocks, a.num_kv_heads, a.shares, a.row_cost, group, a);
    return hipGetLastError();
}

}  // namespace

int decode_row_cost(int, int fmt)
{
    // What a wave spends on each row it starts (the table staging, the ring
    // filling again, the query and the epilogue), in tiles of streaming: per-
    // wave clock stamps put it near 3 us per row touched against 0.7 us per
    // INT8 tile, and a sweep of the mixed-length batch was fastest from 8 to
    // 12 for the one-byte caches (each share then also ends nearer the die
    // mean), 10 being 1.6 % faster than 8 on 300 ragged sequences; fp16
    // tiles take twice as long to stream, and with two-tile slots 6 to 10
    // suited the ragged batches of 300 and 1,000 sequences best (2 % and
    // 0.6 % faster than 3), the mixed batch alike within 0.3 %.
    return fmt == kKvF16 ? 6 : 10;
}

int decode_waves_per_cu(int head_dim, int fmt)
{
    // four SIMDs per compute unit
    if (head_dim == 64) return 4 * (fmt == kKvF16 ? Launch<64, kKvF16>::WAVES : Launch<64, kKvI8>::WAVES);
    return 4 * (fmt == kKvF16 ? Launch<128, kKvF16>::WAVES : Launch<128, kKvI8>::WAVES);
}

hipError_t launch_decode_waves(const DecodeArgs& a, int head_dim, int group, int fmt, hipStream_t st)
{
    if (head_dim == 128) {
        if (fmt == kKvI8) return launch_waves<128, kKvI8>(a, group, st);
        if (fmt == kKvF8) return launch_waves<128, kKvF8>(a, group, st);
        return launch_waves<128, kKvF16>(a, group, st);
    }
    if (head_dim == 64) {
        if (fmt == kKvI8) return launch_waves<64, kKvI8>(a, group, st);
        if (fmt == kKvF8) return launch_waves<64, kKvF8>(a, group, st);
        return launch_waves<64, kKvF16>(a, group, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace pa
