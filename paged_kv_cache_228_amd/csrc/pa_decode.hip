// Paged decode attention for gfx950 (MI355X): the work split that precedes
// the matrix-core decode waves (pa_decode_mfma.hip).
//
// What is computed (paged-attention-runtime summary, "CORE CAPABILITIES" 2:
// block-table indirection, online single-pass softmax, fp32 accumulation;
// PagedKV-Fusion README, "Overview": per-(block, head) INT8 decode attention
// with GQA): for sequence s and query head h, out = sum_t softmax_t(scale *
// q.k_t) v_t over the sequence's tokens, K/V reached through the block table
// (glossary monograph, section 2.1).
//
// 1. the work split: the context lengths become tile prefix sums
//    rows[s] = sum_{s' < s} ceil(ctx_s' / 16) (total T = rows[S]) and cost
//    prefix sums (each row with tiles also costs the row cost; pa_split.h).
//    Up to kScanSeqs sequences every decode wave scans them itself; beyond
//    that the prep kernel below does it once, before the waves, and also
//    stores for every share k the row whose cost range holds b_k = k Q / K.
// 2. the decode waves (pa_decode_mfma.hip) stream their shares; rows inside
//    one share are finished there, cut rows leave one partial per share.
// 3. merge: one wave per (sequence, query head) of a cut row combines its
//    partials (log-sum-exp: M = max m_k, out = sum 2^(m_k - M) acc_k /
//    sum 2^(m_k - M) l_k); the rows of empty contexts are written as zeros.
#include <mutex>

#include "pa_internal.h"
#include "pa_split.h"

namespace pa {
namespace {

__global__ __launch_bounds__(kPrepThreads) void decode_prep_kernel(DecodeArgs a)
{
    const int t = threadIdx.x;
    __shared__ int wsum[2][kPrepThreads / 64];
    __shared__ int carry_s[2];
    const int lane = t & 63, w = t >> 6;
    int32_t* costs = a.rows + ws_costs(a.num_seqs);
    int carry = 0, ccarry = 0;  // tiles and cost of the rows so far
    for (int base = 0; base < a.num_seqs; base += kPrepThreads) {
        const int s = base + t;
        const int nb = s < a.num_seqs ? clamp_blocks(a.ctx[s], a.max_blocks) : 0;
        const int rc = (int)row_cost_of(nb, a.row_cost);
        // inclusive scans within the wave, then across the waves
        int x = nb, y = rc;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int xu = __shfl_up(x, d, 64), yu = __shfl_up(y, d, 64);
            if (lane >= d) {
                x += xu;
                y += yu;
            }
        }
        if (lane == 63) {
            wsum[0][w] = x;
            wsum[1][w] = y;
        }
        __syncthreads();
        int before = carry, cbefore = ccarry;
        for (int i = 0; i < w; ++i) {
            before += wsum[0][i];
            cbefore += wsum[1][i];
        }
        if (s < a.num_seqs) {
            a.rows[s] = before + x - nb;
            costs[s] = cbefore + y - rc;
        }
        if (t == kPrepThreads - 1) {
            carry_s[0] = before + x;
            carry_s[1] = cbefore + y;
        }
        __syncthreads();
        carry = carry_s[0];
        ccarry = carry_s[1];
        __syncthreads();
    }
    if (t == 0) {
        a.rows[a.num_seqs] = carry;
        costs[a.num_seqs] = ccarry;
    }
    __syncthreads();  // rows[] and costs[] complete for this workgroup

    // the row holding share k's first tile is the row whose cost range holds
    // b_k (none when no sequence has a tile)
    const int64_t Q = ccarry, K = a.shares;
    if (Q == 0) return;
    int32_t* first_row = a.rows + ws_first_row(a.num_seqs);
    for (int s = t; s < a.num_seqs; s += kPrepThreads) {
        const int64_t c0 = costs[s], c1 = costs[s + 1];
        const int64_t k1 = min(first_share_at(c1, Q, K), K);
        for (int64_t k = first_share_at(c0, Q, K); k < k1; ++k) first_row[k] = s;
    }
}

constexpr int kMergeShares = 8;

template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(int32_t* rows, int num_seqs, int shares,
                                                          int num_kv_heads, int group, DecodeArgs args)
{
    // the leading arguments (the same values as args' fields) are preloaded
    // into registers, so the first loads wait for no argument load
    DecodeArgs a = args;
    a.rows = rows;
    a.num_seqs = num_seqs;
    a.shares = shares;
    a.num_kv_heads = num_kv_heads;
    const int hq = blockIdx.x, s = blockIdx.y;
    const int lane = threadIdx.x;
    const int32_t* costs = a.rows + ws_costs(a.num_seqs);
    const int32_t r0 = a.rows[s], r1 = a.rows[s + 1], cs0 = costs[s], cs1 = costs[s + 1],
                  cq = costs[a.num_seqs];
    // these scalar loads (and the arguments used later) in flight together:
    // one memory round trip, not one per use
    asm volatile("" ::"s"(r0), "s"(r1), "s"(cs0), "s"(cs1), "s"(cq), "s"(a.shares), "s"(a.num_kv_heads),
                 "s"(a.part), "s"(group));
    const int64_t nb = r1 - r0;
    const int64_t c0 = cs0, c1 = cs1, Q = cq, K = a.shares;
    float* o = a.out + ((int64_t)s * a.num_q_heads + hq) * D;
    constexpr int NC = D / 64;
    if (nb == 0) {  // empty context: a zero row
#pragma unroll
        for (int c = 0; c < NC; ++c) o[lane + 64 * c] = 0.0f;
        return;
    }
    // the shares holding the row's first and last tile (pa_split.h: the
    // shares of the last units of their cost intervals)
    const int64_t R = c1 - c0;  // nb + c, below 2^31 like every row's tile count
    const int64_t kf = share_of(c0 + (int64_t)((uint32_t)R / (uint32_t)nb) - 1, Q, K);
    const int64_t kl = share_of(c1 - 1, Q, K);
    if (kf == kl) return;  // finished by its one share
    const int kvh = hq / group, qi = hq - kvh * group;
    const int64_t nslot = K * a.num_kv_heads * 2 * group;
    // Partial entry of share k, and whether share k holds tiles of the row:
    // the first does; a later one from the tile at b_k up to the one before
    // the tile at b_{k+1}, if that is another tile, or to the row's end. No
    // share is empty when each spans at least the widest tile (1 + c units,
    // c the row cost the split used: R - nb, the same for every row of the
    // call, and 0 for rows of equal length); with c = 0 a tile is one unit.
    const int64_t c = R - nb;
    const bool none_empty = Q >= K * (1 + c);
    // kMergeShares shares per round: lane u (mod kMergeShares) finds whether
    // share k0 + u holds tiles of the row and where its partial is, so the
    // shares' tests run side by side and every load of the round (m, l and
    // acc of each share) is in flight together; the combine then takes the
    // shares in order, as one wave-uniform sum (rows rarely span more than
    // one round). Across rounds a running maximum M rescales what has been
    // summed (the log-sum-exp combine, one round at a time).
    const int u = lane & (kMergeShares - 1);
    float num[NC] = {};
    float den = 0.0f, M = -INFINITY;
    for (int64_t k0 = kf; k0 <= kl; k0 += kMergeShares) {
        const int64_t k = k0 + u;
        bool live = k <= kl;
        if (live && k != kf && !none_empty) {
            const int64_t b0 = share_start(k, Q, K), b1 = share_start(k + 1, Q, K);
            live = b1 >= c1 ||
                   (c == 0 ? b1 != b0 : tile_at_cost(b1 - c0, nb, R) != tile_at_cost(b0 - c0, nb, R));
        }
        // slot 1 holds the row in the share holding its first tile (the row
        // is that share's last segment), slot 0 in every later share (the
        // row is that share's first segment)
        const int slot = k == kf ? 1 : 0;
        const int64_t e = ((k * a.num_kv_heads + kvh) * 2 + slot) * group + qi;
        const float m = live ? a.part[nslot * D + e] : -INFINITY;
        const float l = live ? a.part[nslot * (D + 1) + e] : 0.0f;
        const uint64_t lives = __builtin_amdgcn_ballot_w64(live);
        float x[kMergeShares][NC];
#pragma unroll
        for (int v = 0; v < kMergeShares; ++v) {
            const int64_t ev = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(e >> 32), v) << 32) |
                                         (uint32_t)__builtin_amdgcn_readlane((int)e, v));
#pragma unroll
            for (int cc = 0; cc < NC; ++cc)
                x[v][cc] = (lives >> v & 1) ? a.part[ev * D + lane + 64 * cc] : 0.0f;
        }
        float mv[kMergeShares], lvv[kMergeShares];
        float mn = M;
#pragma unroll
        for (int v = 0; v < kMergeShares; ++v) {
            mv[v] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m), v));
            lvv[v] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l), v));
            mn = fmaxf(mn, mv[v]);
        }
        const float al = mn == M ? 1.0f : __builtin_amdgcn_exp2f(M - mn);  // 0 on the first round
        den *= al;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) num[cc] *= al;
#pragma unroll
        for (int v = 0; v < kMergeShares; ++v) {
            const float w = mv[v] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mv[v] - mn);
            den += w * lvv[v];
#pragma unroll
            for (int cc = 0; cc < NC; ++cc) num[cc] += w * x[v][cc];
        }
        M = mn;
    }
    const float inv = 1.0f / den;
#pragma unroll
    for (int c = 0; c < NC; ++c) o[lane + 64 * c] = num[c] * inv;
}

}  // namespace

// The decode workspace of pa_paged_decode_int8_noalloc: a file-scope device
// array each GPU holds from the library's load until the process ends. On the
// host its name stands in for the array and is not a device address, so its
// per-device address is looked up once per device (with that device current)
// and only that address is handed to kernels.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, int head_dim, int group, int fmt, hipStream_t st)
{
    hipError_t e;
    if (a.num_seqs > kScanSeqs) {
        hipLaunchKernelGGL(decode_prep_kernel, dim3(1), dim3(kPrepThreads), 0, st, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    e = launch_decode_waves(a, head_dim, group, fmt, st);
    if (e != hipSuccess) return e;
    const dim3 grid(a.num_q_heads, a.num_seqs);
    if (head_dim == 64)
        hipLaunchKernelGGL(decode_merge_kernel<64>, grid, dim3(64), 0, st, a.rows, a.num_seqs, a.shares,
                           a.num_kv_heads, group, a);
    else if (head_dim == 128)
        hipLaunchKernelGGL(decode_merge_kernel<128>, grid, dim3(64), 0, st, a.rows, a.num_seqs, a.shares,
                           a.num_kv_heads, group, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pa
