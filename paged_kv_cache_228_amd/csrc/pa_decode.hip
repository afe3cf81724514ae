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
//    rows[s] = sum_{s' < s} ceil(ctx_s' / 16) (total T = rows[S]). Up to
//    kScanSeqs sequences every decode wave scans them itself; beyond that
//    the prep kernel below does it once, before the waves, and also stores
//    for every share k of [0, T) the row holding its first tile k T / shares.
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
    __shared__ int wsum[kPrepThreads / 64];
    __shared__ int carry_s;
    const int lane = t & 63, w = t >> 6;
    int carry = 0;
    for (int base = 0; base < a.num_seqs; base += kPrepThreads) {
        const int s = base + t;
        const int nb = s < a.num_seqs ? clamp_blocks(a.ctx[s], a.max_blocks) : 0;
        // inclusive scan within the wave, then across the waves
        int x = nb;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(x, d, 64);
            if (lane >= d) x += y;
        }
        if (lane == 63) wsum[w] = x;
        __syncthreads();
        int before = carry;
        for (int i = 0; i < w; ++i) before += wsum[i];
        if (s < a.num_seqs) a.rows[s] = before + x - nb;
        if (t == kPrepThreads - 1) carry_s = before + x;
        __syncthreads();
        carry = carry_s;
        __syncthreads();
    }
    if (t == 0) a.rows[a.num_seqs] = carry;
    __syncthreads();  // rows[] complete for this workgroup

    const int64_t T = carry, K = a.shares;
    int32_t* first_row = a.rows + ws_first_row(a.num_seqs);
    for (int s = t; s < a.num_seqs; s += kPrepThreads) {
        const int64_t r0 = a.rows[s], r1 = a.rows[s + 1];
        // shares whose first tile lies in [r0, r1)
        const int64_t k1 = min(first_share_at(r1, T, K), K);
        for (int64_t k = first_share_at(r0, T, K); k < k1; ++k) first_row[k] = s;
    }
}

constexpr int kMergeShares = 8;

template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a, int group)
{
    const int hq = blockIdx.x, s = blockIdx.y;
    const int lane = threadIdx.x;
    const int64_t r0 = a.rows[s], r1 = a.rows[s + 1], T = a.rows[a.num_seqs], K = a.shares;
    float* o = a.out + ((int64_t)s * a.num_q_heads + hq) * D;
    constexpr int NC = D / 64;
    if (r1 == r0) {  // empty context: a zero row
#pragma unroll
        for (int c = 0; c < NC; ++c) o[lane + 64 * c] = 0.0f;
        return;
    }
    // the first and the last share holding the row's tiles
    const int64_t kf = share_of(r0, T, K), kl = share_of(r1 - 1, T, K);
    if (kf == kl) return;  // finished by its one share
    const int kvh = hq / group, qi = hq - kvh * group;
    const int64_t nslot = K * a.num_kv_heads * 2 * group;
    // partial entry of share k (0 when it holds no tile of the row)
    auto entry = [&](int64_t k, bool& live) {
        live = k <= kl && (T >= K || !share_empty(k, T, K));
        // the first share holds the row in its last slot unless the row starts its range
        const int slot = (k == kf && k * T / K < r0) ? 1 : 0;
        return ((k * a.num_kv_heads + kvh) * 2 + slot) * group + qi;
    };
    // kMergeShares shares per round, their m, l and acc loads all in flight
    // together (rows rarely span more); across rounds a running maximum M
    // rescales what has been summed (the log-sum-exp combine, one round at a
    // time)
    float num[NC] = {};
    float den = 0.0f, M = -INFINITY;
    for (int64_t k0 = kf; k0 <= kl; k0 += kMergeShares) {
        float m[kMergeShares], l[kMergeShares], x[kMergeShares][NC];
#pragma unroll
        for (int u = 0; u < kMergeShares; ++u) {
            bool live;
            const int64_t e = entry(k0 + u, live);
            m[u] = live ? a.part[nslot * D + e] : -INFINITY;
            l[u] = live ? a.part[nslot * (D + 1) + e] : 0.0f;
#pragma unroll
            for (int c = 0; c < NC; ++c) x[u][c] = live ? a.part[e * D + lane + 64 * c] : 0.0f;
        }
        float mn = M;
#pragma unroll
        for (int u = 0; u < kMergeShares; ++u) mn = fmaxf(mn, m[u]);
        const float al = mn == M ? 1.0f : __builtin_amdgcn_exp2f(M - mn);  // 0 on the first round
        den *= al;
#pragma unroll
        for (int c = 0; c < NC; ++c) num[c] *= al;
#pragma unroll
        for (int u = 0; u < kMergeShares; ++u) {
            const float w = m[u] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m[u] - mn);
            den += w * l[u];
#pragma unroll
            for (int c = 0; c < NC; ++c) num[c] += w * x[u][c];
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
    if (head_dim == 64) hipLaunchKernelGGL(decode_merge_kernel<64>, grid, dim3(64), 0, st, a, group);
    else if (head_dim == 128) hipLaunchKernelGGL(decode_merge_kernel<128>, grid, dim3(64), 0, st, a, group);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pa
