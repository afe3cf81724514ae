// Eviction choice over the physical KV blocks, gfx950.
//
// Scores (PagedAttention & KV-Cache Memory Management monograph, section
// 4.3.1, least reference count plus age): over the allocated blocks
// (reference count > 0),
//     score = 0.7 (max_refcnt - refcnt) + 0.3 (current_tick - last_used),
// higher = better to evict; the k best (PagedKV-Fusion README: scoring plus a
// top-k over the paged blocks, "bottom-k eviction ids"), equal scores to the
// smaller block id, are returned in ascending id order, -1 past the number of
// candidates.
//
// Ten times the score minus the constant 7 max_refcnt is the integer
//     key = 3 (current_tick - last_used) - 7 refcnt     (int64, exact),
// which orders the blocks exactly as the score does, so no rounding and no
// pass for max_refcnt is needed. One workgroup of 1024 threads:
//   1. min and max key and the candidate count (k' = min(k, count));
//   2. radix select of the k'-th largest key, 8 bits per pass over
//      u = key - min (at most 36 bits: 5 passes, as many as the range needs),
//      with a 256-bin histogram in LDS;
//   3. one pass in block order: keys above the threshold, plus the first
//      (by id) of those equal to it until k' are chosen; block-wide prefix
//      counts (wave ballots) give each chosen id its output slot.
// The block metadata (8 bytes per block) is re-read per pass from the cache.
#include <climits>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kEvictThreads = 1024;
constexpr int kWaves = kEvictThreads / 64;

__device__ __forceinline__ int64_t block_key(int32_t ref, int32_t last, int32_t tick)
{
    return 3 * ((int64_t)tick - last) - 7 * (int64_t)ref;
}

// Exclusive prefix count of `flag` over the workgroup (thread order) and the
// workgroup's total. `part` holds kWaves ints of LDS.
__device__ __forceinline__ int block_prefix(bool flag, int* part, int& total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t m = __ballot(flag);
    const int before_in_wave = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) part[w] = __popcll(m);
    __syncthreads();
    int before = 0;
    total = 0;
    for (int i = 0; i < kWaves; ++i) {
        const int c = part[i];
        before += i < w ? c : 0;
        total += c;
    }
    __syncthreads();  // part[] is reused by the next call
    return before + before_in_wave;
}

__global__ __launch_bounds__(kEvictThreads) void evict_kernel(EvictArgs a)
{
    __shared__ unsigned hist[256];
    __shared__ long long red_min[kWaves], red_max[kWaves];
    __shared__ int red_cnt[kWaves];
    __shared__ int part[kWaves];
    __shared__ unsigned long long s_prefix;
    __shared__ long long s_remaining;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;

    // 1. range of the keys and number of candidates
    long long kmin = LLONG_MAX, kmax = LLONG_MIN;
    int cnt = 0;
    for (int64_t b = t; b < a.num_blocks; b += kEvictThreads) {
        const int32_t r = a.refcount[b];
        if (r <= 0) continue;
        const long long key = block_key(r, a.last_used[b], a.tick);
        kmin = key < kmin ? key : kmin;
        kmax = key > kmax ? key : kmax;
        ++cnt;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        const long long omin = __shfl_xor(kmin, d, 64), omax = __shfl_xor(kmax, d, 64);
        kmin = omin < kmin ? omin : kmin;
        kmax = omax > kmax ? omax : kmax;
        cnt += __shfl_xor(cnt, d, 64);
    }
    if (lane == 0) {
        red_min[w] = kmin;
        red_max[w] = kmax;
        red_cnt[w] = cnt;
    }
    __syncthreads();
    kmin = LLONG_MAX;
    kmax = LLONG_MIN;
    long long count = 0;
    for (int i = 0; i < kWaves; ++i) {
        kmin = red_min[i] < kmin ? red_min[i] : kmin;
        kmax = red_max[i] > kmax ? red_max[i] : kmax;
        count += red_cnt[i];
    }
    const long long keff = a.k < count ? a.k : count;

    // 2. radix select: the keff-th largest u = key - kmin
    if (t == 0) {
        s_prefix = 0;
        s_remaining = keff;
    }
    __syncthreads();
    if (keff > 0) {
        const unsigned long long range = (unsigned long long)(kmax - kmin);
        const int nbits = range ? 64 - __clzll(range) : 0;
        for (int shift = ((nbits + 7) / 8 - 1) * 8; shift >= 0; shift -= 8) {
            if (t < 256) hist[t] = 0;
            __syncthreads();
            const unsigned long long prefix = s_prefix;
            for (int64_t b = t; b < a.num_blocks; b += kEvictThreads) {
                const int32_t r = a.refcount[b];
                if (r <= 0) continue;
                const unsigned long long u = (unsigned long long)(block_key(r, a.last_used[b], a.tick) - kmin);
                if (shift + 8 < 64 && (u >> (shift + 8)) != (prefix >> (shift + 8))) continue;
                atomicAdd(&hist[(u >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (t == 0) {  // the digit holding the remaining-th largest
                long long above = 0, rem = s_remaining;
                int d = 255;
                for (; d > 0; --d) {
                    if (above + hist[d] >= rem) break;
                    above += hist[d];
                }
                s_remaining = rem - above;
                s_prefix = prefix | ((unsigned long long)d << shift);
            }
            __syncthreads();
        }
    }
    const unsigned long long thr = s_prefix;  // the keff-th largest u
    const long long take_equal = s_remaining;  // how many of u == thr are chosen

    // 3. chosen ids in block order
    long long chosen = 0, equal_seen = 0;
    for (int64_t base = 0; keff > 0 && base < a.num_blocks; base += kEvictThreads) {
        const int64_t b = base + t;
        bool gt = false, eq = false;
        if (b < a.num_blocks) {
            const int32_t r = a.refcount[b];
            if (r > 0) {
                const unsigned long long u = (unsigned long long)(block_key(r, a.last_used[b], a.tick) - kmin);
                gt = u > thr;
                eq = u == thr;
            }
        }
        int n_eq;
        const long long eq_rank = equal_seen + block_prefix(eq, part, n_eq);
        const bool sel = gt || (eq && eq_rank < take_equal);
        int n_sel;
        const long long pos = chosen + block_prefix(sel, part, n_sel);
        if (sel && pos < keff) a.out[pos] = (int32_t)b;  // pos < keff always; the guard keeps
                                                       // a wrong threshold from writing out of bounds
        equal_seen += n_eq;
        chosen += n_sel;
    }
    for (int64_t i = keff + t; i < a.k; i += kEvictThreads) a.out[i] = -1;
}

}  // namespace

hipError_t launch_evict(const EvictArgs& a, hipStream_t st)
{
    if (a.k == 0) return hipSuccess;
    hipLaunchKernelGGL(evict_kernel, dim3(1), dim3(kEvictThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace pa
