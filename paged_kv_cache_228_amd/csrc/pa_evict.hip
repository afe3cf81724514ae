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
//      sums of per-thread counts give each chosen id its output slot.
// Each thread takes 16 consecutive blocks per step (16-byte loads); the block
// metadata (8 bytes per block) is re-read per pass from the cache.
#include <climits>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kEvictThreads = 1024;
constexpr int kWaves = kEvictThreads / 64;
constexpr int kPerThread = 16;                          // consecutive blocks per thread and step
constexpr int kPerStep = kEvictThreads * kPerThread;    // blocks per step

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int64_t block_key(int32_t ref, int32_t last, int32_t tick)
{
    return 3 * ((int64_t)tick - last) - 7 * (int64_t)ref;
}

// The metadata of this thread's kPerThread blocks starting at `first`;
// blocks past the pool read as free (refcount 0).
__device__ __forceinline__ void load_blocks(const EvictArgs& a, int64_t first, int32_t (&ref)[kPerThread],
                                            int32_t (&last)[kPerThread])
{
    if (first + kPerThread <= a.num_blocks) {
#pragma unroll
        for (int c = 0; c < kPerThread / 4; ++c) {
            const i32x4 r = *reinterpret_cast<const i32x4*>(a.refcount + first + 4 * c);
            const i32x4 l = *reinterpret_cast<const i32x4*>(a.last_used + first + 4 * c);
            ref[4 * c] = r.x, ref[4 * c + 1] = r.y, ref[4 * c + 2] = r.z, ref[4 * c + 3] = r.w;
            last[4 * c] = l.x, last[4 * c + 1] = l.y, last[4 * c + 2] = l.z, last[4 * c + 3] = l.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const bool in = first + i < a.num_blocks;
            ref[i] = in ? a.refcount[first + i] : 0;
            last[i] = in ? a.last_used[first + i] : 0;
        }
    }
}

// Exclusive prefix sum of `x` over the workgroup (thread order) and the
// workgroup's total. `part` holds kWaves ints of LDS.
__device__ __forceinline__ int block_prefix(int x, int* part, int& total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int incl = x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d, 64);
        incl += lane >= d ? y : 0;
    }
    if (lane == 63) part[w] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
    for (int i = 0; i < kWaves; ++i) {
        const int c = part[i];
        before += i < w ? c : 0;
        total += c;
    }
    __syncthreads();  // part[] is reused by the next call
    return before + incl - x;
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
    int32_t ref[kPerThread], last[kPerThread];

    // 1. range of the keys and number of candidates
    long long kmin = LLONG_MAX, kmax = LLONG_MIN;
    int cnt = 0;
    for (int64_t base = 0; base < a.num_blocks; base += kPerStep) {
        load_blocks(a, base + (int64_t)t * kPerThread, ref, last);
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            if (ref[i] <= 0) continue;
            const long long key = block_key(ref[i], last[i], a.tick);
            kmin = key < kmin ? key : kmin;
            kmax = key > kmax ? key : kmax;
            ++cnt;
        }
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
            for (int64_t base = 0; base < a.num_blocks; base += kPerStep) {
                load_blocks(a, base + (int64_t)t * kPerThread, ref, last);
#pragma unroll
                for (int i = 0; i < kPerThread; ++i) {
                    if (ref[i] <= 0) continue;
                    const unsigned long long u = (unsigned long long)(block_key(ref[i], last[i], a.tick) - kmin);
                    if (shift + 8 < 64 && (u >> (shift + 8)) != (prefix >> (shift + 8))) continue;
                    atomicAdd(&hist[(u >> shift) & 255u], 1u);
                }
            }
            __syncthreads();
            // the digit holding the remaining-th largest: thread j looks at
            // digit 255 - j; an exclusive prefix sum over the threads counts
            // the keys in larger digits
            const int d = 255 - t;
            const int h = t < 256 ? (int)hist[d] : 0;
            int all;
            const long long above = block_prefix(h, part, all);
            const long long rem = s_remaining;
            __syncthreads();  // everyone has read s_remaining
            if (t < 256 && above < rem && rem <= above + h) {
                s_remaining = rem - above;
                s_prefix = prefix | ((unsigned long long)d << shift);
            }
            __syncthreads();
        }
    }
    const unsigned long long thr = s_prefix;  // the keff-th largest u
    const long long take_equal = s_remaining;  // how many of u == thr are chosen

    // 3. chosen ids in block order: each thread holds kPerThread consecutive
    // blocks; prefix sums of per-thread counts give each its rank among the
    // keys equal to the threshold and its first output slot
    long long chosen = 0, equal_seen = 0;
    for (int64_t base = 0; keff > 0 && base < a.num_blocks; base += kPerStep) {
        const int64_t first = base + (int64_t)t * kPerThread;
        load_blocks(a, first, ref, last);
        unsigned gt = 0, eq = 0;  // bit i: block first + i
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            if (ref[i] <= 0) continue;
            const unsigned long long u = (unsigned long long)(block_key(ref[i], last[i], a.tick) - kmin);
            gt |= (u > thr ? 1u : 0u) << i;
            eq |= (u == thr ? 1u : 0u) << i;
        }
        int n_eq;
        long long eq_rank = equal_seen + block_prefix(__popc(eq), part, n_eq);
        unsigned sel = gt;
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            if (!((eq >> i) & 1u)) continue;
            if (eq_rank < take_equal) sel |= 1u << i;
            ++eq_rank;
        }
        int n_sel;
        long long pos = chosen + block_prefix(__popc(sel), part, n_sel);
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            if (!((sel >> i) & 1u)) continue;
            if (pos < keff) a.out[pos] = (int32_t)(first + i);  // pos < keff always; the guard keeps
            ++pos;                                              // a wrong threshold in bounds
        }
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
