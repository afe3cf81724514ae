// Share arithmetic of the decode's work split, used by the prep kernel and the
// decode waves. Share k of a KV head's T tiles is [k T / K, (k + 1) T / K)
// (integer division), K shares in all.
#pragma once

#include "pa_internal.h"

namespace pa {

__device__ __forceinline__ int clamp_blocks(int ctx, int max_blocks)
{
    const int c = ctx < 0 ? 0 : (ctx > max_blocks * kBlockTokens ? max_blocks * kBlockTokens : ctx);
    return (c + kBlockTokens - 1) / kBlockTokens;
}

// First share whose range starts at or after tile x: the least k with
// k T / K >= x, i.e. ceil(x K / T).
__device__ __forceinline__ int64_t first_share_at(int64_t x, int64_t T, int64_t K)
{
    return (x * K + T - 1) / T;
}

// The share holding tile x (0 <= x < T): the largest k with k T / K <= x.
__device__ __forceinline__ int64_t share_of(int64_t x, int64_t T, int64_t K)
{
    return ((x + 1) * K - 1) / T;
}

// Whether share k holds no tile (possible only when T < K).
__device__ __forceinline__ bool share_empty(int64_t k, int64_t T, int64_t K)
{
    return (k + 1) * T / K == k * T / K;
}

}  // namespace pa
