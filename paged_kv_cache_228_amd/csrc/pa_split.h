// Share arithmetic of the decode's work split, used by the prep kernel, the
// decode waves and the merge. Each KV head's tiles (all sequences in order)
// are laid on a cost line: a row of nb > 0 tiles costs R = nb + c (c, the row
// cost, stands for what a wave spends on starting a row), spread over its
// tiles, so tile j of the row covers [C + j R / nb, C + (j + 1) R / nb) with
// C the cost of the rows before it (integer division). The total cost Q is cut
// into K shares at b_k = k Q / K, and a tile belongs to the share holding the
// last unit of its interval: share k holds the tiles whose interval ends in
// (b_k, b_{k+1}], i.e. from the tile whose interval holds b_k up to the one
// before the tile whose interval holds b_{k+1}. With c = 0 a tile is one unit
// and share k is the tiles [k T / K, (k + 1) T / K).
#pragma once

#include "pa_internal.h"

namespace pa {

// floor(x / y) for 0 <= x < 2^63 and 0 < y, when the quotient is below 2^31
// (every quotient of the split is: a share index, a tile index or a cost
// below 2^31): a double-precision estimate, within one of the quotient, then
// corrected exactly in integers, branch-free and much shorter code than a
// 64-bit division. The estimate multiplies by the hardware reciprocal of y
// refined by two Newton steps (each squares the relative error: from the
// reciprocal's 2^-23 or better to the rounding of double arithmetic), so x/y
// is off by far less than one for quotients below 2^31.
__device__ __forceinline__ int64_t div_floor(int64_t x, int64_t y)
{
    const double yd = (double)y;
    double r = __builtin_amdgcn_rcp(yd);
    r = __builtin_fma(__builtin_fma(-yd, r, 1.0), r, r);
    r = __builtin_fma(__builtin_fma(-yd, r, 1.0), r, r);
    int64_t q = (int64_t)((double)x * r);
    if (q * y > x)
        --q;
    else if ((q + 1) * y <= x)
        ++q;
    return q;
}

__device__ __forceinline__ int clamp_blocks(int ctx, int max_blocks)
{
    const int c = ctx < 0 ? 0 : (ctx > max_blocks * kBlockTokens ? max_blocks * kBlockTokens : ctx);
    return (c + kBlockTokens - 1) / kBlockTokens;
}

// First share whose range starts at or after tile x: the least k with
// k T / K >= x, i.e. ceil(x K / T).
__device__ __forceinline__ int64_t first_share_at(int64_t x, int64_t T, int64_t K)
{
    return div_floor(x * K + T - 1, T);
}

// The share holding tile x (0 <= x < T): the largest k with k T / K <= x.
__device__ __forceinline__ int64_t share_of(int64_t x, int64_t T, int64_t K)
{
    return div_floor((x + 1) * K - 1, T);
}

// Whether share k holds no tile (possible only when T < K).
__device__ __forceinline__ bool share_empty(int64_t k, int64_t T, int64_t K)
{
    return div_floor((k + 1) * T, K) == div_floor(k * T, K);
}

// The cost at which share k starts, b_k = k Q / K.
__device__ __forceinline__ int64_t share_start(int64_t k, int64_t Q, int64_t K) { return div_floor(k * Q, K); }

// Cost of a row of nb tiles with row cost c.
__device__ __forceinline__ int64_t row_cost_of(int64_t nb, int64_t c) { return nb > 0 ? nb + c : 0; }

// The tile of a row (nb tiles, cost R) whose interval holds the cost offset d
// (0 <= d < R): the largest j with j R / nb <= d.
__device__ __forceinline__ int64_t tile_at_cost(int64_t d, int64_t nb, int64_t R)
{
    return div_floor((d + 1) * nb - 1, R);
}

}  // namespace pa
