// KV append for gfx950: the K and V rows of one new token per sequence go
// into the paged cache.
//
// Token t of sequence s lives in physical block b = table[s][t / 16] at slot
// o = t mod 16 (glossary monograph, section 2.1; PagedAttention article,
// "Kernel Mechanics": the new K/V are written at phys_block_id * B +
// token_offset). A negative position, one past the table row, or a table
// entry outside the pool appends nothing.
//
// fp16 cache: the row is copied into the slot.
// INT8 cache (codes plus one fp32 scale per (block, head), the layout that
// pa_quantize_kv_int8 writes): with x the new row, s_old the tile's scale and
// s_new = amax(x) / 127,
//   o == 0 (the block's first token): scale = s_new, row 0 = q(x, s_new);
//   o > 0, s_new <= s_old: row o = q(x, s_old);
//   o > 0, s_new >  s_old: rows r < o become q(code * s_old, s_new) (one fp32
//                          multiply), row o = q(x, s_new), scale = s_new;
// q(v, s) = 0 if s == 0, else clamp(rint(v / s), -127, 127) with an IEEE
// fp32 division -- the quantizer of pa_quantize_kv_int8 at a given scale.
// Rows after o are not touched.
//
// One workgroup per (KV head, sequence): wave 0 appends K, wave 1 V. The work
// is a few hundred bytes per wave; the kernel is bound by its launch.
#include "pa_internal.h"

namespace pa {
namespace {

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x = fmaxf(x, __shfl_xor(x, d, 64));
    return x;
}

// The quantizer at a given scale; NaN inputs give code 0.
__device__ __forceinline__ int quantize_one(float v, float scale)
{
    if (scale == 0.0f) return 0;
    const float r = __builtin_rintf(v / scale);
    if (r != r) return 0;
    return (int)fminf(fmaxf(r, -127.0f), 127.0f);
}

template <int D, bool I8>
__global__ __launch_bounds__(128) void append_kernel(AppendArgs a)
{
    constexpr int EPL = D / 64;  // elements of the row per lane
    const int h = blockIdx.x, s = blockIdx.y;
    const int tensor = threadIdx.x >> 6, lane = threadIdx.x & 63;
    // the new row does not depend on the slot: its load goes out with the
    // position's, before the table entry that the position selects
    const uint16_t* src = (tensor ? a.v_new : a.k_new) + ((int64_t)s * a.num_kv_heads + h) * D + lane * EPL;
    uint32_t raw = EPL == 2 ? *reinterpret_cast<const uint32_t*>(src) : (uint32_t)*src;
    const int t = a.positions[s];
    if (t < 0 || t / kBlockTokens >= a.max_blocks) return;
    const int64_t b = a.tables[(int64_t)s * a.max_blocks + t / kBlockTokens];
    if (b < 0 || b >= a.num_blocks) return;
    const int o = t % kBlockTokens;
    const int64_t tile = (b * a.num_kv_heads + h) * (int64_t)(kBlockTokens * D);

    if (!I8) {
        uint16_t* dst = static_cast<uint16_t*>(tensor ? a.v : a.k) + tile + o * D + lane * EPL;
        if (EPL == 2)
            *reinterpret_cast<uint32_t*>(dst) = raw;
        else
            *dst = (uint16_t)raw;
        return;
    }

    float x[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(raw >> (16 * e)));
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
    amax = wave_max(amax);
    const float s_new = amax / 127.0f;
    float* sp = (tensor ? a.vs : a.ks) + b * a.num_kv_heads + h;
    const float s_old = *sp;
    int8_t* codes = static_cast<int8_t*>(tensor ? a.v : a.k) + tile;
    float sc = s_new;
    if (o > 0 && s_new <= s_old) {
        sc = s_old;
    } else if (o > 0) {
        // re-scale the live rows 0 .. o-1, four codes per lane and step
        for (int e0 = lane * 4; e0 < o * D; e0 += 256) {
            uint32_t w = *reinterpret_cast<const uint32_t*>(codes + e0);
            uint32_t r = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = (int)(int8_t)(w >> (8 * i));
                const int q = quantize_one(__fmul_rn((float)c, s_old), s_new);
                r |= (uint32_t)(q & 0xFF) << (8 * i);
            }
            *reinterpret_cast<uint32_t*>(codes + e0) = r;
        }
    }
    int8_t* row = codes + o * D + lane * EPL;
    if (EPL == 2) {
        const uint32_t q0 = (uint32_t)quantize_one(x[0], sc) & 0xFF;
        const uint32_t q1 = (uint32_t)quantize_one(x[EPL - 1], sc) & 0xFF;
        *reinterpret_cast<uint16_t*>(row) = (uint16_t)(q0 | (q1 << 8));
    } else {
        *row = (int8_t)quantize_one(x[0], sc);
    }
    if (lane == 0) *sp = sc;
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int head_dim, bool int8, hipStream_t st)
{
    if (a.num_seqs == 0) return hipSuccess;
    const dim3 grid(a.num_kv_heads, a.num_seqs);
    if (head_dim == 128) {
        if (int8) hipLaunchKernelGGL((append_kernel<128, true>), grid, dim3(128), 0, st, a);
        else hipLaunchKernelGGL((append_kernel<128, false>), grid, dim3(128), 0, st, a);
    } else if (head_dim == 64) {
        if (int8) hipLaunchKernelGGL((append_kernel<64, true>), grid, dim3(128), 0, st, a);
        else hipLaunchKernelGGL((append_kernel<64, false>), grid, dim3(128), 0, st, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pa
