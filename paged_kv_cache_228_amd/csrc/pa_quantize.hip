// Symmetric per-(block, KV head) INT8 quantization of fp16 K/V pools, gfx950.
//
// For one (block, head) tile of 16 x D fp16 values (PagedKV-Fusion README,
// "Overview" and "Architecture": per-block,head symmetric INT8; "Memory
// footprint (exact arithmetic)": one fp32 scale for K and one for V per
// (block, head); glossary monograph, section 5.1: code = round(x / S)):
//     amax  = max |x|
//     scale = amax / 127                     IEEE fp32 division
//     code  = clamp(rint(x / scale), -127, 127), rint = round half to even,
//             x / scale an IEEE fp32 division; scale 0 gives code 0.
// One wave per tile: 16-byte loads (1 KiB of contiguous bytes per wave
// instruction), wave-wide max, then 8-byte stores of packed codes.
//
// The quotient x / scale is formed without a full division per element: with
// r = 1 / scale correctly rounded (one IEEE division per tile),
//     q0 = RN(x r),  e = x - q0 scale (exact, one fma),  q = RN(q0 + e r)
// is the correctly rounded quotient (Markstein's correction step; Handbook of
// Floating-Point Arithmetic, Muller et al., section on division with fma).
// For this kernel's domain that was also checked exhaustively: every fp16 x
// with |x| <= amax, for every finite fp16 amax > 0, gives RN(x / scale) bit
// for bit. rint and the int8 conversion use the 1.5 * 2^23 shift: adding it
// rounds a value below 2^22 in magnitude to the nearest integer (ties to
// even) and leaves that integer, two's complement, in the low mantissa bits.
#include "pa_internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

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

__device__ __forceinline__ float wave_max(float x)
{
    x = fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp<0x141>(x));  // row_half_mirror
    x = fmaxf(x, dpp<0x140>(x));  // row_mirror
    x = fmaxf(x, __shfl_xor(x, 16, 64));
    x = fmaxf(x, __shfl_xor(x, 32, 64));
    return x;
}

// Non-temporal loads and stores: the fp16 tiles are read once and the codes
// are read by a later kernel; without the hint the written lines linger in
// the caches in a state that slowed the next reader of those addresses by
// about a fifth.
#ifndef PA_Q_NT
#define PA_Q_NT 1
#endif

// Low byte of the 1.5 * 2^23-shifted code of x (see the file comment).
__device__ __forceinline__ uint32_t shifted_code(float x, float scale, float r)
{
    const float q0 = __fmul_rn(x, r);
    const float e = __builtin_fmaf(-q0, scale, x);
    const float q = __builtin_fmaf(e, r, q0);
    const float c = __builtin_amdgcn_fmed3f(q, -127.0f, 127.0f);
    return __builtin_bit_cast(uint32_t, __fadd_rn(c, 12582912.0f));
}

// Codes of the four fp16 values in words w0, w1, packed as four bytes.
__device__ __forceinline__ uint32_t pack4(uint32_t w0, uint32_t w1, float scale, float r)
{
    const h2_t a = __builtin_bit_cast(h2_t, w0), b = __builtin_bit_cast(h2_t, w1);
    const uint32_t t0 = shifted_code((float)a.x, scale, r), t1 = shifted_code((float)a.y, scale, r);
    const uint32_t t2 = shifted_code((float)b.x, scale, r), t3 = shifted_code((float)b.y, scale, r);
    return __builtin_amdgcn_perm(t1, t0, 0x0C0C0400u) | __builtin_amdgcn_perm(t3, t2, 0x04000C0Cu);
}

// FP8 (OCP E4M3) codes of the four fp16 values in words w0, w1, packed as
// four bytes: the correctly rounded quotient x / scale (as for INT8, with
// the sign of zero kept), then
// the hardware's round-to-nearest-even conversion to E4M3 (|x / scale| <= 448,
// so it never reaches the format's end).
__device__ __forceinline__ uint32_t pack4_fp8(uint32_t w0, uint32_t w1, float scale, float r)
{
    const h2_t a = __builtin_bit_cast(h2_t, w0), b = __builtin_bit_cast(h2_t, w1);
    float q[4] = {(float)a.x, (float)a.y, (float)b.x, (float)b.y};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float q0 = __fmul_rn(q[i], r);
        const float e = __builtin_fmaf(-q0, scale, q[i]);
        // the correction turns -0 into +0; the quotient keeps x's sign (E4M3
        // has a negative zero)
        q[i] = __builtin_copysignf(__builtin_fmaf(e, r, q0), q[i]);
    }
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], v, true);
    return (uint32_t)v;
}

template <int D, bool FP8>
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs a)
{
    constexpr int kChunks = kBlockTokens * D * 2 / 16 / 64;  // 16-byte chunks per lane
    const int lane = threadIdx.x & 63;
    const int64_t per_tensor = a.num_ids * a.num_kv_heads;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= 2 * per_tensor) return;
    const int tensor = t >= per_tensor ? 1 : 0;
    const int64_t r = t - tensor * per_tensor;
    const int64_t idx = r / a.num_kv_heads;
    const int h = (int)(r - idx * a.num_kv_heads);
    const int64_t b = a.ids ? (int64_t)a.ids[idx] : idx;
    if (b < 0 || b >= a.num_blocks) return;

    const int64_t tile = (b * a.num_kv_heads + h) * (int64_t)(kBlockTokens * D);
    const u32x4* src = reinterpret_cast<const u32x4*>((tensor ? a.v : a.k) + tile);
    u32x2* dst = reinterpret_cast<u32x2*>((tensor ? a.vc : a.kc) + tile);
    float* sdst = (tensor ? a.vs : a.ks) + b * a.num_kv_heads + h;

    u32x4 x[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
        x[c] = PA_Q_NT ? __builtin_nontemporal_load(src + lane + 64 * c) : src[lane + 64 * c];

    // max |x| on fp16 pairs (clearing the sign bits is an exact fabs)
    h2_t m2 = {(_Float16)0.0f, (_Float16)0.0f};
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
#pragma unroll
        for (int w = 0; w < 4; ++w)
            m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(h2_t, word(x[c], w) & 0x7FFF7FFFu));
    const float amax = wave_max(fmaxf((float)m2.x, (float)m2.y));
    const float scale = amax / (FP8 ? 448.0f : 127.0f);
    if (lane == 0) *sdst = scale;
    const float rcp = 1.0f / scale;  // correctly rounded; unused when scale is 0

#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        u32x2 packed = {0u, 0u};
        if (scale != 0.0f) {
            if (FP8) {
                packed.x = pack4_fp8(word(x[c], 0), word(x[c], 1), scale, rcp);
                packed.y = pack4_fp8(word(x[c], 2), word(x[c], 3), scale, rcp);
            } else {
                packed.x = pack4(word(x[c], 0), word(x[c], 1), scale, rcp);
                packed.y = pack4(word(x[c], 2), word(x[c], 3), scale, rcp);
            }
        }
        if (PA_Q_NT)
            __builtin_nontemporal_store(packed, dst + lane + 64 * c);
        else
            dst[lane + 64 * c] = packed;
    }
}

}  // namespace

template <bool FP8>
hipError_t launch_quantize_fmt(const QuantArgs& a, int head_dim, hipStream_t st)
{
    const int64_t tiles = 2 * a.num_ids * a.num_kv_heads;
    if (tiles == 0) return hipSuccess;
    const dim3 grid((unsigned)((tiles + 3) / 4));
    if (head_dim == 64)
        hipLaunchKernelGGL((quantize_kernel<64, FP8>), grid, dim3(256), 0, st, a);
    else if (head_dim == 128)
        hipLaunchKernelGGL((quantize_kernel<128, FP8>), grid, dim3(256), 0, st, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_quantize(const QuantArgs& a, int head_dim, hipStream_t st)
{
    return launch_quantize_fmt<false>(a, head_dim, st);
}

hipError_t launch_quantize_fp8(const QuantArgs& a, int head_dim, hipStream_t st)
{
    return launch_quantize_fmt<true>(a, head_dim, st);
}

}  // namespace pa
