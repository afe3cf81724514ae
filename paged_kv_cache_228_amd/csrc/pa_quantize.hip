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

__device__ __forceinline__ uint32_t code_of(float x, float scale)
{
    float r = rintf(x / scale);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (uint32_t)(int32_t)r & 0xFFu;
}

template <int D>
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
    const uint16_t* src = (tensor ? a.v : a.k) + tile;
    int8_t* dst = (tensor ? a.vc : a.kc) + tile;
    float* sdst = (tensor ? a.vs : a.ks) + b * a.num_kv_heads + h;

    u32x4 x[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) x[c] = reinterpret_cast<const u32x4*>(src)[lane + 64 * c];

    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const h2_t v = __builtin_bit_cast(h2_t, word(x[c], w));
            amax = fmaxf(amax, fmaxf(fabsf((float)v.x), fabsf((float)v.y)));
        }
    amax = wave_max(amax);
    const float scale = amax / 127.0f;
    if (lane == 0) *sdst = scale;

#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        uint32_t packed[2] = {0u, 0u};
        if (scale != 0.0f) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const h2_t v = __builtin_bit_cast(h2_t, word(x[c], w));
                const uint32_t two = code_of((float)v.x, scale) | (code_of((float)v.y, scale) << 8);
                packed[w >> 1] |= two << (16 * (w & 1));
            }
        }
        reinterpret_cast<u32x2*>(dst)[lane + 64 * c] = u32x2{packed[0], packed[1]};
    }
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, int head_dim, hipStream_t st)
{
    const int64_t tiles = 2 * a.num_ids * a.num_kv_heads;
    if (tiles == 0) return hipSuccess;
    const dim3 grid((unsigned)((tiles + 3) / 4));
    if (head_dim == 64)
        hipLaunchKernelGGL(quantize_kernel<64>, grid, dim3(256), 0, st, a);
    else if (head_dim == 128)
        hipLaunchKernelGGL(quantize_kernel<128>, grid, dim3(256), 0, st, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pa
