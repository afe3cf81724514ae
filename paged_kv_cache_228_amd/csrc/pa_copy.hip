// Block copy for copy-on-write, gfx950: block dst_ids[i] of a pool receives
// the bytes of block src_ids[i] (the same or another pool of the same
// layout). One workgroup per pair, 16-byte loads and stores when the block
// size and the pools allow, bytes otherwise; pairs naming a block outside
// [0, num_blocks) are skipped.
#include "pa_internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool WIDE>
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyArgs a)
{
    const int64_t i = blockIdx.x;
    const int64_t s = a.src_ids[i], d = a.dst_ids[i];
    if (s < 0 || s >= a.num_blocks || d < 0 || d >= a.num_blocks) return;
    const char* src = a.src + s * a.bytes_per_block;
    char* dst = a.dst + d * a.bytes_per_block;
    if (WIDE) {
        const int64_t n = a.bytes_per_block / 16;
        for (int64_t e = threadIdx.x; e < n; e += 256)
            reinterpret_cast<u32x4*>(dst)[e] = reinterpret_cast<const u32x4*>(src)[e];
    } else {
        for (int64_t e = threadIdx.x; e < a.bytes_per_block; e += 256) dst[e] = src[e];
    }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t st)
{
    if (a.num_pairs == 0) return hipSuccess;
    const bool wide = a.bytes_per_block % 16 == 0 && (reinterpret_cast<uintptr_t>(a.src) & 15u) == 0 &&
                      (reinterpret_cast<uintptr_t>(a.dst) & 15u) == 0;
    if (wide)
        hipLaunchKernelGGL(copy_blocks_kernel<true>, dim3((unsigned)a.num_pairs), dim3(256), 0, st, a);
    else
        hipLaunchKernelGGL(copy_blocks_kernel<false>, dim3((unsigned)a.num_pairs), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace pa
