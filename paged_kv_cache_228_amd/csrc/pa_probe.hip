// HBM read-bandwidth probe, gfx950: the practical ceiling a streaming read
// reaches on the device, measured in the same run as the kernels whose
// roofline it frames. The buffer is cut into chunks of 32 KiB; workgroup w
// takes chunks w, w + G, w + 2G, ... (G workgroups), each as eight 16-byte
// non-temporal loads per lane issued together (256 lanes), and XOR-folds the
// words it read into one 32-bit value written to sink[w], so no load can be
// dropped by the compiler. A second kernel reads and writes (two bytes read
// per byte written, the quantizer's traffic).
#include "pa_internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;
constexpr int64_t kProbeChunk = (int64_t)kProbeThreads * kProbeUnroll;  // 16-byte words per chunk

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(ProbeArgs a)
{
    const int t = threadIdx.x;
    const u32x4* src = static_cast<const u32x4*>(a.src);
    uint32_t acc = 0;
    const int64_t chunks = (a.words + kProbeChunk - 1) / kProbeChunk;
    for (int64_t c = blockIdx.x; c < chunks; c += gridDim.x) {
        const int64_t base = c * kProbeChunk + t;
        u32x4 x[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const int64_t e = base + (int64_t)u * kProbeThreads;
            x[u] = e < a.words ? __builtin_nontemporal_load(src + e) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, d, 64);
    __shared__ uint32_t wacc[kProbeThreads / 64];
    if ((t & 63) == 0) wacc[t >> 6] = acc;
    __syncthreads();
    if (t == 0) {
        uint32_t r = 0;
        for (int i = 0; i < kProbeThreads / 64; ++i) r ^= wacc[i];
        a.sink[blockIdx.x] = r;
    }
}

// The read-and-write variant: the traffic of the INT8 quantizer (two bytes
// read for every byte written). 16-byte word e of the source becomes 8-byte
// word e of the destination, its two halves XORed; same chunks, same
// non-temporal loads, non-temporal 8-byte stores.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(kProbeThreads) void rw_probe_kernel(ProbeArgs a)
{
    const int t = threadIdx.x;
    const u32x4* src = static_cast<const u32x4*>(a.src);
    u32x2* dst = static_cast<u32x2*>(a.dst);
    const int64_t chunks = (a.words + kProbeChunk - 1) / kProbeChunk;
    for (int64_t c = blockIdx.x; c < chunks; c += gridDim.x) {
        const int64_t base = c * kProbeChunk + t;
        u32x4 x[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const int64_t e = base + (int64_t)u * kProbeThreads;
            x[u] = e < a.words ? __builtin_nontemporal_load(src + e) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const int64_t e = base + (int64_t)u * kProbeThreads;
            if (e < a.words) __builtin_nontemporal_store(u32x2{x[u].x ^ x[u].z, x[u].y ^ x[u].w}, dst + e);
        }
    }
}

}  // namespace

hipError_t launch_read_probe(const ProbeArgs& a, int workgroups, hipStream_t st)
{
    if (a.dst)
        hipLaunchKernelGGL(rw_probe_kernel, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, st, a);
    else
        hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace pa
