// Internal interface between the C-ABI front end (pa_api.cpp) and the HIP
// kernels (pa_decode.hip, pa_quantize.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlockTokens = 16;   // tokens per physical KV block
constexpr int kWaves = 4;          // waves per decode workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxPartitionBlocks = kThreads;  // one staged block id per thread
constexpr int kMaxGroup = 8;       // query heads per KV head

struct DecodeArgs {
    const void* q;          // fp16 [S][Hq][D]
    const void* k;          // fp16 or int8 pool [NB][Hkv][16][D]
    const void* v;
    const float* k_scale;   // INT8 only: [NB][Hkv]
    const float* v_scale;
    const int32_t* tables;  // [S][max_blocks]
    const int32_t* ctx;     // [S]
    float* out;             // fp32 [S][Hq][D]
    float* ws;              // split-K partials, see pa_api.cpp for the layout
    int64_t num_blocks;
    int num_seqs;
    int num_q_heads;
    int num_kv_heads;
    int max_blocks;         // table row length
    int part_blocks;        // blocks per context partition (<= kMaxPartitionBlocks)
    int max_parts;          // partitions of the longest possible context
    float scale_log2;       // softmax_scale * log2(e)
};

// Workspace layout (floats): acc [S][Hq][P][D], then m [S][Hq][P], then l [S][Hq][P].
inline size_t workspace_floats(int S, int Hq, int P, int D)
{
    return (size_t)S * Hq * P * (size_t)(D + 2);
}

// Partition kernel + (when max_parts > 1) the split-K merge kernel.
hipError_t launch_decode(const DecodeArgs& a, int head_dim, int group, bool int8, hipStream_t st);
hipError_t launch_decode_partitions_mfma(const DecodeArgs& a, int head_dim, int group, bool int8,
                                         hipStream_t st);
hipError_t launch_decode_partitions_valu(const DecodeArgs& a, int head_dim, int group, bool int8,
                                         hipStream_t st);
hipError_t launch_decode_merge(const DecodeArgs& a, int head_dim, hipStream_t st);

struct QuantArgs {
    const uint16_t* k;
    const uint16_t* v;
    int8_t* kc;
    int8_t* vc;
    float* ks;
    float* vs;
    const int32_t* ids;     // NULL = all blocks
    int64_t num_ids;        // tiles per tensor = num_ids * num_kv_heads
    int64_t num_blocks;
    int num_kv_heads;
};

hipError_t launch_quantize(const QuantArgs& a, int head_dim, hipStream_t st);

}  // namespace pa
