// Host-side launchers of the libxs kernels. Arguments are validated by the C ABI layer
// (xs_api.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xs {

hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens, int batch,
                            int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                            int num_blocks, int elt_bytes, hipStream_t stream);

// Returns hipErrorInvalidValue for a shape without a compiled kernel (checked beforehand by the caller).
hipError_t launch_paged_decode(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens, float scale,
                               void* out, float* part_o, float* part_m, float* part_l, int batch,
                               int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                               int max_blocks_per_seq, int num_blocks, int partition_size,
                               int max_partitions, bool bf16, hipStream_t stream);

hipError_t launch_paged_reduce(const float* part_o, const float* part_m, const float* part_l,
                               const int32_t* context_lens, void* out, int batch, int num_q_heads,
                               int head_dim, int partition_size, int max_partitions, bool bf16,
                               hipStream_t stream);

// Matrix-core variant of launch_paged_decode, for the shapes mfma_decode_supported accepts.
bool mfma_decode_supported(bool bf16, int head_dim, int block_size);
hipError_t launch_paged_decode_mfma(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables, const int32_t* context_lens, float scale, void* out,
                                    float* part_o, float* part_m, float* part_l, int batch, int num_q_heads,
                                    int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                                    int num_blocks, int partition_size, int max_partitions, hipStream_t stream);

// Heads handled together by one wavefront: the largest of 8, 4, 2, 1 that divides the group size.
int heads_per_chunk(int group);

}  // namespace xs
