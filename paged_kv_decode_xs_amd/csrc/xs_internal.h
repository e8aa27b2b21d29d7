// Host-side launchers of the libxs kernels. Arguments are validated by the C ABI layer
// (xs_api.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xs {

// One decode launch. k_new/v_new non-null asks for the fused append: the kernel then takes the
// K/V of token L_b - 1 from k_new/v_new and writes them into the pools, exactly as
// launch_kv_append followed by a plain decode would.
struct DecodeArgs {
  const void* q;
  void* k_cache;
  void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const void* k_new;
  const void* v_new;
  float scale;
  void* out;
  float* part_o;
  float* part_m;
  float* part_l;
  int batch, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks;
  int partition_size, max_partitions;
  bool bf16;
  const void* sinks = nullptr;  // bf16 [num_q_heads] sink logits, or null
  int window = 0;               // > 0: attend to the last `window` positions only
};

// What one decode kernel receives (by value, in the kernel argument segment).
struct DecodeParams {
  const uint4* q;
  const uint4* k_cache;
  const uint4* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const uint4* k_new;  // non-null: fused append
  const uint4* v_new;
  uint4* k_cache_w;    // the pools again, for the fused append's writes
  uint4* v_cache_w;
  float scale_log2e;
  void* out;
  float* part_o;
  float* part_m;
  float* part_l;
  int num_q_heads, num_kv_heads, group, chunks, max_blocks_per_seq, num_blocks, part_blocks, max_partitions;
  const uint16_t* sinks;  // bf16 sink logit per query head, or null
  int window;             // 0: all positions
  int batch;
  int ncu;                // compute units of the device (the split grid's work order)
  int dense;              // split grid: 1 = ranked item order (reads every length), 0 = partition-major ids
};

DecodeParams make_params(const DecodeArgs& a, int heads_per_wave);

hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens, int batch,
                            int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                            int num_blocks, int elt_bytes, hipStream_t stream);

// Picks the matrix-core kernel when it supports the shape, else the generic one.
hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream);

hipError_t launch_paged_reduce(const float* part_o, const float* part_m, const float* part_l,
                               const int32_t* context_lens, void* out, int batch, int num_q_heads,
                               int head_dim, int partition_size, int max_partitions, bool bf16,
                               hipStream_t stream);

// The merge with per-head sinks (bf16, or null) and a sliding window (0: none): partitions
// before the window start are skipped and the sink joins the denominator once.
hipError_t launch_paged_reduce_sinks(const float* part_o, const float* part_m, const float* part_l,
                                     const int32_t* context_lens, const void* sinks, int window, void* out,
                                     int batch, int num_q_heads, int head_dim, int partition_size,
                                     int max_partitions, bool bf16, hipStream_t stream);

// Matrix-core variant, for the shapes mfma_decode_supported accepts.
bool mfma_decode_supported(bool bf16, int head_dim, int block_size);
hipError_t launch_paged_decode_mfma(const DecodeArgs& a, hipStream_t stream);

// Heads handled together by one wavefront: the largest of 8, 4, 2, 1 that divides the group size.
int heads_per_chunk(int group);

// Block swap: pair i copies block src_idx[i] of (src_k, src_v) to block dst_idx[i] of (dst_k, dst_v),
// block_bytes each (a multiple of 16); pairs with an index outside [0, n_src) / [0, n_dst) are skipped.
// Host-side pointers must already be the device addresses of pinned host memory.
hipError_t launch_kv_swap(const void* src_k, const void* src_v, void* dst_k, void* dst_v, const int32_t* src_idx,
                          const int32_t* dst_idx, int num_pairs, int n_src, int n_dst, size_t block_bytes,
                          hipStream_t stream);

// Chunked prefill (xs_prefill.hip). The append copies rows i < chunk_lens[b] of k_src/v_src
// [batch, num_kv_heads, chunk, head_dim] to positions start_pos[b] + i.
hipError_t launch_kv_append_chunk(const void* k_src, const void* v_src, void* k_cache, void* v_cache,
                                  const int32_t* block_tables, const int32_t* start_pos, const int32_t* chunk_lens,
                                  int batch, int num_kv_heads, int head_dim, int chunk, int block_size,
                                  int max_blocks_per_seq, int num_blocks, int elt_bytes, hipStream_t stream);

// Causal attention of a chunk of bf16 queries [batch, num_q_heads, chunk, head_dim] over the pool.
struct PrefillArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* start_pos;
  const int32_t* chunk_lens;
  float scale;
  void* out;
  int batch, num_q_heads, num_kv_heads, head_dim, chunk, block_size, max_blocks_per_seq, num_blocks;
  // Split-K over the key range (partition_size 0: none): per-row partials of each piece.
  float* part_o = nullptr;   // [B, Hq, C, max_partitions, D]
  float* part_ml = nullptr;  // [B, Hq, C, max_partitions, 2]
  int partition_size = 0;    // keys per piece, a multiple of 64
  int max_partitions = 0;
  // Sinks and a sliding window (bf16 [Hq] sink logits or null; window 0 = none).
  const void* sinks = nullptr;
  int window = 0;
};
// Row blocks per (sequence, kv head) of the prefill attention: chunk * group rows, 256 per block.
int prefill_row_blocks(int chunk, int group);
hipError_t launch_paged_prefill(const PrefillArgs& a, hipStream_t stream);

// Streaming-read probe over `bytes` (a multiple of 16) of device memory.
hipError_t launch_stream_read(const void* buf, size_t bytes, unsigned* sink, bool nontemporal, int shape,
                              hipStream_t stream);

// Compute units of the current device (cached per device).
int device_cu_count();

}  // namespace xs
