// Decode-step KV append: one new K/V row per sequence into its paged slot.
//
// xserv compare phase10...cf1e9e41, crates/xserv-kernels/src/attention.rs: the batched
// scatter reads the same block table as the attention kernel, and kv_lens = current length
// + 1, so the new token goes to position kv_lens - 1. Each thread moves one 16-byte piece
// of one row: a bit-exact copy with no arithmetic on the values.
#include "xs_internal.h"

namespace xs {
namespace {

__global__ __launch_bounds__(256) void kv_append_kernel(const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
                                                        uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                                                        const int32_t* __restrict__ block_tables,
                                                        const int32_t* __restrict__ context_lens, int batch,
                                                        int num_kv_heads, int pieces_per_row, int block_size,
                                                        int max_blocks_per_seq, int num_blocks) {
  const long long per_seq = (long long)num_kv_heads * pieces_per_row;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= 2 * (long long)batch * per_seq) return;
  const bool is_v = idx >= (long long)batch * per_seq;
  const long long r = is_v ? idx - (long long)batch * per_seq : idx;
  const int b = (int)(r / per_seq);
  const int g = (int)((r % per_seq) / pieces_per_row);
  const int piece = (int)(r % pieces_per_row);
  const int L = context_lens[b];
  if (L < 1 || L > max_blocks_per_seq * block_size) return;
  const int pos = L - 1;
  const int blk = block_tables[(long long)b * max_blocks_per_seq + pos / block_size];
  if (blk < 0 || blk >= num_blocks) return;
  const long long dst = (((long long)blk * num_kv_heads + g) * block_size + pos % block_size) * pieces_per_row + piece;
  const long long src = ((long long)b * num_kv_heads + g) * pieces_per_row + piece;
  if (is_v)
    v_cache[dst] = v_new[src];
  else
    k_cache[dst] = k_new[src];
}

}  // namespace

hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens, int batch,
                            int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                            int num_blocks, int elt_bytes, hipStream_t stream) {
  const int pieces_per_row = head_dim * elt_bytes / 16;
  const long long total = 2LL * batch * num_kv_heads * pieces_per_row;
  const int threads = 256;
  const long long blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new), static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), block_tables, context_lens, batch, num_kv_heads, pieces_per_row,
                     block_size, max_blocks_per_seq, num_blocks);
  return hipGetLastError();
}

}  // namespace xs
