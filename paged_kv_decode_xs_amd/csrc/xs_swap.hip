// KV block swap between the paged pools (device memory) and a swap space in pinned host memory.
//
// The xserv README (xserv compare phase10...cf1e9e41) lists CPU swap-out / swap-in of the paged
// KV cache into pinned host memory (`--swap-space-gb`). Here one launch moves a whole list of
// blocks: pair i copies block src[i] of the source (K and V, all kv heads) to block dst[i] of the
// destination. The GPU itself reads or writes the host memory over the host link, so a list of
// scattered 32 KB blocks costs one launch instead of two copy commands per block.
#include "xs_internal.h"

namespace xs {
namespace {

constexpr int kSwapThreads = 256;
constexpr int kSwapUnroll = 8;  // 16-byte loads in flight per thread (host reads are slow to return)

__global__ __launch_bounds__(kSwapThreads) void kv_swap_kernel(const uint4* __restrict__ src_k,
                                                               const uint4* __restrict__ src_v,
                                                               uint4* __restrict__ dst_k, uint4* __restrict__ dst_v,
                                                               const int32_t* __restrict__ src_idx,
                                                               const int32_t* __restrict__ dst_idx, int n_src,
                                                               int n_dst, int pieces) {
  const int s = src_idx[blockIdx.x];
  const int d = dst_idx[blockIdx.x];
  if (s < 0 || s >= n_src || d < 0 || d >= n_dst) return;  // out-of-range pairs are skipped
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const uint4* src = (kv == 0 ? src_k : src_v) + (size_t)s * pieces;
    uint4* dst = (kv == 0 ? dst_k : dst_v) + (size_t)d * pieces;
    for (int base = threadIdx.x; base < pieces; base += kSwapThreads * kSwapUnroll) {
      uint4 r[kSwapUnroll];
#pragma unroll
      for (int u = 0; u < kSwapUnroll; ++u) {
        const int e = base + u * kSwapThreads;
        if (e < pieces) r[u] = src[e];
      }
#pragma unroll
      for (int u = 0; u < kSwapUnroll; ++u) {
        const int e = base + u * kSwapThreads;
        if (e < pieces) dst[e] = r[u];
      }
    }
  }
}

}  // namespace

hipError_t launch_kv_swap(const void* src_k, const void* src_v, void* dst_k, void* dst_v, const int32_t* src_idx,
                          const int32_t* dst_idx, int num_pairs, int n_src, int n_dst, size_t block_bytes,
                          hipStream_t stream) {
  hipLaunchKernelGGL(kv_swap_kernel, dim3((unsigned)num_pairs), dim3(kSwapThreads), 0, stream,
                     static_cast<const uint4*>(src_k), static_cast<const uint4*>(src_v), static_cast<uint4*>(dst_k),
                     static_cast<uint4*>(dst_v), src_idx, dst_idx, n_src, n_dst, (int)(block_bytes / 16));
  return hipGetLastError();
}

}  // namespace xs
