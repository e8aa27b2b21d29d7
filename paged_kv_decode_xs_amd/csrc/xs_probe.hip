// Streaming-read probe: the HBM read rate that 16-byte loads reach on this device, the
// reference the decode kernel's bandwidth is compared with. Each workgroup reads whole 64 KiB
// chunks of the buffer (chunks dealt round-robin over the grid, eight loads in flight per thread)
// and folds them into one word; the word reaches memory only if it equals a value no data here
// produces, so the loads cannot be removed. Contiguous chunks with nontemporal loads were the
// fastest of the patterns measured (a grid-stride loop over single pieces reads about 12% slower).
#include "xs_device.h"
#include "xs_internal.h"

namespace xs {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeChunk = 4096;  // 16-byte pieces per chunk (64 KiB): two rounds of 8 loads

template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* __restrict__ buf, size_t n,
                                                                    unsigned* __restrict__ sink) {
  static_assert(kProbeChunk % (8 * kProbeThreads) == 0, "chunk");
  unsigned acc = 0;
  const size_t nchunks = n / kProbeChunk;
  for (size_t ch = blockIdx.x; ch < nchunks; ch += gridDim.x) {
    const uint4* base = buf + ch * kProbeChunk;
    for (int i = threadIdx.x; i < kProbeChunk; i += 8 * kProbeThreads) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = NT ? load_stream(base + i + u * kProbeThreads) : base[i + u * kProbeThreads];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
  // Pieces past the last whole chunk.
  for (size_t i = nchunks * kProbeChunk + (size_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n;
       i += (size_t)gridDim.x * kProbeThreads) {
    const uint4 v = NT ? load_stream(buf + i) : buf[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, unsigned* sink, bool nontemporal, hipStream_t stream) {
  const size_t n = bytes / 16;
  const unsigned grid = 16u * (unsigned)device_cu_count();
  if (nontemporal)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3(grid), dim3(kProbeThreads), 0, stream,
                       static_cast<const uint4*>(buf), n, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3(grid), dim3(kProbeThreads), 0, stream,
                       static_cast<const uint4*>(buf), n, sink);
  return hipGetLastError();
}

}  // namespace xs
