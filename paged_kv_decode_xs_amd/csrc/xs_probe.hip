// Streaming-read probe: the HBM read rate that 16-byte loads reach on this device, the
// reference the decode kernel's bandwidth is compared with. Workgroups take chunks of the buffer in
// turn (chunk c goes to workgroup c mod grid), so at any moment the GPU reads one window of the
// buffer that moves through it in address order. Two shapes, the fastest of a sweep on MI355X (one
// to 32 workgroups per CU, 4 KiB to 256 KiB chunks, one to 16 loads in flight, plain and
// nontemporal loads, and one contiguous stream per wavefront instead):
//   shape 0 ("wide"):   16 workgroups of 256 threads per CU, 256 KiB chunks, 8 loads in flight;
//   shape 1 ("narrow"):  2 workgroups per CU, 16 KiB chunks, 4 loads in flight.
// The narrow shape was the fastest in the sweep, at about 7.3 TB/s with nontemporal loads, but
// varies with the buffer's placement (6.5-7.3 TB/s across processes). The wide one held 7.1 TB/s.
// A caller takes the faster of the two. Each thread folds its data into one word, which reaches
// memory only if it equals a value no data here produces, so the loads cannot be removed.
#include "xs_device.h"
#include "xs_internal.h"

namespace xs {
namespace {

constexpr int kProbeThreads = 256;

// CHUNK: 16-byte pieces per chunk, U: loads in flight per thread (CHUNK / (U * 256) rounds).
template <bool NT, int CHUNK, int U>
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* __restrict__ buf, size_t n,
                                                                    unsigned* __restrict__ sink) {
  static_assert(CHUNK % (U * kProbeThreads) == 0, "whole rounds of loads per chunk");
  unsigned acc = 0;
  const size_t nchunks = n / CHUNK;
  for (size_t ch = blockIdx.x; ch < nchunks; ch += gridDim.x) {
    const uint4* base = buf + ch * CHUNK + threadIdx.x;
    for (int i = 0; i < CHUNK; i += U * kProbeThreads) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = NT ? load_stream(base + i + u * kProbeThreads) : base[i + u * kProbeThreads];
#pragma unroll
      for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
  // Pieces past the last whole chunk.
  for (size_t i = nchunks * CHUNK + (size_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n;
       i += (size_t)gridDim.x * kProbeThreads) {
    const uint4 v = NT ? load_stream(buf + i) : buf[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

template <int CHUNK, int U>
void launch_shape(const uint4* buf, size_t n, unsigned* sink, bool nontemporal, unsigned grid, hipStream_t stream) {
  if (nontemporal)
    hipLaunchKernelGGL((stream_read_kernel<true, CHUNK, U>), dim3(grid), dim3(kProbeThreads), 0, stream, buf, n, sink);
  else
    hipLaunchKernelGGL((stream_read_kernel<false, CHUNK, U>), dim3(grid), dim3(kProbeThreads), 0, stream, buf, n, sink);
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, unsigned* sink, bool nontemporal, int shape,
                              hipStream_t stream) {
  const size_t n = bytes / 16;
  const unsigned cus = (unsigned)device_cu_count();
  const uint4* b = static_cast<const uint4*>(buf);
  if (shape == 1)
    launch_shape<1024, 4>(b, n, sink, nontemporal, 2u * cus, stream);
  else
    launch_shape<16384, 8>(b, n, sink, nontemporal, 16u * cus, stream);
  return hipGetLastError();
}

}  // namespace xs
