// Log-sum-exp merge of split-K partitions: one wavefront per (sequence, query head).
//
// Partition j holds (o_j, m_j, l_j) with m_j the max scaled score, l_j = sum exp(s - m_j) and
// o_j the partition's normalised output. With M = max_j m_j and w_j = l_j exp(m_j - M),
//   out = sum_j w_j o_j / sum_j w_j,
// which equals the softmax over the whole context (the partitions split its sum). The split
// and its merge are this library's design for long contexts; the pages have no split.
#include <math.h>

#include "xs_device.h"
#include "xs_internal.h"

namespace xs {
namespace {

template <bool BF16, int D>
__global__ __launch_bounds__(64) void paged_reduce_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_m,
                                                          const float* __restrict__ part_l,
                                                          const int32_t* __restrict__ context_lens,
                                                          void* __restrict__ out, int num_q_heads,
                                                          int partition_size, int max_partitions) {
  constexpr int DPL = D / 64;  // output elements per lane
  constexpr int PRE = 8;       // partitions whose o is fetched before the count is known
  const int lane = threadIdx.x;
  const size_t row = blockIdx.x;  // (b, h)
  const int b = (int)(row / num_q_heads);
  const float* pm = part_m + row * max_partitions;
  const float* pl = part_l + row * max_partitions;
  const float* po = part_o + row * max_partitions * D + (size_t)lane * DPL;

  // Loads that do not depend on L go out together with it: (m, l) of the first 64 slots and o of
  // the first PRE slots, all inside this row's max_partitions slots. Slots at or past the
  // partition count n are ignored below.
  const int L = context_lens[b];
  float mj = lane < max_partitions ? pm[lane] : -INFINITY;
  float lj = lane < max_partitions ? pl[lane] : 0.f;
  float opre[PRE][DPL];
#pragma unroll
  for (int u = 0; u < PRE; ++u) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) opre[u][e] = u < max_partitions ? po[(size_t)u * D + e] : 0.f;
  }
  int n = L > 0 ? (L + partition_size - 1) / partition_size : 0;
  n = min(n, max_partitions);
  if (lane >= n) {
    mj = -INFINITY;
    lj = 0.f;
  }

  float M = mj;
  for (int j = lane + 64; j < n; j += 64) M = fmaxf(M, pm[j]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));

  float acc[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
  float W = 0.f;
  if (M != -INFINITY) {
    const float M2 = M * kLog2e;
    for (int base = 0; base < n; base += 64) {
      const int jj = base + lane;
      float w = 0.f;
      if (jj < n) w = base == 0 ? lj * fast_exp2(fmaf(mj, kLog2e, -M2)) : pl[jj] * fast_exp2(fmaf(pm[jj], kLog2e, -M2));
      W += w;
      const int cnt = min(64, n - base);
      int k = 0;
      if (base == 0) {
#pragma unroll
        for (int u = 0; u < PRE; ++u) {
          if (u < cnt) {
            const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u));
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[e] = fmaf(wk, opre[u][e], acc[e]);
          }
        }
        k = PRE;
      }
      // Eight partitions per round so that their loads are in flight together.
      for (; k + 8 <= cnt; k += 8) {
        float o[8][DPL];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
#pragma unroll
          for (int e = 0; e < DPL; ++e) o[u][e] = po[(size_t)(base + k + u) * D + e];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k + u));
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[e] = fmaf(wk, o[u][e], acc[e]);
        }
      }
      for (; k < cnt; ++k) {
        const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] = fmaf(wk, po[(size_t)(base + k) * D + e], acc[e]);
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) W += __shfl_xor(W, off, 64);
  const float inv = W > 0.f ? 1.f / W : 0.f;
  if constexpr (BF16) {
    if constexpr (DPL == 2) {
      reinterpret_cast<uint32_t*>(out)[row * (D / 2) + lane] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    } else {
      reinterpret_cast<uint16_t*>(out)[row * D + lane] = (uint16_t)f32_to_bf16_rne(acc[0] * inv);
    }
  } else {
    float* o = reinterpret_cast<float*>(out) + row * D + (size_t)lane * DPL;
#pragma unroll
    for (int k = 0; k < DPL; ++k) o[k] = acc[k] * inv;
  }
}


// The merge with attention sinks and a sliding window (xserv compare phase10...cf1e9e41,
// attention.rs, `paged_decode_attention_sinks`). The window keeps positions from
// t0 = max(0, L - window); partitions j < t0 / P hold none of them and were never written.
// Head h's sink sigma joins the denominator once:
//   M = max(sigma, max_j m_j),  out = sum_j l_j e^(m_j - M) o_j / (e^(sigma - M) + sum_j l_j e^(m_j - M)).
template <bool BF16, int D>
__global__ __launch_bounds__(64) void paged_reduce_sinks_kernel(const float* __restrict__ part_o,
                                                                const float* __restrict__ part_m,
                                                                const float* __restrict__ part_l,
                                                                const int32_t* __restrict__ context_lens,
                                                                const uint16_t* __restrict__ sinks, int window,
                                                                void* __restrict__ out, int num_q_heads,
                                                                int partition_size, int max_partitions) {
  constexpr int DPL = D / 64;  // output elements per lane
  const int lane = threadIdx.x;
  const size_t row = blockIdx.x;  // (b, h)
  const int b = (int)(row / num_q_heads);
  const int h = (int)(row % num_q_heads);
  const float* pm = part_m + row * max_partitions;
  const float* pl = part_l + row * max_partitions;
  const float* po = part_o + row * max_partitions * D + (size_t)lane * DPL;

  const int L = context_lens[b];
  const int t0 = window > 0 ? max(0, L - window) : 0;
  const int j0 = L > 0 ? t0 / partition_size : 0;
  const int n = L > 0 ? min((L + partition_size - 1) / partition_size, max_partitions) : 0;
  const float sig = sinks ? __uint_as_float((uint32_t)sinks[h] << 16) : -INFINITY;

  float M = -INFINITY;
  for (int j = j0 + lane; j < n; j += 64) M = fmaxf(M, pm[j]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  M = fmaxf(M, sig);

  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  float W = 0.f;
  if (n > j0 && M != -INFINITY) {
    const float M2 = M * kLog2e;
    for (int base = j0; base < n; base += 64) {
      const int jj = base + lane;
      const float w = jj < n ? pl[jj] * fast_exp2(fmaf(pm[jj], kLog2e, -M2)) : 0.f;
      W += w;
      const int cnt = min(64, n - base);
      int k = 0;
      for (; k + 8 <= cnt; k += 8) {  // eight partitions' o in flight together
        float o[8][DPL];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
#pragma unroll
          for (int e = 0; e < DPL; ++e) o[u][e] = po[(size_t)(base + k + u) * D + e];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k + u));
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[e] = fmaf(wk, o[u][e], acc[e]);
        }
      }
      for (; k < cnt; ++k) {
        const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] = fmaf(wk, po[(size_t)(base + k) * D + e], acc[e]);
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) W += __shfl_xor(W, off, 64);
  if (n > j0 && sig != -INFINITY) W += fast_exp2((sig - M) * kLog2e);
  const float inv = W > 0.f ? 1.f / W : 0.f;
  if constexpr (BF16) {
    if constexpr (DPL == 2) {
      reinterpret_cast<uint32_t*>(out)[row * (D / 2) + lane] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    } else {
      reinterpret_cast<uint16_t*>(out)[row * D + lane] = (uint16_t)f32_to_bf16_rne(acc[0] * inv);
    }
  } else {
    float* o = reinterpret_cast<float*>(out) + row * D + (size_t)lane * DPL;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] = acc[e] * inv;
  }
}

}  // namespace

hipError_t launch_paged_reduce(const float* part_o, const float* part_m, const float* part_l,
                               const int32_t* context_lens, void* out, int batch, int num_q_heads, int head_dim,
                               int partition_size, int max_partitions, bool bf16, hipStream_t stream) {
  const dim3 grid((unsigned)((long long)batch * num_q_heads));
#define XS_LAUNCH(BF, D_)                                                                                      \
  hipLaunchKernelGGL((paged_reduce_kernel<BF, D_>), grid, dim3(64), 0, stream, part_o, part_m, part_l,       \
                     context_lens, out, num_q_heads, partition_size, max_partitions)
  if (bf16) {
    if (head_dim == 64) XS_LAUNCH(true, 64);
    else if (head_dim == 128) XS_LAUNCH(true, 128);
    else return hipErrorInvalidValue;
  } else {
    if (head_dim == 64) XS_LAUNCH(false, 64);
    else if (head_dim == 128) XS_LAUNCH(false, 128);
    else return hipErrorInvalidValue;
  }
#undef XS_LAUNCH
  return hipGetLastError();
}

hipError_t launch_paged_reduce_sinks(const float* part_o, const float* part_m, const float* part_l,
                                     const int32_t* context_lens, const void* sinks, int window, void* out,
                                     int batch, int num_q_heads, int head_dim, int partition_size,
                                     int max_partitions, bool bf16, hipStream_t stream) {
  const dim3 grid((unsigned)((long long)batch * num_q_heads));
  const uint16_t* sk = static_cast<const uint16_t*>(sinks);
#define XS_LAUNCH(BF, D_)                                                                                        \
  hipLaunchKernelGGL((paged_reduce_sinks_kernel<BF, D_>), grid, dim3(64), 0, stream, part_o, part_m, part_l,    \
                     context_lens, sk, window, out, num_q_heads, partition_size, max_partitions)
  if (bf16) {
    if (head_dim == 64) XS_LAUNCH(true, 64);
    else if (head_dim == 128) XS_LAUNCH(true, 128);
    else return hipErrorInvalidValue;
  } else {
    if (head_dim == 64) XS_LAUNCH(false, 64);
    else if (head_dim == 128) XS_LAUNCH(false, 128);
    else return hipErrorInvalidValue;
  }
#undef XS_LAUNCH
  return hipGetLastError();
}

}  // namespace xs
