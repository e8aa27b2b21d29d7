// Log-sum-exp merge of split-K partitions: one workgroup per (sequence, query head).
//
// Partition j holds (o_j, m_j, l_j) with m_j the max scaled score, l_j = sum exp(s - m_j) and
// o_j the partition's normalised output. With M = max_j m_j and w_j = l_j exp(m_j - M),
//   out = sum_j w_j o_j / sum_j w_j,
// which equals the softmax over the whole context (the partitions split its sum). The split
// and its merge are this library's design for long contexts; the pages have no split.
//
// The merge is a chain of dependent memory round trips (the length, then the partials), so the
// kernel is built to need as few as it can: every partial of a row is requested in one round.
// A row of D floats is read by D/4 lanes (16 bytes each), so a wavefront holds S = 256/D rows
// ("slots") per load; NW wavefronts of a workgroup hold 8 loads each in flight, i.e. 8 * S * NW
// partitions per round (64 for D = 128 and NW = 4). Each slot folds its partitions into a running
// (m, l, o) with the same rule, o kept normalised:
//   m' = max(m, m_j),  a = l e^(m-m'),  c = l_j e^(m_j-m'),  l' = a + c,  o' = (a o + c o_j) / l',
// then the slots and the wavefronts fold their states together (shuffles, then LDS). Without a
// window the first round's loads go out before the length arrives (they stay inside the row's
// max_partitions slots; those past the row's partition count are discarded, never multiplied).
#include <math.h>

#include "xs_device.h"
#include "xs_internal.h"

namespace xs {
namespace {

constexpr int kRedU = 8;  // loads in flight per lane and round

struct LseState {
  float m, l;
  float4 o;
};

__device__ __forceinline__ void lse_fold(LseState& s, float m2, float l2, const float4& o2) {
  const float mn = fmaxf(s.m, m2);
  const float ms = mn == -INFINITY ? 0.f : mn;
  const float a = s.m == -INFINITY ? 0.f : fast_exp2((s.m - ms) * kLog2e) * s.l;
  const float c = m2 == -INFINITY ? 0.f : fast_exp2((m2 - ms) * kLog2e) * l2;
  const float ln = a + c;
  const float inv = ln > 0.f ? 1.f / ln : 0.f;
  s.o.x = (s.o.x * a + o2.x * c) * inv;
  s.o.y = (s.o.y * a + o2.y * c) * inv;
  s.o.z = (s.o.z * a + o2.z * c) * inv;
  s.o.w = (s.o.w * a + o2.w * c) * inv;
  s.m = mn;
  s.l = ln;
}

// One round: the slot's partitions j = base + k * stride, k < kRedU, folded in if j0 <= j < n.
template <int D>
__device__ __forceinline__ void fold_round(LseState& st, const float* pm, const float* pl, const float4* po, int base,
                                           int stride, int j0, int n, int maxp) {
  constexpr int LPR = D / 4;
  float4 o[kRedU];
  float m[kRedU], l[kRedU];
#pragma unroll
  for (int k = 0; k < kRedU; ++k) {  // every load inside the row's max_partitions slots
    const int j = min(base + k * stride, maxp - 1);
    o[k] = po[(size_t)j * LPR];
    m[k] = pm[j];
    l[k] = pl[j];
  }
#pragma unroll
  for (int k = 0; k < kRedU; ++k) {
    const int j = base + k * stride;
    if (j >= j0 && j < n) lse_fold(st, m[k], l[k], o[k]);
  }
}

// SW: per-head sinks and a sliding window (xserv compare phase10...cf1e9e41, attention.rs,
// `paged_decode_attention_sinks`): partitions before the window start t0 = max(0, L - window)
// hold no kept position and were never written; head h's sink sigma joins the denominator once:
//   M = max(sigma, max_j m_j),  out = sum_j l_j e^(m_j - M) o_j / (e^(sigma - M) + sum_j l_j e^(m_j - M)).
template <bool BF16, int D, int NW, bool SW>
__global__ __launch_bounds__(64 * NW) void paged_reduce_kernel(const float* __restrict__ part_o,
                                                               const float* __restrict__ part_m,
                                                               const float* __restrict__ part_l,
                                                               const int32_t* __restrict__ context_lens,
                                                               const uint16_t* __restrict__ sinks, int window,
                                                               void* __restrict__ out, int num_q_heads,
                                                               int partition_size, int max_partitions) {
  constexpr int LPR = D / 4;   // lanes per partial row
  constexpr int S = 64 / LPR;  // slots per wavefront
  __shared__ __align__(16) float lds[(NW > 1 ? NW - 1 : 1) * (2 + 4) * LPR];
  const int wave = NW > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
  const int lane = threadIdx.x & 63;
  const int slot = lane / LPR, c = lane % LPR;
  const size_t row = blockIdx.x;  // (b, h)
  const int b = (int)(row / num_q_heads);
  const int maxp = max_partitions;
  const float* pm = part_m + row * maxp;
  const float* pl = part_l + row * maxp;
  const float4* po = reinterpret_cast<const float4*>(part_o + row * maxp * D) + c;
  const int stride = S * NW;           // between a slot's consecutive partitions
  const int first = wave * S + slot;   // the slot's first partition
  const int per_round = stride * kRedU;

  LseState st{-INFINITY, 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
  const int L = context_lens[b];
  const int n_all = L > 0 ? (L + partition_size - 1) / partition_size : 0;
  const bool overflow = n_all > maxp;  // partitions were cut: the output is NaN
  const int n = min(n_all, maxp);
  int j0 = 0;
  if constexpr (SW) {
    j0 = (L > 0 && window > 0 ? max(0, L - window) : 0) / partition_size;
    for (int base = j0 - j0 % per_round + first; base - first < n; base += per_round)
      fold_round<D>(st, pm, pl, po, base, stride, j0, n, maxp);
  } else {
    // Round 0 is issued with the length load (before n is known).
    fold_round<D>(st, pm, pl, po, first, stride, 0, n, maxp);
    for (int base = first + per_round; base - first < n; base += per_round)
      fold_round<D>(st, pm, pl, po, base, stride, 0, n, maxp);
  }
  // Fold the slots of the wavefront, then the wavefronts.
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
    const float4 o2 = make_float4(__shfl_xor(st.o.x, off, 64), __shfl_xor(st.o.y, off, 64),
                                  __shfl_xor(st.o.z, off, 64), __shfl_xor(st.o.w, off, 64));
    lse_fold(st, __shfl_xor(st.m, off, 64), __shfl_xor(st.l, off, 64), o2);
  }
  if constexpr (NW > 1) {
    if (wave > 0 && slot == 0) {
      float* mine = lds + (wave - 1) * 6 * LPR;
      mine[c] = st.m;
      mine[LPR + c] = st.l;
      reinterpret_cast<float4*>(mine + 2 * LPR)[c] = st.o;
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      const float* other = lds + (w - 1) * 6 * LPR;
      lse_fold(st, other[c], other[LPR + c], reinterpret_cast<const float4*>(other + 2 * LPR)[c]);
    }
  }
  float f = 1.f;
  if (SW && sinks && n > j0) {
    const float sg = __uint_as_float((uint32_t)sinks[row % num_q_heads] << 16);
    const float M = fmaxf(st.m, sg);
    const float a = st.m == -INFINITY ? 0.f : fast_exp2((st.m - M) * kLog2e) * st.l;
    const float den = a + (sg == -INFINITY ? 0.f : fast_exp2((sg - M) * kLog2e));
    f = den > 0.f ? a / den : 0.f;
  }
  if (overflow) f = NAN;
  if (slot != 0) return;
  const float4 v = make_float4(st.o.x * f, st.o.y * f, st.o.z * f, st.o.w * f);
  if constexpr (BF16) {
    reinterpret_cast<uint2*>(out)[row * LPR + c] = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
  } else {
    reinterpret_cast<float4*>(out)[row * LPR + c] = v;
  }
}

// Wavefronts per row: enough that one round covers max_partitions, at most 4.
int reduce_waves(int head_dim, int max_partitions) {
  const int per_wave = kRedU * (256 / head_dim);
  return max_partitions <= per_wave ? 1 : max_partitions <= 2 * per_wave ? 2 : 4;
}

template <bool BF16, int D, bool SW>
hipError_t launch_rows(const float* part_o, const float* part_m, const float* part_l, const int32_t* context_lens,
                       const void* sinks, int window, void* out, int batch, int num_q_heads, int partition_size,
                       int max_partitions, hipStream_t stream) {
  const dim3 grid((unsigned)((long long)batch * num_q_heads));
  const uint16_t* sk = static_cast<const uint16_t*>(sinks);
  switch (reduce_waves(D, max_partitions)) {
    case 1:
      hipLaunchKernelGGL((paged_reduce_kernel<BF16, D, 1, SW>), grid, dim3(64), 0, stream, part_o, part_m, part_l,
                         context_lens, sk, window, out, num_q_heads, partition_size, max_partitions);
      break;
    case 2:
      hipLaunchKernelGGL((paged_reduce_kernel<BF16, D, 2, SW>), grid, dim3(128), 0, stream, part_o, part_m, part_l,
                         context_lens, sk, window, out, num_q_heads, partition_size, max_partitions);
      break;
    default:
      hipLaunchKernelGGL((paged_reduce_kernel<BF16, D, 4, SW>), grid, dim3(256), 0, stream, part_o, part_m, part_l,
                         context_lens, sk, window, out, num_q_heads, partition_size, max_partitions);
      break;
  }
  return hipGetLastError();
}

template <bool SW>
hipError_t launch_any(const float* part_o, const float* part_m, const float* part_l, const int32_t* context_lens,
                      const void* sinks, int window, void* out, int batch, int num_q_heads, int head_dim,
                      int partition_size, int max_partitions, bool bf16, hipStream_t stream) {
  if (bf16 && head_dim == 64)
    return launch_rows<true, 64, SW>(part_o, part_m, part_l, context_lens, sinks, window, out, batch, num_q_heads,
                                     partition_size, max_partitions, stream);
  if (bf16 && head_dim == 128)
    return launch_rows<true, 128, SW>(part_o, part_m, part_l, context_lens, sinks, window, out, batch, num_q_heads,
                                      partition_size, max_partitions, stream);
  if (!bf16 && head_dim == 64)
    return launch_rows<false, 64, SW>(part_o, part_m, part_l, context_lens, sinks, window, out, batch, num_q_heads,
                                      partition_size, max_partitions, stream);
  if (!bf16 && head_dim == 128)
    return launch_rows<false, 128, SW>(part_o, part_m, part_l, context_lens, sinks, window, out, batch, num_q_heads,
                                       partition_size, max_partitions, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_paged_reduce(const float* part_o, const float* part_m, const float* part_l,
                               const int32_t* context_lens, void* out, int batch, int num_q_heads, int head_dim,
                               int partition_size, int max_partitions, bool bf16, hipStream_t stream) {
  return launch_any<false>(part_o, part_m, part_l, context_lens, nullptr, 0, out, batch, num_q_heads, head_dim,
                           partition_size, max_partitions, bf16, stream);
}

hipError_t launch_paged_reduce_sinks(const float* part_o, const float* part_m, const float* part_l,
                                     const int32_t* context_lens, const void* sinks, int window, void* out,
                                     int batch, int num_q_heads, int head_dim, int partition_size,
                                     int max_partitions, bool bf16, hipStream_t stream) {
  return launch_any<true>(part_o, part_m, part_l, context_lens, sinks, window, out, batch, num_q_heads, head_dim,
                          partition_size, max_partitions, bf16, stream);
}

}  // namespace xs
