// Paged decode attention: one wavefront per (sequence, kv head, head chunk, partition).
//
// What is computed (xserv compare phase10...cf1e9e41, crates/xserv-kernels/src/attention.rs,
// `paged_decode_attention`; GQA from xserv compare phase8...phase13, `repeat_kv`): for the
// query heads h of kv head g, over tokens t of the work item's block range,
//   s_t = scale * q_h . K_t,   m = max s_t,   l = sum exp(s_t - m),   o = sum exp(s_t - m) V_t / l.
// No split: o is the output. Split-K: (o, m, l) are the partition's partials, merged later by
// the log-sum-exp reduce.
//
// Data flow, for one (block, kv head) chunk of BS x D contiguous elements:
//   - each load instruction moves 64 lanes x 16 bytes = 1 KiB of consecutive token rows, so
//     lane l holds token row (i*TPI + l/LPT), elements (l%LPT)*EPL .. +EPL of it;
//   - QK: each lane dots its EPL elements with the matching slice of the GC query rows
//     (v_dot2_f32_bf16 for bf16, fp32 FMA for fp32), then the LPT lanes of a token row sum
//     by DPP (row mirrors and quad permutes), so every lane of the row holds the row's scores;
//   - softmax and PV are row-local: each group of LPT lanes keeps its own running max, sum and
//     fp32 accumulator over the tokens it saw (online softmax, exp2 of log2e-scaled scores);
//   - at the end the TPI row states merge by the same max/rescale rule through lane shuffles.
// Tokens at or past L (the tail of the last block) get score -inf and a zeroed V, so whatever
// the pool holds there (NaN included) never reaches the result.
// The block ids of up to 64 blocks sit in one VGPR (one per lane) and are read by v_readlane.
// The next block's K and V are loaded while the current block is processed.
#include <math.h>

#include "xs_device.h"
#include "xs_internal.h"

namespace xs {
namespace {

template <bool BF16, int D, int BS>
struct Geo {
  static constexpr int kEltBytes = BF16 ? 2 : 4;
  static constexpr int kEPL = 16 / kEltBytes;  // elements per lane per 16-byte load
  static constexpr int kLPT = D / kEPL;        // lanes per token row
  static constexpr int kTPI = 64 / kLPT;       // token rows per load instruction
  static constexpr int kNI = BS / kTPI;        // load instructions per (block, kv head) chunk
  static_assert(kLPT * kEPL == D, "head_dim must fill whole 16-byte pieces");
  static_assert(kTPI * kLPT == 64, "a token row must divide the wavefront");
  static_assert(kNI * kTPI == BS, "block_size must be a multiple of the rows per load");
};

// Unpack one 16-byte piece into EPL fp32 values.
template <bool BF16>
__device__ __forceinline__ void unpack(const uint4& w, float* f) {
  if constexpr (BF16) {
    f[0] = bf16lo_to_f32(w.x); f[1] = bf16hi_to_f32(w.x);
    f[2] = bf16lo_to_f32(w.y); f[3] = bf16hi_to_f32(w.y);
    f[4] = bf16lo_to_f32(w.z); f[5] = bf16hi_to_f32(w.z);
    f[6] = bf16lo_to_f32(w.w); f[7] = bf16hi_to_f32(w.w);
  } else {
    f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
  }
}

// Partial dot product of one lane's piece of q and K.
template <bool BF16>
__device__ __forceinline__ float piece_dot(const uint4& q, const uint4& k) {
  if constexpr (BF16) {
    float s = dot2_bf16(q.x, k.x, 0.f);
    s = dot2_bf16(q.y, k.y, s);
    s = dot2_bf16(q.z, k.z, s);
    return dot2_bf16(q.w, k.w, s);
  } else {
    float s = __uint_as_float(q.x) * __uint_as_float(k.x);
    s = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), s);
    s = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), s);
    return fmaf(__uint_as_float(q.w), __uint_as_float(k.w), s);
  }
}

template <bool BF16, int D, int BS, int GC>
__global__ __launch_bounds__(64) void paged_decode_kernel(
    const uint4* __restrict__ q, const uint4* __restrict__ k_cache, const uint4* __restrict__ v_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens, float scale_log2e,
    void* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_m, float* __restrict__ part_l,
    int num_q_heads, int num_kv_heads, int group, int chunks, int max_blocks_per_seq, int num_blocks,
    int part_blocks, int max_partitions) {
  using Gm = Geo<BF16, D, BS>;
  constexpr int EPL = Gm::kEPL, LPT = Gm::kLPT, TPI = Gm::kTPI, NI = Gm::kNI;
  constexpr float kNegInf = -INFINITY;

  const int lane = threadIdx.x;
  const int row = lane / LPT;
  const int col = lane % LPT;

  const bool split = part_blocks > 0;
  const int np = split ? max_partitions : 1;
  // Work items are numbered partition-major. The hardware deals workgroups round-robin to the
  // eight XCDs, so neighbouring ids must carry similar work: every (sequence, kv head) has a
  // first partition but only long sequences have late ones, and with the partition index
  // outermost each XCD gets an even share of every partition depth.
  unsigned wg = blockIdx.x;
  const unsigned per_p = gridDim.x / (unsigned)np;  // batch * num_kv_heads * chunks
  const int p = wg / per_p;
  wg %= per_p;
  const int ch = wg % chunks;
  wg /= chunks;
  const int g = wg % num_kv_heads;
  const int b = wg / num_kv_heads;
  const int h0 = g * group + ch * GC;

  int L = context_lens[b];
  L = min(L, max_blocks_per_seq * BS);
  const int nblk_seq = L > 0 ? (L + BS - 1) / BS : 0;
  int jb = 0, je = nblk_seq;
  if (split) {
    jb = p * part_blocks;
    je = min(jb + part_blocks, nblk_seq);
    if (jb >= je) return;  // partition past the end of this sequence
  }

  const size_t q_row0 = (size_t)b * num_q_heads + h0;
  if (jb >= je) {  // no split and an empty context: the output is zero
    if (row == 0) {
#pragma unroll
      for (int h = 0; h < GC; ++h) reinterpret_cast<uint4*>(out)[(q_row0 + h) * LPT + col] = make_uint4(0, 0, 0, 0);
    }
    return;
  }

  uint4 qv[GC];
#pragma unroll
  for (int h = 0; h < GC; ++h) qv[h] = q[(q_row0 + h) * LPT + col];

  float m[GC], l[GC], acc[GC][EPL];
#pragma unroll
  for (int h = 0; h < GC; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  const int32_t* bt = block_tables + (size_t)b * max_blocks_per_seq;
  const size_t chunk_stride = (size_t)NI * 64;  // uint4 pieces per (block, kv head) chunk

  auto load_chunk = [&](int blk, uint4 (&kr)[NI], uint4 (&vr)[NI]) {
    const size_t base = ((size_t)blk * num_kv_heads + g) * chunk_stride + lane;
#pragma unroll
    for (int i = 0; i < NI; ++i) kr[i] = k_cache[base + i * 64];
#pragma unroll
    for (int i = 0; i < NI; ++i) vr[i] = v_cache[base + i * 64];
  };

  auto process = [&](const uint4 (&kr)[NI], const uint4 (&vr)[NI], int nvalid) {
    float s[NI][GC];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int h = 0; h < GC; ++h) s[i][h] = group_sum<LPT>(piece_dot<BF16>(qv[h], kr[i])) * scale_log2e;
    }
    float v[NI][EPL];
#pragma unroll
    for (int i = 0; i < NI; ++i) unpack<BF16>(vr[i], v[i]);
    if (nvalid < BS) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if (i * TPI + row >= nvalid) {
#pragma unroll
          for (int h = 0; h < GC; ++h) s[i][h] = kNegInf;
#pragma unroll
          for (int e = 0; e < EPL; ++e) v[i][e] = 0.f;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < GC; ++h) {
      float mb = s[0][h];
#pragma unroll
      for (int i = 1; i < NI; ++i) mb = fmaxf(mb, s[i][h]);
      const float mn = fmaxf(m[h], mb);
      const float ms = mn == kNegInf ? 0.f : mn;
      const float alpha = fast_exp2(m[h] - ms);
      m[h] = mn;
      float lh = l[h] * alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const float pr = fast_exp2(s[i][h] - ms);
        lh += pr;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pr, v[i][e], acc[h][e]);
      }
      l[h] = lh;
    }
  };

  for (int base = jb; base < je; base += 64) {
    const int n = min(64, je - base);
    const int ids = lane < n ? bt[base + lane] : -1;
    uint4 kr[NI], vr[NI];
    int blk = __builtin_amdgcn_readfirstlane(ids);
    bool ok = blk >= 0 && blk < num_blocks;
    if (ok) load_chunk(blk, kr, vr);
    for (int jj = 0; jj < n; ++jj) {
      uint4 kn[NI], vn[NI];
      int blkn = -1;
      bool okn = false;
      if (jj + 1 < n) {
        blkn = __builtin_amdgcn_readlane(ids, jj + 1);
        okn = blkn >= 0 && blkn < num_blocks;
        if (okn) load_chunk(blkn, kn, vn);
      }
      if (ok) {
        const int nvalid = min(BS, L - (base + jj) * BS);
        process(kr, vr, nvalid);
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        kr[i] = kn[i];
        vr[i] = vn[i];
      }
      ok = okn;
    }
  }

  // Merge the TPI row states: max, rescale, add. Both lanes of a pair form the same two
  // products and add them in swapped order, so every row ends with identical bits.
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < GC; ++h) {
      const float mo = __shfl_xor(m[h], off, 64);
      const float lo = __shfl_xor(l[h], off, 64);
      const float mn = fmaxf(m[h], mo);
      const float ms = mn == kNegInf ? 0.f : mn;
      const float fs = fast_exp2(m[h] - ms);
      const float fo = fast_exp2(mo - ms);
      l[h] = l[h] * fs + lo * fo;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float ao = __shfl_xor(acc[h][e], off, 64);
        acc[h][e] = acc[h][e] * fs + ao * fo;
      }
      m[h] = mn;
    }
  }

  if (row != 0) return;
#pragma unroll
  for (int h = 0; h < GC; ++h) {
    const float inv = l[h] > 0.f ? 1.f / l[h] : 0.f;
    float o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = acc[h][e] * inv;
    if (split) {
      const size_t prow = (q_row0 + h) * (size_t)max_partitions + p;
      float4* po = reinterpret_cast<float4*>(part_o + prow * D + (size_t)col * EPL);
#pragma unroll
      for (int e = 0; e < EPL; e += 4) po[e / 4] = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
      if (col == 0) {
        part_m[prow] = m[h] == kNegInf ? kNegInf : m[h] * kLn2;
        part_l[prow] = l[h];
      }
    } else {
      uint4 w;
      if constexpr (BF16) {
        w = make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                       pack_bf16x2(o[6], o[7]));
      } else {
        w = make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3]));
      }
      reinterpret_cast<uint4*>(out)[(q_row0 + h) * LPT + col] = w;
    }
  }
}

template <bool BF16, int D, int BS, int GC>
hipError_t launch_t(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                    const int32_t* context_lens, float scale, void* out, float* part_o, float* part_m,
                    float* part_l, int batch, int num_q_heads, int num_kv_heads, int max_blocks_per_seq,
                    int num_blocks, int partition_size, int max_partitions, hipStream_t stream) {
  const int group = num_q_heads / num_kv_heads;
  const int chunks = group / GC;
  const int part_blocks = partition_size > 0 ? partition_size / BS : 0;
  const long long np = part_blocks > 0 ? max_partitions : 1;
  const long long grid = (long long)batch * num_kv_heads * chunks * np;
  hipLaunchKernelGGL((paged_decode_kernel<BF16, D, BS, GC>), dim3((unsigned)grid), dim3(64), 0, stream,
                     static_cast<const uint4*>(q), static_cast<const uint4*>(k_cache),
                     static_cast<const uint4*>(v_cache), block_tables, context_lens, scale * kLog2e, out, part_o,
                     part_m, part_l, num_q_heads, num_kv_heads, group, chunks, max_blocks_per_seq, num_blocks,
                     part_blocks, max_partitions);
  return hipGetLastError();
}

template <bool BF16, int D, int BS>
hipError_t launch_gc(int gc, const void* q, const void* kc, const void* vc, const int32_t* bt, const int32_t* cl,
                     float scale, void* out, float* po, float* pm, float* pl, int B, int Hq, int Hkv, int MBPS,
                     int NB, int P, int NP, hipStream_t s) {
  switch (gc) {
    case 1: return launch_t<BF16, D, BS, 1>(q, kc, vc, bt, cl, scale, out, po, pm, pl, B, Hq, Hkv, MBPS, NB, P, NP, s);
    case 2: return launch_t<BF16, D, BS, 2>(q, kc, vc, bt, cl, scale, out, po, pm, pl, B, Hq, Hkv, MBPS, NB, P, NP, s);
    case 4: return launch_t<BF16, D, BS, 4>(q, kc, vc, bt, cl, scale, out, po, pm, pl, B, Hq, Hkv, MBPS, NB, P, NP, s);
    case 8: return launch_t<BF16, D, BS, 8>(q, kc, vc, bt, cl, scale, out, po, pm, pl, B, Hq, Hkv, MBPS, NB, P, NP, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16, int D>
hipError_t launch_bs(int bs, int gc, const void* q, const void* kc, const void* vc, const int32_t* bt,
                     const int32_t* cl, float scale, void* out, float* po, float* pm, float* pl, int B, int Hq,
                     int Hkv, int MBPS, int NB, int P, int NP, hipStream_t s) {
  switch (bs) {
    case 8: return launch_gc<BF16, D, 8>(gc, q, kc, vc, bt, cl, scale, out, po, pm, pl, B, Hq, Hkv, MBPS, NB, P, NP, s);
    case 16: return launch_gc<BF16, D, 16>(gc, q, kc, vc, bt, cl, scale, out, po, pm, pl, B, Hq, Hkv, MBPS, NB, P, NP, s);
    case 32: return launch_gc<BF16, D, 32>(gc, q, kc, vc, bt, cl, scale, out, po, pm, pl, B, Hq, Hkv, MBPS, NB, P, NP, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int heads_per_chunk(int group) {
  for (int gc = 8; gc > 1; gc >>= 1)
    if (group % gc == 0) return gc;
  return 1;
}

hipError_t launch_paged_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                               const int32_t* context_lens, float scale, void* out, float* part_o, float* part_m,
                               float* part_l, int batch, int num_q_heads, int num_kv_heads, int head_dim,
                               int block_size, int max_blocks_per_seq, int num_blocks, int partition_size,
                               int max_partitions, bool bf16, hipStream_t stream) {
  if (mfma_decode_supported(bf16, head_dim, block_size))
    return launch_paged_decode_mfma(q, k_cache, v_cache, block_tables, context_lens, scale, out, part_o, part_m,
                                    part_l, batch, num_q_heads, num_kv_heads, head_dim, block_size,
                                    max_blocks_per_seq, num_blocks, partition_size, max_partitions, stream);
  const int gc = heads_per_chunk(num_q_heads / num_kv_heads);
#define XS_ARGS                                                                                                 \
  block_size, gc, q, k_cache, v_cache, block_tables, context_lens, scale, out, part_o, part_m, part_l, batch, \
      num_q_heads, num_kv_heads, max_blocks_per_seq, num_blocks, partition_size, max_partitions, stream
  if (bf16) {
    if (head_dim == 64) return launch_bs<true, 64>(XS_ARGS);
    if (head_dim == 128) return launch_bs<true, 128>(XS_ARGS);
  } else {
    if (head_dim == 64) return launch_bs<false, 64>(XS_ARGS);
    if (head_dim == 128) return launch_bs<false, 128>(XS_ARGS);
  }
#undef XS_ARGS
  return hipErrorInvalidValue;
}

}  // namespace xs
