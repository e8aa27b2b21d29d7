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

#include <atomic>

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
__global__ __launch_bounds__(64) void paged_decode_kernel(const DecodeParams prm) {
  using Gm = Geo<BF16, D, BS>;
  constexpr int EPL = Gm::kEPL, LPT = Gm::kLPT, TPI = Gm::kTPI, NI = Gm::kNI;
  constexpr float kNegInf = -INFINITY;

  const int lane = threadIdx.x;
  const int row = lane / LPT;
  const int col = lane % LPT;

  const int num_kv_heads = prm.num_kv_heads;
  const bool split = prm.part_blocks > 0;
  const int np = split ? prm.max_partitions : 1;
  // Work items are numbered partition-major. The hardware deals workgroups round-robin to the
  // eight XCDs, so neighbouring ids must carry similar work: every (sequence, kv head) has a
  // first partition but only long sequences have late ones, and with the partition index
  // outermost each XCD gets an even share of every partition depth.
  unsigned wg = blockIdx.x;
  const unsigned per_p = gridDim.x / (unsigned)np;  // batch * num_kv_heads * chunks
  const int p = wg / per_p;
  wg %= per_p;
  const int ch = wg % prm.chunks;
  wg /= prm.chunks;
  const int g = wg % num_kv_heads;
  const int b = wg / num_kv_heads;
  const int h0 = g * prm.group + ch * GC;

  const int L_in = prm.context_lens[b];
  const int L = min(L_in, prm.max_blocks_per_seq * BS);
  const int nblk_seq = L > 0 ? (L + BS - 1) / BS : 0;
  int jb = 0, je = nblk_seq;
  if (split) {
    jb = p * prm.part_blocks;
    je = min(jb + prm.part_blocks, nblk_seq);
    if (jb >= je) return;  // partition past the end of this sequence
  }

  const size_t q_row0 = (size_t)b * prm.num_q_heads + h0;
  if (jb >= je) {  // no split and an empty context: the output is zero
    if (row == 0) {
#pragma unroll
      for (int h = 0; h < GC; ++h)
        reinterpret_cast<uint4*>(prm.out)[(q_row0 + h) * LPT + col] = make_uint4(0, 0, 0, 0);
    }
    return;
  }
  const int32_t* bt = prm.block_tables + (size_t)b * prm.max_blocks_per_seq;
  auto valid = [&](int blk) { return blk >= 0 && blk < prm.num_blocks; };

  // Fused append: token L-1 comes from k_new/v_new; the item holding it writes them to the pools.
  const bool append = prm.k_new != nullptr && L_in >= 1 && L_in == L;
  const int last = append ? L - 1 : -1;
  const size_t new_row = ((size_t)b * num_kv_heads + g) * LPT;  // LPT 16-byte pieces per row
  if (append && ch == 0 && last / BS >= jb && last / BS < je && lane < 2 * LPT) {
    const int blk = bt[last / BS];
    if (valid(blk)) {
      const size_t dst = (((size_t)blk * num_kv_heads + g) * BS + last % BS) * LPT;
      if (lane < LPT)
        prm.k_cache_w[dst + lane] = prm.k_new[new_row + lane];
      else
        prm.v_cache_w[dst + lane - LPT] = prm.v_new[new_row + lane - LPT];
    }
  }

  uint4 qv[GC];
#pragma unroll
  for (int h = 0; h < GC; ++h) qv[h] = prm.q[(q_row0 + h) * LPT + col];

  float m[GC], l[GC], acc[GC][EPL];
#pragma unroll
  for (int h = 0; h < GC; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  const size_t chunk_stride = (size_t)NI * 64;  // uint4 pieces per (block, kv head) chunk

  auto load_chunk = [&](int blk, int jblk, uint4 (&kr)[NI], uint4 (&vr)[NI]) {
    const size_t base = ((size_t)blk * num_kv_heads + g) * chunk_stride + lane;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const bool is_new = jblk * BS + i * TPI + row == last;
      kr[i] = load_stream(is_new ? prm.k_new + new_row + col : prm.k_cache + base + i * 64);
      vr[i] = load_stream(is_new ? prm.v_new + new_row + col : prm.v_cache + base + i * 64);
    }
  };

  auto process = [&](const uint4 (&kr)[NI], const uint4 (&vr)[NI], int nvalid) {
    float s[NI][GC];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int h = 0; h < GC; ++h) s[i][h] = group_sum<LPT>(piece_dot<BF16>(qv[h], kr[i])) * prm.scale_log2e;
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
    bool ok = valid(blk);
    if (ok) load_chunk(blk, base, kr, vr);
    for (int jj = 0; jj < n; ++jj) {
      uint4 kn[NI], vn[NI];
      int blkn = -1;
      bool okn = false;
      if (jj + 1 < n) {
        blkn = __builtin_amdgcn_readlane(ids, jj + 1);
        okn = valid(blkn);
        if (okn) load_chunk(blkn, base + jj + 1, kn, vn);
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
      const size_t prow = (q_row0 + h) * (size_t)prm.max_partitions + p;
      float4* po = reinterpret_cast<float4*>(prm.part_o + prow * D + (size_t)col * EPL);
#pragma unroll
      for (int e = 0; e < EPL; e += 4) po[e / 4] = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
      if (col == 0) {
        prm.part_m[prow] = m[h] == kNegInf ? kNegInf : m[h] * kLn2;
        prm.part_l[prow] = l[h];
      }
    } else {
      uint4 w;
      if constexpr (BF16) {
        w = make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                       pack_bf16x2(o[6], o[7]));
      } else {
        w = make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3]));
      }
      reinterpret_cast<uint4*>(prm.out)[(q_row0 + h) * LPT + col] = w;
    }
  }
}

template <bool BF16, int D, int BS, int GC>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const DecodeParams prm = make_params(a, GC);
  const long long np = prm.part_blocks > 0 ? a.max_partitions : 1;
  const long long grid = (long long)a.batch * a.num_kv_heads * prm.chunks * np;
  hipLaunchKernelGGL((paged_decode_kernel<BF16, D, BS, GC>), dim3((unsigned)grid), dim3(64), 0, stream, prm);
  return hipGetLastError();
}

template <bool BF16, int D, int BS>
hipError_t launch_gc(int gc, const DecodeArgs& a, hipStream_t s) {
  switch (gc) {
    case 1: return launch_t<BF16, D, BS, 1>(a, s);
    case 2: return launch_t<BF16, D, BS, 2>(a, s);
    case 4: return launch_t<BF16, D, BS, 4>(a, s);
    case 8: return launch_t<BF16, D, BS, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16, int D>
hipError_t launch_bs(int gc, const DecodeArgs& a, hipStream_t s) {
  switch (a.block_size) {
    case 8: return launch_gc<BF16, D, 8>(gc, a, s);
    case 16: return launch_gc<BF16, D, 16>(gc, a, s);
    case 32: return launch_gc<BF16, D, 32>(gc, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int heads_per_chunk(int group) {
  for (int gc = 8; gc > 1; gc >>= 1)
    if (group % gc == 0) return gc;
  return 1;
}

int device_cu_count() {
  static std::atomic<int> cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int known = cache[dev].load(std::memory_order_relaxed);
    if (known > 0) return known;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

DecodeParams make_params(const DecodeArgs& a, int heads_per_wave) {
  DecodeParams p;
  p.q = static_cast<const uint4*>(a.q);
  p.k_cache = static_cast<const uint4*>(a.k_cache);
  p.v_cache = static_cast<const uint4*>(a.v_cache);
  p.block_tables = a.block_tables;
  p.context_lens = a.context_lens;
  p.k_new = static_cast<const uint4*>(a.k_new);
  p.v_new = static_cast<const uint4*>(a.v_new);
  p.k_cache_w = static_cast<uint4*>(a.k_cache);
  p.v_cache_w = static_cast<uint4*>(a.v_cache);
  p.scale_log2e = a.scale * kLog2e;
  p.sinks = static_cast<const uint16_t*>(a.sinks);
  p.window = a.window;
  p.batch = a.batch;
  p.ncu = device_cu_count();
  p.out = a.out;
  p.part_o = a.part_o;
  p.part_m = a.part_m;
  p.part_l = a.part_l;
  p.num_q_heads = a.num_q_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.group = a.num_q_heads / a.num_kv_heads;
  p.chunks = p.group / heads_per_wave;
  p.max_blocks_per_seq = a.max_blocks_per_seq;
  p.num_blocks = a.num_blocks;
  p.part_blocks = a.partition_size > 0 ? a.partition_size / a.block_size : 0;
  p.max_partitions = a.max_partitions;
  p.dense = 0;
  return p;
}

hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream) {
  if (mfma_decode_supported(a.bf16, a.head_dim, a.block_size)) return launch_paged_decode_mfma(a, stream);
  if (a.sinks || a.window > 0) return hipErrorInvalidValue;  // sinks and windows: matrix-core shapes only
  const int gc = heads_per_chunk(a.num_q_heads / a.num_kv_heads);
  if (a.bf16) {
    if (a.head_dim == 64) return launch_bs<true, 64>(gc, a, stream);
    if (a.head_dim == 128) return launch_bs<true, 128>(gc, a, stream);
  } else {
    if (a.head_dim == 64) return launch_bs<false, 64>(gc, a, stream);
    if (a.head_dim == 128) return launch_bs<false, 128>(gc, a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace xs
