// Split-K paged decode attention on the matrix cores (bf16 pools, head_dim 64/128, block_size
// 16/32). The per-tile math lives in xs_mfma_tile.h; this file walks the work items.
//
// A work item (sequence, kv head, head chunk, partition) goes to one workgroup of NW = 1, 2 or 4
// wavefronts, chosen at launch so that the grid fills the GPU. With split-K the grid has one
// workgroup per possible item (max_partitions per sequence), but workgroup k takes the k-th item
// that exists: each reads the batch's lengths, counts the partitions, and maps its id onto the
// full partitions first (sequence-major), then every sequence's partial last one. The real items
// thus fill the front of the grid, evenly over the CUs, and the ids past them leave at once.
// Batches of more than 256 sequences keep partition-major ids. The wavefronts take the item's
// 16-token tiles round-robin, each keeps its own online-softmax state, and they merge through
// LDS at the end (max, rescale, add). K/V are read with nontemporal loads (each byte is used
// once), and each wavefront loads its next tile into a second register set while it processes
// the current one.
// Fused append (k_new non-null): every wavefront that loads the tile holding token L-1 takes
// that token's K/V from k_new/v_new, and one wavefront writes them into the pools; no
// wavefront reads the slot being written.
// SW instances add the pages' sinks and sliding window (xserv compare phase10...cf1e9e41,
// attention.rs, `paged_decode_attention_sinks`): the range starts at position
// max(0, L - window), whose block and tile come first, and the unsplit output takes each head's
// sink logit into its softmax denominator. Split partials carry no sink; the sink merge adds it.
#include "xs_internal.h"
#include "xs_mfma_tile.h"

namespace xs {
namespace {

#ifndef XS_DECODE_MIN_WAVES_PER_EU
#define XS_DECODE_MIN_WAVES_PER_EU 4
#endif


template <int D, int BS, int GC, int NW>
constexpr int decode_smem_bytes() {
  using TA = TileAttn<D, GC>;
  constexpr int MERGE_FLOATS = TA::ACC * 4 * 64 + 2 * GC;  // one wavefront's (acc, m, l)
  return NW * TA::STAGE_BYTES > (NW - 1) * MERGE_FLOATS * 4 ? NW * TA::STAGE_BYTES : (NW - 1) * MERGE_FLOATS * 4;
}

// Writes zeros to rows q_row0 .. q_row0+GC-1 of out (one wavefront, 16 bytes per lane and store).
template <int D, int GC>
__device__ __forceinline__ void zero_rows(void* out, size_t q_row0, int lane) {
  constexpr int PIECES = GC * (D / 8);  // 16-byte pieces
  uint4* o = reinterpret_cast<uint4*>(out) + q_row0 * (D / 8);
#pragma unroll
  for (int i = lane; i < PIECES; i += 64) o[i] = make_uint4(0, 0, 0, 0);
}

// One work item: partition p of (sequence b, kv head g, head chunk ch).
template <int D, int BS, int GC, int NW, bool SW>
__device__ __forceinline__ void decode_item(const DecodeParams& prm, unsigned char* smem, const int p, const int b,
                                            const int g, const int ch) {
  using TA = TileAttn<D, GC>;
  constexpr int KK = TA::KK, NH = TA::NH, HP = TA::HP, ROW16 = TA::ROW16, VL = TA::VL, ACC = TA::ACC;
  constexpr int TPB = BS / 16;  // tiles per block
  constexpr int MERGE_FLOATS = ACC * 4 * 64 + 2 * GC;  // one wavefront's (acc, m, l)
  constexpr float kNegInf = -INFINITY;
  static_assert(BS % 16 == 0, "block_size must hold whole 16-token tiles");

  const int wave = NW > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
  const int lane = threadIdx.x & 63;
  unsigned char* vlds = smem + wave * TA::STAGE_BYTES;

  const int num_kv_heads = prm.num_kv_heads;
  const int max_blocks_per_seq = prm.max_blocks_per_seq;
  const int max_partitions = prm.max_partitions;
  const bool split = prm.part_blocks > 0;
  const int h0 = g * prm.group + ch * GC;
  const int32_t* bt = prm.block_tables + (size_t)b * max_blocks_per_seq;

  // The ids of the item's first 64 blocks do not depend on the context length (without a window),
  // so their load goes out together with the length's instead of after it.
  const int jb0 = split ? p * prm.part_blocks : 0;
  int ids_pre = -1;
  if constexpr (!SW) {
    if (jb0 + lane < max_blocks_per_seq) ids_pre = bt[jb0 + lane];
  }
  const int L_in = prm.context_lens[b];
  const int L = min(L_in, max_blocks_per_seq * BS);
  const int nblk_seq = L > 0 ? (L + BS - 1) / BS : 0;
  int jb = jb0, je = split ? min(jb0 + prm.part_blocks, nblk_seq) : nblk_seq;
  // First position in the window (0 without one); blocks wholly before it are skipped.
  const int t0w = SW && prm.window > 0 ? max(0, L - prm.window) : 0;
  if constexpr (SW) jb = max(jb, t0w / BS);
  if (split && jb >= je) return;  // the whole workgroup leaves together
  const size_t q_row0 = (size_t)b * prm.num_q_heads + h0;
  if (jb >= je) {  // no split, empty context
    if (wave == 0) zero_rows<D, GC>(prm.out, q_row0, lane);
    return;
  }
  auto valid = [&](int blk) { return blk >= 0 && blk < prm.num_blocks; };

  // Fused append: token L-1 comes from k_new/v_new; the item holding it writes them to the pools.
  const bool append = prm.k_new != nullptr && L_in >= 1 && L_in == L;
  const int last = append ? L - 1 : -1;
  const size_t new_row = ((size_t)b * num_kv_heads + g) * ROW16;
  if (append && ch == 0 && wave == 0 && last / BS >= jb && last / BS < je && lane < 2 * ROW16) {
    const int blk = bt[last / BS];
    if (valid(blk)) {
      const size_t dst = (((size_t)blk * num_kv_heads + g) * BS + last % BS) * ROW16;
      if (lane < ROW16)
        prm.k_cache_w[dst + lane] = prm.k_new[new_row + lane];
      else
        prm.v_cache_w[dst + lane - ROW16] = prm.v_new[new_row + lane - ROW16];
    }
  }

  TA st;
  st.reset();
  st.load_q(prm.q, q_row0, lane);

  auto load = [&](int blk, int tile, uint4 (&kr)[KK], uint4 (&vr)[VL]) {
    const size_t row0 = ((size_t)blk * num_kv_heads + g) * BS + (tile % TPB) * 16;
    TA::load_tile(prm.k_cache + row0 * ROW16, prm.v_cache + row0 * ROW16, last - 16 * tile, prm.k_new + new_row,
                  prm.v_new + new_row, lane, kr, vr);
  };

  // Block ids of 64 consecutive blocks of the range sit in one VGPR, one per lane.
  int id_chunk = -1, ids = -1;
  if constexpr (!SW) {
    id_chunk = 0;
    ids = jb + lane < je ? ids_pre : -1;
  }
  auto block_of = [&](int tile) -> int {
    const int rel = tile / TPB - jb;
    const int c64 = rel >> 6;
    if (c64 != id_chunk) {
      id_chunk = c64;
      const int idx = jb + (c64 << 6) + lane;
      ids = idx < je ? bt[idx] : -1;
    }
    return __builtin_amdgcn_readlane(ids, rel & 63);
  };

  // Tiles of the range, dealt round-robin to the NW wavefronts; the next tile of a wavefront is
  // loaded (into the other register set) while the current one is processed.
  const int t_end = (min(je * BS, L) + 15) / 16;
  int t = (SW ? max(jb * TPB, t0w / 16) : jb * TPB) + wave;
  uint4 kA[KK], vA[VL], kB[KK], vB[VL];
  int bA = -1, bB = -1;
  if (t < t_end) {
    bA = block_of(t);
    if (valid(bA)) load(bA, t, kA, vA);
  }
  while (t < t_end) {
    const int t2 = t + NW;
    if (t2 < t_end) {
      bB = block_of(t2);
      if (valid(bB)) load(bB, t2, kB, vB);
    }
    if (valid(bA)) st.process_range(kA, vA, SW ? t0w - 16 * t : 0, min(16, L - 16 * t), vlds, prm.scale_log2e, lane);
    if (t2 >= t_end) break;
    const int t3 = t2 + NW;
    if (t3 < t_end) {
      bA = block_of(t3);
      if (valid(bA)) load(bA, t3, kA, vA);
    }
    if (valid(bB)) st.process_range(kB, vB, SW ? t0w - 16 * t2 : 0, min(16, L - 16 * t2), vlds, prm.scale_log2e, lane);
    t = t3;
  }

  float m_h[HP * 4], l_h[HP * 4];
  st.head_stats(m_h, l_h);

  if constexpr (NW > 1) {
    // Merge the NW wavefront states through LDS, once every wavefront is done with its staging.
    float* mrg = reinterpret_cast<float*>(smem);
    __syncthreads();
    if (wave > 0) {
      float* mine = mrg + (wave - 1) * MERGE_FLOATS;
#pragma unroll
      for (int a = 0; a < ACC; ++a) {
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[(a * 4 + i) * 64 + lane] = st.acc[a][i];
      }
      if (lane < GC) {
        mine[ACC * 4 * 64 + lane] = m_h[lane];
        mine[ACC * 4 * 64 + GC + lane] = l_h[lane];
      }
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int r = 0; r < HP * 4; ++r) {
      const int hr = r % GC;
      float M = m_h[r];
#pragma unroll
      for (int w = 1; w < NW; ++w) M = fmaxf(M, mrg[(w - 1) * MERGE_FLOATS + ACC * 4 * 64 + hr]);
      const float Ms = M == kNegInf ? 0.f : M;
      const float f0 = fast_exp2(m_h[r] - Ms);
      float lsum = l_h[r] * f0;
      const int hp = r / 4, i = r % 4;
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) st.acc[hp * NH + hf][i] *= f0;
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        const float* other = mrg + (w - 1) * MERGE_FLOATS;
        const float fw = fast_exp2(other[ACC * 4 * 64 + hr] - Ms);
        lsum += other[ACC * 4 * 64 + GC + hr] * fw;
#pragma unroll
        for (int hf = 0; hf < NH; ++hf)
          st.acc[hp * NH + hf][i] += other[((hp * NH + hf) * 4 + i) * 64 + lane] * fw;
      }
      m_h[r] = M;
      l_h[r] = lsum;
    }
  }

  // Output rows: head r = 4hp + i < GC, d = 64hf + lane (64 consecutive elements per store).
#pragma unroll
  for (int r = 0; r < GC; ++r) {
    const int hp = r / 4, i = r % 4;
    const float inv = l_h[r] > 0.f ? 1.f / l_h[r] : 0.f;
    if (split) {
      const size_t prow = (q_row0 + r) * (size_t)max_partitions + p;
      float* po = prm.part_o + prow * D;
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) po[64 * hf + lane] = st.acc[hp * NH + hf][i] * inv;
      if (lane == 0) {
        prm.part_m[prow] = m_h[r] == kNegInf ? kNegInf : m_h[r] * kLn2;
        prm.part_l[prow] = l_h[r];
      }
    } else {
      float f = inv;
      if (SW && prm.sinks) {
        // The sink sigma (scaled-score units) joins the denominator: o = acc e^(m-M) / (l e^(m-M) + e^(sigma-M)).
        const float sg = bf16lo_to_f32((uint32_t)prm.sinks[h0 + r]) * kLog2e;
        const float M = fmaxf(m_h[r], sg);
        const float fo = m_h[r] == kNegInf ? 0.f : fast_exp2(m_h[r] - M);
        const float den = l_h[r] * fo + (sg == kNegInf ? 0.f : fast_exp2(sg - M));
        f = den > 0.f ? fo / den : 0.f;
      }
      uint16_t* o = reinterpret_cast<uint16_t*>(prm.out) + (q_row0 + r) * D;
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) o[64 * hf + lane] = (uint16_t)f32_to_bf16_rne(st.acc[hp * NH + hf][i] * f);
    }
  }
}

// The dense order scans the batch's lengths in every workgroup: up to this many sequences.
constexpr int kDenseMaxBatch = 256;

// Partitions of sequence b that the split grid computes: full ones (part_blocks blocks) and a
// partial last one. Partitions at or past max_partitions are not computed.
template <int BS>
__device__ __forceinline__ void seq_partitions(const DecodeParams& prm, int b, int& nfull, int& npartial) {
  const int L = min(prm.context_lens[b], prm.max_blocks_per_seq * BS);
  const int nblk = L > 0 ? (L + BS - 1) / BS : 0;
  nfull = min(nblk / prm.part_blocks, prm.max_partitions);
  npartial = nblk % prm.part_blocks != 0 && nblk / prm.part_blocks < prm.max_partitions ? 1 : 0;
}

// Split items in the order that evens out the work per CU: full partitions first
// (sequence-major, all the same size), then the partial last partitions by decreasing size (ties
// by sequence). Workgroup k takes the item
// whose rank is k with every second round of ncu consecutive ids reversed: with the whole grid
// resident, ids k and k + ncu share a CU (the device deals workgroups to its CUs in turn), so a CU
// that gets one of the larger partial items in one round gets one of the smaller ones in the
// next. Sets b, p and seg (kv head * chunks + chunk); b = -1 when the rank is past the last item.
template <int BS>
__device__ __forceinline__ void dense_item(const DecodeParams& prm, int k, int& b, int& p, int& seg) {
  const int lane = threadIdx.x & 63;
  const int batch = prm.batch;
  const int segs = prm.num_kv_heads * prm.chunks;
  const int ncu = max(prm.ncu, 1);
  const int rnd = k / ncu, col = k - rnd * ncu;
  // Only whole rounds are reversed, so every rank below the grid size keeps exactly one id.
  if ((rnd & 1) && (long long)(rnd + 1) * ncu <= (long long)gridDim.x) k = rnd * ncu + (ncu - 1 - col);
  int F = 0;
  for (int b0 = 0; b0 < batch; b0 += 64) {
    int nf = 0, np1 = 0;
    if (b0 + lane < batch) seq_partitions<BS>(prm, b0 + lane, nf, np1);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) nf += __shfl_xor(nf, off, 64);
    F += nf * segs;
  }
  const bool full = k < F;
  if (!full) k -= F;
  b = -1;
  p = 0;
  seg = 0;
  if (!full) {
    // The sequence whose partial partition has rank r = k / segs by (size descending, index
    // ascending). Partial sizes (in blocks, 0 for none) sit one per lane, 64 sequences per
    // register; the size of rank r is found by binary search on counts taken with ballots, then
    // the sequence among those of that size by index.
    constexpr int kMaxChunks = kDenseMaxBatch / 64;
    int psz[kMaxChunks], pnf[kMaxChunks];
#pragma unroll
    for (int ch = 0; ch < kMaxChunks; ++ch) {
      psz[ch] = 0;
      pnf[ch] = 0;
      const int bb = 64 * ch + lane;
      if (bb < batch) {
        int nf = 0, np1 = 0;
        seq_partitions<BS>(prm, bb, nf, np1);
        const int L = min(prm.context_lens[bb], prm.max_blocks_per_seq * BS);
        const int nblk = L > 0 ? (L + BS - 1) / BS : 0;
        psz[ch] = np1 ? nblk - nf * prm.part_blocks : 0;
        pnf[ch] = nf;
      }
    }
    auto count_ge = [&](int sz) {  // partial partitions of at least sz blocks
      int n = 0;
#pragma unroll
      for (int ch = 0; ch < kMaxChunks; ++ch) n += __builtin_popcountll(__ballot(psz[ch] >= sz));
      return n;
    };
    const int r = k / segs;
    if (r < count_ge(1)) {
      int lo = 1, hi = prm.part_blocks - 1;  // the size of rank r lies in [lo, hi]
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (count_ge(mid) > r) lo = mid;
        else hi = mid - 1;
      }
      int jth = r - count_ge(lo + 1);  // among the sequences of size lo, in index order
#pragma unroll
      for (int ch = 0; ch < kMaxChunks; ++ch) {
        const unsigned long long m = __ballot(psz[ch] == lo);
        const int cnt = __builtin_popcountll(m);
        if (b < 0 && jth < cnt) {
          const unsigned long long below = lane ? m & ((~0ull) >> (64 - lane)) : 0ull;
          const unsigned long long hit = __ballot(((m >> lane) & 1ull) && __builtin_popcountll(below) == jth);
          const int first = __builtin_ctzll(hit);
          b = 64 * ch + first;
          p = __shfl(pnf[ch], first, 64);
          seg = k % segs;
        }
        jth -= cnt;
      }
    }
  } else {
    int base = 0;
    for (int b0 = 0; b0 < batch && b < 0; b0 += 64) {
      int nf = 0, np1 = 0;
      if (b0 + lane < batch) seq_partitions<BS>(prm, b0 + lane, nf, np1);
      const int own = nf * segs;
      int incl = own;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      const unsigned long long hit = __ballot(b0 + lane < batch && base + incl > k);
      if (hit) {
        const int first = __builtin_ctzll(hit);
        const int r = k - base - __shfl(incl - own, first, 64);
        b = b0 + first;
        p = r / segs;
        seg = r % segs;
      } else {
        base += __shfl(incl, 63, 64);
      }
    }
  }
  b = __builtin_amdgcn_readfirstlane(b);
  p = __builtin_amdgcn_readfirstlane(p);
  seg = __builtin_amdgcn_readfirstlane(seg);
}

template <int D, int BS, int GC, int NW, bool SW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(XS_DECODE_MIN_WAVES_PER_EU)))
void paged_decode_mfma_kernel(const DecodeParams prm) {
  __shared__ __align__(16) unsigned char smem[decode_smem_bytes<D, BS, GC, NW>()];
  int b, p, seg;
  if (prm.part_blocks > 0 && prm.dense) {
    dense_item<BS>(prm, blockIdx.x, b, p, seg);
    if (b < 0) return;  // past the items that exist
  } else if (prm.part_blocks > 0) {
    // Partition-major ids: for one sequence (the ranked order would list its partitions in this
    // same order, but only after reading its length) and for large batches (where every
    // workgroup would otherwise scan all lengths). Neighbouring ids carry similar work, and every
    // XCD gets each partition depth.
    const int per_p = prm.batch * prm.num_kv_heads * prm.chunks;
    p = blockIdx.x / per_p;
    seg = blockIdx.x % (prm.chunks * prm.num_kv_heads);
    b = (blockIdx.x % per_p) / (prm.chunks * prm.num_kv_heads);
  } else {
    // No split: one item per (sequence, kv head, chunk).
    seg = blockIdx.x % (prm.chunks * prm.num_kv_heads);
    b = blockIdx.x / (prm.chunks * prm.num_kv_heads);
    p = 0;
  }
  decode_item<D, BS, GC, NW, SW>(prm, smem, p, b, seg / prm.chunks, seg % prm.chunks);
}

template <int D, int BS, int GC, bool SW>
hipError_t launch_sw(const DecodeArgs& a, hipStream_t stream) {
  DecodeParams prm = make_params(a, GC);
  const long long np = prm.part_blocks > 0 ? a.max_partitions : 1;
  const long long grid = (long long)a.batch * a.num_kv_heads * prm.chunks * np;
  // Item order of the split grid. The ranked order costs every workgroup one more dependent load
  // (all lengths) before its block ids; it pays when the CUs' loads could differ by whole large
  // items. Partition-major ids are kept for one sequence (the same order), for large batches,
  // and for grids of at most 4 workgroups per CU whose items are at most 8 tiles (any imbalance
  // is then a few tiles; measured on the GPT-2 batch of 8: 11.5 -> 10.6 us per step).
  const bool small_items = a.partition_size <= 128 && grid <= 4LL * device_cu_count();
  prm.dense = prm.part_blocks > 0 && a.batch > 1 && a.batch <= kDenseMaxBatch && !small_items ? 1 : 0;
  // Wavefronts per work item: the most that keep the whole grid resident at once (4 per SIMD),
  // or 4 when the grid needs several rounds anyway (finer pieces even out the last round).
  const long long resident = 16LL * device_cu_count();
  int nw = 4;
  if (grid <= resident) nw = grid * 4 <= resident ? 4 : grid * 2 <= resident ? 2 : 1;
  const dim3 g3((unsigned)grid);
  switch (nw) {
    case 1: hipLaunchKernelGGL((paged_decode_mfma_kernel<D, BS, GC, 1, SW>), g3, dim3(64), 0, stream, prm); break;
    case 2: hipLaunchKernelGGL((paged_decode_mfma_kernel<D, BS, GC, 2, SW>), g3, dim3(128), 0, stream, prm); break;
    default: hipLaunchKernelGGL((paged_decode_mfma_kernel<D, BS, GC, 4, SW>), g3, dim3(256), 0, stream, prm); break;
  }
  return hipGetLastError();
}

template <int D, int BS, int GC>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  if (a.sinks || a.window > 0) return launch_sw<D, BS, GC, true>(a, stream);
  return launch_sw<D, BS, GC, false>(a, stream);
}

template <int D, int BS>
hipError_t launch_gc(int gc, const DecodeArgs& a, hipStream_t s) {
  switch (gc) {
    case 1: return launch_t<D, BS, 1>(a, s);
    case 2: return launch_t<D, BS, 2>(a, s);
    case 4: return launch_t<D, BS, 4>(a, s);
    case 8: return launch_t<D, BS, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool mfma_decode_supported(bool bf16, int head_dim, int block_size) {
  return bf16 && (head_dim == 64 || head_dim == 128) && (block_size == 16 || block_size == 32);
}

hipError_t launch_paged_decode_mfma(const DecodeArgs& a, hipStream_t stream) {
  const int gc = heads_per_chunk(a.num_q_heads / a.num_kv_heads);
  if (a.head_dim == 128 && a.block_size == 16) return launch_gc<128, 16>(gc, a, stream);
  if (a.head_dim == 128 && a.block_size == 32) return launch_gc<128, 32>(gc, a, stream);
  if (a.head_dim == 64 && a.block_size == 16) return launch_gc<64, 16>(gc, a, stream);
  if (a.head_dim == 64 && a.block_size == 32) return launch_gc<64, 32>(gc, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace xs
