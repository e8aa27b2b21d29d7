// Balanced paged decode attention: every wavefront streams the same number of tiles.
//
// Same result as xs_paged_attn_decode followed by xs_paged_attn_reduce (xserv compare
// phase10...cf1e9e41, attention.rs, `paged_decode_attention`; GQA by `repeat_kv` in xserv
// compare phase8...phase13), with a different split of the work:
//   - A segment is one (sequence b, kv head g, head chunk ch). It has T_b = ceil(L_b / 16)
//     tiles of 16 tokens. Segments are numbered s = (b * Hkv + g) * chunks + ch, and their tiles
//     are laid end to end: T = sum_b T_b * Hkv * chunks tiles in all.
//   - W_eff = min(workers, ceil(T / min_tiles)) wavefronts ("workers") each take one
//     contiguous range, [floor(w T / W_eff), floor((w+1) T / W_eff)). A worker streams its range
//     with the next tile always in flight, across segment boundaries, so no worker idles
//     between work items and all of them finish together.
//   - The part of segment s inside worker w's range is a piece. A segment that lies inside one
//     worker's range is finished there: its output is written directly. Otherwise each piece
//     leaves its (o, m, l) in workspace row (s + w) * GC + r, for head r of the chunk. That row
//     is unique: if w and w' both touch s and s', then s < s' forces w <= w', so s + w = s' + w'
//     only when s = s' and w = w'. The merge kernel then combines the pieces of each segment
//     with the log-sum-exp rule.
//   - The worker holding tile x is ((x + 1) W_eff - 1) / T, so the merge finds a segment's
//     pieces without any record of the schedule.
// The per-tile math is TileAttn (xs_mfma_tile.h). Fused append (k_new non-null): as in the
// split-K kernel, token L-1 is read from k_new/v_new, and the worker holding it writes it to
// the pools.
#include <math.h>

#include <algorithm>
#include <atomic>

#include "xs_internal.h"
#include "xs_mfma_tile.h"

namespace xs {
namespace {

constexpr int kWavesPerGroup = 4;

// The worker whose range holds global tile x.
__device__ __forceinline__ int worker_of(long long x, int weff, long long T) {
  return (int)(((x + 1) * (long long)weff - 1) / T);
}

// Tiles of sequence b (after clamping its length to the block table).
__device__ __forceinline__ int seq_tiles(int L, int cap) {
  L = min(L, cap);
  return L > 0 ? (L + 15) >> 4 : 0;
}

// A wave-uniform 64-bit value moved into scalar registers.
__device__ __forceinline__ long long uniform64(long long x) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)(x & 0xffffffffLL));
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((unsigned long long)x >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

// Sum of x over the wavefront.
__device__ __forceinline__ long long wave_sum(long long x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const int lo = __shfl_xor((int)(x & 0xffffffffLL), off, 64);
    const int hi = __shfl_xor((int)(x >> 32), off, 64);
    x += ((long long)hi << 32) | (unsigned)lo;
  }
  return x;
}

// Inclusive prefix sum of x over the lanes of the wavefront.
__device__ __forceinline__ long long wave_incl_scan(long long x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int lo = __shfl_up((int)(x & 0xffffffffLL), off, 64);
    const int hi = __shfl_up((int)(x >> 32), off, 64);
    const long long y = ((long long)hi << 32) | (unsigned)lo;
    if (lane >= off) x += y;
  }
  return x;
}

// Total tiles T of the batch.
__device__ long long total_tiles(const int32_t* lens, int batch, int cap, int segs, int lane) {
  long long t = 0;
  for (int b0 = 0; b0 < batch; b0 += 64) {
    const int b = b0 + lane;
    t += b < batch ? (long long)seq_tiles(lens[b], cap) * segs : 0;
  }
  return uniform64(wave_sum(t));
}

// Finds the sequence b holding global tile x; returns C_b (tiles before sequence b).
__device__ long long locate(const int32_t* lens, int batch, int cap, int segs, long long x, int lane, int* b_out) {
  long long base = 0;
  for (int b0 = 0; b0 < batch; b0 += 64) {
    const int b = b0 + lane;
    const long long own = b < batch ? (long long)seq_tiles(lens[b], cap) * segs : 0;
    const long long incl = wave_incl_scan(own, lane);
    const unsigned long long hit = __ballot(b < batch && base + incl > x);
    if (hit) {
      const int first = __builtin_ctzll(hit);
      const long long excl = incl - own;
      *b_out = __builtin_amdgcn_readfirstlane(b0 + first);
      return uniform64(base + __shfl(excl, first, 64));
    }
    base = uniform64(base + __shfl(incl, 63, 64));
  }
  *b_out = batch;
  return base;
}

template <int D, int BS, int GC>
#ifndef XS_BALANCED_WAVES_PER_EU
#define XS_BALANCED_WAVES_PER_EU 4
#endif
__global__ __launch_bounds__(64 * kWavesPerGroup) __attribute__((amdgpu_waves_per_eu(XS_BALANCED_WAVES_PER_EU)))
void paged_decode_balanced_kernel(const BalancedParams prm) {
  using TA = TileAttn<D, GC>;
  constexpr int KK = TA::KK, NH = TA::NH, HP = TA::HP, ROW16 = TA::ROW16, VL = TA::VL;
  constexpr int TPB = BS / 16;  // tiles per block
  constexpr float kNegInf = -INFINITY;
  static_assert(BS % 16 == 0, "block_size must hold whole 16-token tiles");

  __shared__ __align__(16) unsigned char smem[kWavesPerGroup * TA::STAGE_BYTES];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  unsigned char* vlds = smem + wave * TA::STAGE_BYTES;
  const DecodeParams& d = prm.d;

  const int w = blockIdx.x * kWavesPerGroup + wave;
  const int W = prm.workers;
  if (w >= W) return;
  const int batch = prm.batch;
  const int Hkv = d.num_kv_heads;
  const int chunks = d.chunks;
  const int segs = Hkv * chunks;
  const int cap = d.max_blocks_per_seq * BS;
  const int32_t* lens = d.context_lens;

  // Sequences with no tokens get zeros (worker w takes sequences w, w + W, ...).
  for (int b = w; b < batch; b += W) {
    if (lens[b] <= 0) {
      uint4* o = reinterpret_cast<uint4*>(d.out) + (size_t)b * d.num_q_heads * ROW16;
      for (int i = lane; i < d.num_q_heads * ROW16; i += 64) o[i] = make_uint4(0, 0, 0, 0);
    }
  }

  const long long T = total_tiles(lens, batch, cap, segs, lane);
  if (T == 0) return;
  const int weff = (int)min((long long)W, max(1LL, (T + prm.min_tiles - 1) / prm.min_tiles));
  if (w >= weff) return;
  const long long x0 = (long long)w * T / weff;
  const long long x1 = (long long)(w + 1) * T / weff;
  if (x0 >= x1) return;

  // Cursor over the worker's tiles: sequence b (C = tiles before it), segment sib within b,
  // tile t within the segment (Tb tiles per segment).
  struct Cursor {
    int b, sib, t, Tb, L, L_in;
    long long C;
  };
  Cursor cur;
  cur.C = locate(lens, batch, cap, segs, x0, lane, &cur.b);
  if (cur.b >= batch) return;  // not reached: x0 < T
  cur.L_in = __builtin_amdgcn_readfirstlane(lens[cur.b]);
  cur.L = min(cur.L_in, cap);
  cur.Tb = seq_tiles(cur.L_in, cap);
  if (cur.Tb == 0) return;  // not reached: the located sequence holds tile x0
  {
    const long long r = x0 - cur.C;
    cur.sib = (int)(r / cur.Tb);
    cur.t = (int)(r % cur.Tb);
  }
  auto advance = [&](Cursor c) -> Cursor {
    if (++c.t < c.Tb) return c;
    c.t = 0;
    if (++c.sib < segs) return c;
    c.sib = 0;
    c.C += (long long)c.Tb * segs;
    do {  // next sequence with tiles (one exists: the caller stays below x1 <= T)
      ++c.b;
      c.L_in = __builtin_amdgcn_readfirstlane(lens[c.b]);
      c.L = min(c.L_in, cap);
      c.Tb = seq_tiles(c.L_in, cap);
    } while (c.Tb == 0 && c.b + 1 < batch);
    return c;
  };

  // Block ids of 64 consecutive blocks of one sequence sit in one VGPR, one per lane.
  int id_b = -1, id_chunk = -1, ids = -1;
  auto block_of = [&](const Cursor& c) -> int {
    const int blk = c.t / TPB;
    const int c64 = blk >> 6;
    if (c.b != id_b || c64 != id_chunk) {
      id_b = c.b;
      id_chunk = c64;
      const int idx = (c64 << 6) + lane;
      ids = idx < d.max_blocks_per_seq ? d.block_tables[(size_t)c.b * d.max_blocks_per_seq + idx] : -1;
    }
    return __builtin_amdgcn_readlane(ids, blk & 63);
  };
  auto valid = [&](int blk) { return blk >= 0 && blk < d.num_blocks; };
  auto appending = [&](const Cursor& c) { return d.k_new != nullptr && c.L_in >= 1 && c.L_in == c.L; };
  auto load = [&](const Cursor& c, int blk, uint4 (&kr)[KK], uint4 (&vr)[VL]) {
    const int g = c.sib / chunks;
    const size_t row0 = ((size_t)blk * Hkv + g) * BS + (c.t % TPB) * 16;
    const size_t new_row = ((size_t)c.b * Hkv + g) * ROW16;
    const int new_tok = appending(c) ? c.L - 1 - 16 * c.t : -1;
    TA::load_tile(d.k_cache + row0 * ROW16, d.v_cache + row0 * ROW16, new_tok, d.k_new + new_row,
                  d.v_new + new_row, lane, kr, vr);
  };

  TA st;
  auto start_piece = [&](const Cursor& c) {
    st.reset();
    const int g = c.sib / chunks, ch = c.sib % chunks;
    st.load_q(d.q, (size_t)c.b * d.num_q_heads + g * d.group + ch * GC, lane);
    // The append of (b, g): done by the worker holding the segment's last tile, chunk 0.
    if (appending(c) && ch == 0 && lane < 2 * ROW16) {
      const long long seg_last = c.C + (long long)c.sib * c.Tb + c.Tb - 1;
      const long long here = c.C + (long long)c.sib * c.Tb + c.t;
      if (seg_last >= here && seg_last < x1) {
        const int last = c.L - 1;
        const int blk = d.block_tables[(size_t)c.b * d.max_blocks_per_seq + last / BS];
        if (valid(blk)) {
          const size_t dst = (((size_t)blk * Hkv + g) * BS + last % BS) * ROW16;
          const size_t src = ((size_t)c.b * Hkv + g) * ROW16;
          if (lane < ROW16)
            d.k_cache_w[dst + lane] = d.k_new[src + lane];
          else
            d.v_cache_w[dst + lane - ROW16] = d.v_new[src + lane - ROW16];
        }
      }
    }
  };
  auto finish_piece = [&](const Cursor& c) {
    float m_h[HP * 4], l_h[HP * 4];
    st.head_stats(m_h, l_h);
    const int g = c.sib / chunks, ch = c.sib % chunks;
    const size_t q_row0 = (size_t)c.b * d.num_q_heads + g * d.group + ch * GC;
    const long long seg_start = c.C + (long long)c.sib * c.Tb;
    const bool whole = worker_of(seg_start, weff, T) == worker_of(seg_start + c.Tb - 1, weff, T);
    const size_t slot = (size_t)(c.b * segs + c.sib) + w;
#pragma unroll
    for (int r = 0; r < GC; ++r) {
      const int hp = r / 4, i = r % 4;
      const float inv = l_h[r] > 0.f ? 1.f / l_h[r] : 0.f;
      if (whole) {
        uint16_t* o = reinterpret_cast<uint16_t*>(d.out) + (q_row0 + r) * D;
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) o[64 * hf + lane] = (uint16_t)f32_to_bf16_rne(st.acc[hp * NH + hf][i] * inv);
      } else {
        const size_t row = slot * GC + r;
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) prm.ws_o[row * D + 64 * hf + lane] = st.acc[hp * NH + hf][i] * inv;
        if (lane == 0) {
          prm.ws_m[row] = m_h[r] == kNegInf ? kNegInf : m_h[r] * kLn2;
          prm.ws_l[row] = l_h[r];
        }
      }
    }
  };

  uint4 kA[KK], vA[VL], kB[KK], vB[VL];
  int bA = block_of(cur);
  if (valid(bA)) load(cur, bA, kA, vA);
  start_piece(cur);
  long long x = x0;
  // One tile of the range: prefetch the next one into the other register set, process this one,
  // and close the piece when the segment or the range ends.
  auto step = [&](uint4 (&kc)[KK], uint4 (&vc)[VL], int bc, uint4 (&kn)[KK], uint4 (&vn)[VL], int& bn,
                  Cursor& nxt) -> bool {
    const bool more = x + 1 < x1;
    if (more) {
      nxt = advance(cur);
      bn = block_of(nxt);
      if (valid(bn)) load(nxt, bn, kn, vn);
    }
    if (valid(bc)) st.process(kc, vc, min(16, cur.L - 16 * cur.t), vlds, d.scale_log2e, lane);
    const bool new_seg = !more || nxt.b != cur.b || nxt.sib != cur.sib;
    if (new_seg) {
      finish_piece(cur);
      if (more) start_piece(nxt);
    }
    ++x;
    if (more) cur = nxt;
    return more;
  };
  Cursor nxt = cur;
  int bB = -1;
  while (true) {
    if (!step(kA, vA, bA, kB, vB, bB, nxt)) break;
    if (!step(kB, vB, bB, kA, vA, bA, nxt)) break;
  }
}

// Merges the pieces of each (sequence, head) row that the decode kernel did not finish itself.
template <int D>
__global__ __launch_bounds__(64) void balanced_merge_kernel(const BalancedParams prm) {
  constexpr int DPL = D / 64;
  const DecodeParams& d = prm.d;
  const int lane = threadIdx.x;
  const int row = blockIdx.x;  // b * Hq + h
  const int b = row / d.num_q_heads, h = row % d.num_q_heads;
  const int batch = prm.batch;
  const int segs = d.num_kv_heads * d.chunks;
  const int cap = d.max_blocks_per_seq * prm.block_size;
  const int Tb = seq_tiles(d.context_lens[b], cap);
  if (Tb == 0) return;  // zeros were written by the decode kernel
  const long long T = total_tiles(d.context_lens, batch, cap, segs, lane);
  const int weff = (int)min((long long)prm.workers, max(1LL, (T + prm.min_tiles - 1) / prm.min_tiles));
  // Tiles before sequence b.
  long long C = 0;
  for (int b0 = 0; b0 < b; b0 += 64) {
    const int bb = b0 + lane;
    C += bb < b ? (long long)seq_tiles(d.context_lens[bb], cap) * segs : 0;
  }
  C = wave_sum(C);
  const int gc = d.group / d.chunks;  // heads per segment
  const int g = h / d.group, ch = (h % d.group) / gc, r = h % gc;
  const int sib = g * d.chunks + ch;
  const long long seg_start = C + (long long)sib * Tb;
  const int wf = worker_of(seg_start, weff, T);
  const int wl = worker_of(seg_start + Tb - 1, weff, T);
  if (wf == wl) return;  // finished inside one worker
  const int n = wl - wf + 1;
  // Piece k of the segment lives in slot s + wf + k, row slot * gc + r.
  const size_t row0 = ((size_t)(b * segs + sib) + wf) * gc + r;
  auto piece_row = [&](int k) { return row0 + (size_t)k * gc; };
  float M = -INFINITY;
  for (int k = lane; k < n; k += 64) M = fmaxf(M, prm.ws_m[piece_row(k)]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  float W = 0.f;
  if (M != -INFINITY) {
    const float M2 = M * kLog2e;
    for (int base = 0; base < n; base += 64) {
      const int kk = base + lane;
      const float wgt = kk < n ? prm.ws_l[piece_row(kk)] * fast_exp2(fmaf(prm.ws_m[piece_row(kk)], kLog2e, -M2)) : 0.f;
      W += wgt;
      const int cnt = min(64, n - base);
      int k = 0;
      for (; k + 8 <= cnt; k += 8) {
        float o[8][DPL];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
#pragma unroll
          for (int e = 0; e < DPL; ++e) o[u][e] = prm.ws_o[piece_row(base + k + u) * D + lane * DPL + e];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), k + u));
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[e] = fmaf(wk, o[u][e], acc[e]);
        }
      }
      for (; k < cnt; ++k) {
        const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), k));
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] = fmaf(wk, prm.ws_o[piece_row(base + k) * D + lane * DPL + e], acc[e]);
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) W += __shfl_xor(W, off, 64);
  const float inv = W > 0.f ? 1.f / W : 0.f;
  if constexpr (DPL == 2) {
    reinterpret_cast<uint32_t*>(d.out)[(size_t)row * (D / 2) + lane] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  } else {
    reinterpret_cast<uint16_t*>(d.out)[(size_t)row * D + lane] = (uint16_t)f32_to_bf16_rne(acc[0] * inv);
  }
}

constexpr int kMinTilesPerWorker = 16;

// Workers that the device keeps resident for this kernel instance: occupancy x CUs x waves per group.
template <int D, int BS, int GC>
int resident_workers() {
  static std::atomic<int> cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64) {
    const int known = cache[dev].load(std::memory_order_relaxed);
    if (known > 0) return known;
  }
  int groups_per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&groups_per_cu, paged_decode_balanced_kernel<D, BS, GC>,
                                                   64 * kWavesPerGroup, 0) != hipSuccess ||
      groups_per_cu < 1)
    groups_per_cu = 1;
  const int w = groups_per_cu * kWavesPerGroup * device_cu_count();
  if (dev < 64) cache[dev].store(w, std::memory_order_relaxed);
  return w;
}

template <int D, int BS, int GC>
hipError_t launch_t(BalancedParams prm, int batch, int num_q_heads, hipStream_t stream) {
  prm.workers = std::min(prm.workers, resident_workers<D, BS, GC>());
  const unsigned groups = (unsigned)((prm.workers + kWavesPerGroup - 1) / kWavesPerGroup);
  hipLaunchKernelGGL((paged_decode_balanced_kernel<D, BS, GC>), dim3(groups), dim3(64 * kWavesPerGroup), 0, stream,
                     prm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((balanced_merge_kernel<D>), dim3((unsigned)((long long)batch * num_q_heads)), dim3(64), 0, stream,
                     prm);
  return hipGetLastError();
}

template <int D, int BS>
hipError_t launch_gc(int gc, const BalancedParams& prm, int batch, int hq, hipStream_t s) {
  switch (gc) {
    case 1: return launch_t<D, BS, 1>(prm, batch, hq, s);
    case 2: return launch_t<D, BS, 2>(prm, batch, hq, s);
    case 4: return launch_t<D, BS, 4>(prm, batch, hq, s);
    case 8: return launch_t<D, BS, 8>(prm, batch, hq, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Upper bound on the workers of any instance: 4 wavefronts per SIMD, 4 SIMDs per CU.
int balanced_workers() { return 16 * device_cu_count(); }

size_t balanced_workspace_bytes(int batch, int num_q_heads, int num_kv_heads, int head_dim, int workers) {
  const int gc = heads_per_chunk(num_q_heads / num_kv_heads);
  const size_t rows = (size_t)batch * num_q_heads + (size_t)workers * gc;
  return rows * ((size_t)head_dim + 2) * sizeof(float);
}

bool balanced_supported(bool bf16, int head_dim, int block_size) {
  return mfma_decode_supported(bf16, head_dim, block_size);
}

hipError_t launch_paged_decode_balanced(const DecodeArgs& a, void* workspace, int workers, hipStream_t stream) {
  const int gc = heads_per_chunk(a.num_q_heads / a.num_kv_heads);
  BalancedParams prm;
  prm.d = make_params(a, gc);
  prm.block_size = a.block_size;
  const size_t rows = (size_t)a.batch * a.num_q_heads + (size_t)workers * gc;
  prm.ws_o = static_cast<float*>(workspace);
  prm.ws_m = prm.ws_o + rows * a.head_dim;
  prm.ws_l = prm.ws_m + rows;
  prm.batch = a.batch;
  prm.workers = workers;
  prm.min_tiles = kMinTilesPerWorker;
  if (a.head_dim == 128 && a.block_size == 16) return launch_gc<128, 16>(gc, prm, a.batch, a.num_q_heads, stream);
  if (a.head_dim == 128 && a.block_size == 32) return launch_gc<128, 32>(gc, prm, a.batch, a.num_q_heads, stream);
  if (a.head_dim == 64 && a.block_size == 16) return launch_gc<64, 16>(gc, prm, a.batch, a.num_q_heads, stream);
  if (a.head_dim == 64 && a.block_size == 32) return launch_gc<64, 32>(gc, prm, a.batch, a.num_q_heads, stream);
  return hipErrorInvalidValue;
}

}  // namespace xs
