// Paged decode attention on the matrix cores (bf16 pools, head_dim 64/128, block_size 16/32).
//
// Same result as the generic kernel in xs_decode.hip (xserv compare phase10...cf1e9e41,
// attention.rs, `paged_decode_attention`; GQA by `repeat_kv` in xserv compare
// phase8...phase13): for the GC query heads of one kv head, over a block range,
//   s_t = scale * q_h . K_t,  m = max s_t,  l = sum exp(s_t - m),  o = sum exp(s_t - m) V_t / l.
//
// A work item (sequence, kv head, head chunk, partition) goes to one workgroup of NW = 1, 2 or 4
// wavefronts, chosen at launch so that the grid fills the GPU. The wavefronts take the item's
// 16-token tiles round-robin, each keeps its own online-softmax state, and they merge through
// LDS at the end (max, rescale, add). Per tile:
//   QK  C[16 tokens x 16] = K_tile[16 x D] . Q^T[D x 16] with v_mfma_f32_16x16x32_bf16 (D/32 of
//       them). The 16 columns hold the GC heads repeated, so lane l ends with the scores of
//       tokens 4(l/16)+i (i = 0..3) for head (l%16) % GC. The A operand (K) needs lane l to hold
//       16 bytes of token l%16, so each K load moves four 64-byte runs per token row.
//   softmax  The running max is kept per head and shared by the whole wavefront: a tile max
//       over the lane's 4 scores, then across the four lane rows. p = 2^(s*log2e*scale - m).
//   PV  O[4 heads x D] += P[4 heads x 4 tokens] . V[4 tokens x D] per group of 4 tokens, with
//       v_mfma_f32_4x4x4_16b_bf16: its 16 blocks each take 4 columns of d, and all of them use
//       the P operand of one block (CBSZ/ABID broadcast). That operand (P, rounded to bf16) is
//       exactly what the QK output left in lanes 16kg..16kg+3. The B operand needs 4 tokens of
//       one d per lane, so V goes through the wavefront's own LDS slice and comes back 2 bytes
//       at a time; lane l reads column d = 64h + l, 128 consecutive bytes per wavefront.
//       The accumulator is O[head][64h + lane]: D/16 registers, and the stores coalesce.
// Tokens at or past L get score -inf and a zeroed V, so pool tails (NaN included) never reach
// the result. K/V are read with nontemporal loads (each byte is used once). Each wavefront
// loads its next tile into a second register set while it processes the current one.
// Fused append (k_new non-null): every wavefront that loads the tile holding token L-1 takes
// that token's K/V from k_new/v_new, and one wavefront writes them into the pools; no
// wavefront reads the slot being written.
#include <math.h>

#include <type_traits>
#include <utility>

#include "xs_device.h"
#include "xs_internal.h"

namespace xs {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef short __attribute__((ext_vector_type(4))) short4_t;
typedef float __attribute__((ext_vector_type(4))) float4_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }

// Calls f(std::integral_constant<int, I>) for I = 0..N-1 (the broadcast block is an immediate).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// 16 blocks of 4x4x4 (bf16 in, fp32 accumulate); every block uses the A operand of block ABID.
template <int ABID>
__device__ __forceinline__ float4_t mfma_4x4x4_bcast(short4_t a, short4_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, b, c, 4, ABID, 0);
}

// Orders LDS traffic between the lanes of one wavefront: LDS executes a wavefront's
// instructions in issue order, so only the compiler must be kept from reordering.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

#ifndef XS_DECODE_MIN_WAVES_PER_EU
#define XS_DECODE_MIN_WAVES_PER_EU 4
#endif

template <int D, int BS, int GC, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(XS_DECODE_MIN_WAVES_PER_EU)))
void paged_decode_mfma_kernel(const DecodeParams prm) {
  constexpr int KK = D / 32;                // QK matrix ops per tile
  constexpr int NH = D / 64;                // 64-wide d halves of the PV output
  constexpr int HP = (GC + 3) / 4;          // PV passes of 4 heads
  constexpr int ROW16 = D / 8;              // 16-byte pieces per token row
  constexpr int VL = 16 * ROW16 / 64;       // V loads per lane per tile
  constexpr int TPB = BS / 16;              // tiles per block
  constexpr int STRIDE = 2 * D;             // LDS bytes per token row
  constexpr int STAGE_BYTES = 16 * STRIDE;  // one wavefront's V tile
  constexpr int ACC = HP * NH;              // 4-float accumulators per lane
  constexpr int MERGE_FLOATS = ACC * 4 * 64 + 2 * GC;  // one wavefront's (acc, m, l)
  constexpr int SMEM = NW * STAGE_BYTES > (NW - 1) * MERGE_FLOATS * 4 ? NW * STAGE_BYTES
                                                                      : (NW - 1) * MERGE_FLOATS * 4;
  constexpr float kNegInf = -INFINITY;
  static_assert(BS % 16 == 0 && (D == 64 || D == 128), "tile shape");
  static_assert(GC == 1 || GC == 2 || GC == 4 || GC == 8, "heads per wavefront");

  __shared__ __align__(16) unsigned char smem[SMEM];

  const int wave = NW > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
  const int lane = threadIdx.x & 63;
  const int j = lane >> 4;  // lane row: tokens 4j..4j+3 of a tile
  const int c = lane & 15;  // column: token of the K operand; head c % GC of the scores
  unsigned char* vlds = smem + wave * STAGE_BYTES;

  const int num_kv_heads = prm.num_kv_heads;
  const int max_blocks_per_seq = prm.max_blocks_per_seq;
  const int max_partitions = prm.max_partitions;
  const bool split = prm.part_blocks > 0;
  const int np = split ? max_partitions : 1;
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
  const int L = min(L_in, max_blocks_per_seq * BS);
  const int nblk_seq = L > 0 ? (L + BS - 1) / BS : 0;
  int jb = 0, je = nblk_seq;
  if (split) {
    jb = p * prm.part_blocks;
    je = min(jb + prm.part_blocks, nblk_seq);
    if (jb >= je) return;  // the whole workgroup leaves together
  }
  const size_t q_row0 = (size_t)b * prm.num_q_heads + h0;
  if (jb >= je) {  // no split, empty context
    if (wave == 0 && lane < GC * ROW16)
      reinterpret_cast<uint4*>(prm.out)[q_row0 * ROW16 + lane] = make_uint4(0, 0, 0, 0);
    return;
  }
  const int32_t* bt = prm.block_tables + (size_t)b * max_blocks_per_seq;
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

  // B operand of QK: lane l holds q[h0 + c%GC][32kk + 8j .. +8].
  uint4 qop[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) qop[kk] = prm.q[(q_row0 + c % GC) * ROW16 + 4 * kk + j];

  // acc[hp*NH + hf][i] = O[head 4hp+i][64hf + lane] (rows past GC repeat lower heads).
  float4_t acc[ACC];
#pragma unroll
  for (int a = 0; a < ACC; ++a) acc[a] = float4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf;  // running max of head c%GC (same in every lane of that head)
  float l_part = 0.f;     // this lane's share of the softmax sum of head c%GC

  // Block ids of 64 consecutive blocks of the range sit in one VGPR, one per lane.
  int id_chunk = -1, ids = -1;
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

  // Tile loads. K: token c of the tile, pieces 4kk + j. V: pieces r*64 + lane of the tile.
  auto load_tile = [&](int blk, int tile, uint4 (&kr)[KK], uint4 (&vr)[VL]) {
    const size_t row0 = ((size_t)blk * num_kv_heads + g) * BS + (tile % TPB) * 16;
    const int tok0 = 16 * tile;
    const uint4* ks = tok0 + c == last ? prm.k_new + new_row : prm.k_cache + (row0 + c) * ROW16;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) kr[kk] = load_stream(ks + 4 * kk + j);
#pragma unroll
    for (int r = 0; r < VL; ++r) {
      const int piece = r * 64 + lane;
      const uint4* vs = tok0 + piece / ROW16 == last ? prm.v_new + new_row + piece % ROW16
                                                     : prm.v_cache + row0 * ROW16 + piece;
      vr[r] = load_stream(vs);
    }
  };

  auto process = [&](const uint4 (&kr)[KK], const uint4 (&vr)[VL], int nvalid) {
    // Stage V in LDS (rows of 2D bytes); tokens at or past nvalid become zeros.
#pragma unroll
    for (int r = 0; r < VL; ++r) {
      const int piece = r * 64 + lane;
      uint4 v = vr[r];
      if (piece / ROW16 >= nvalid) v = make_uint4(0, 0, 0, 0);
      reinterpret_cast<uint4*>(vlds)[piece] = v;
    }
    // QK on the matrix cores.
    float4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[kk]), as_bf16x8(qop[kk]), s, 0, 0, 0);
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = s[i] * prm.scale_log2e;
      if (4 * j + i >= nvalid) sc[i] = kNegInf;
    }
    float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float ms = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - ms);
    const bool grew = m_new != m_run;
    m_run = m_new;
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(sc[i] - ms);
    l_part = l_part * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    // Rescale when some head's max moved (a wave-uniform decision). Row i of PV pass hp is the
    // head of lane 4hp+i, whose alpha every lane reads as a scalar.
    if (__any(grew)) {
#pragma unroll
      for (int hp = 0; hp < HP; ++hp) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 4 * hp + i));
#pragma unroll
          for (int hf = 0; hf < NH; ++hf) acc[hp * NH + hf][i] *= a;
        }
      }
    }
    // A operand of PV: lane 16kg + 4hp + i holds P[head 4hp+i][tokens 4kg..4kg+3] as bf16;
    // the instruction broadcasts block 4kg+hp (lanes 16kg+4hp .. +3) to all 16 blocks.
    short4_t pa;
#pragma unroll
    for (int i = 0; i < 4; ++i) pa[i] = __builtin_bit_cast(short, (__bf16)pr[i]);
    wave_lds_fence();
    // B operand of PV: block b, column x holds V[tokens 4kg..4kg+3][64hf + 4b + x], i.e. lane l
    // reads the 4 tokens at d = 64hf + l.
    static_for<4>([&](auto kg_c) {
      constexpr int kg = decltype(kg_c)::value;
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        short4_t vb;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          vb[k] = *reinterpret_cast<const short*>(vlds + (4 * kg + k) * STRIDE + (64 * hf + lane) * 2);
        static_for<HP>([&](auto hp_c) {
          constexpr int hp = decltype(hp_c)::value;
          acc[hp * NH + hf] = mfma_4x4x4_bcast<4 * kg + hp>(pa, vb, acc[hp * NH + hf]);
        });
      }
    });
    wave_lds_fence();
  };

  // Tiles of the range, dealt round-robin to the NW wavefronts; the next tile of a wavefront is
  // loaded (into the other register set) while the current one is processed.
  const int t_end = (min(je * BS, L) + 15) / 16;
  int t = jb * TPB + wave;
  uint4 kA[KK], vA[VL], kB[KK], vB[VL];
  int bA = -1, bB = -1;
  if (t < t_end) {
    bA = block_of(t);
    if (valid(bA)) load_tile(bA, t, kA, vA);
  }
  while (t < t_end) {
    const int t2 = t + NW;
    if (t2 < t_end) {
      bB = block_of(t2);
      if (valid(bB)) load_tile(bB, t2, kB, vB);
    }
    if (valid(bA)) process(kA, vA, min(16, L - 16 * t));
    if (t2 >= t_end) break;
    const int t3 = t2 + NW;
    if (t3 < t_end) {
      bA = block_of(t3);
      if (valid(bA)) load_tile(bA, t3, kA, vA);
    }
    if (valid(bB)) process(kB, vB, min(16, L - 16 * t2));
    t = t3;
  }

  // Softmax sum per head over this wavefront's tokens: add the four lane rows.
  float l_tot = l_part + __shfl_xor(l_part, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);

  // Per-head (m, l) of this wavefront, as scalars: head of lane x is x % GC.
  float m_h[HP * 4], l_h[HP * 4];
#pragma unroll
  for (int r = 0; r < HP * 4; ++r) {
    m_h[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_run), r));
    l_h[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l_tot), r));
  }

  if constexpr (NW > 1) {
    // Merge the NW wavefront states through LDS, once every wavefront is done with its staging.
    float* mrg = reinterpret_cast<float*>(smem);
    __syncthreads();
    if (wave > 0) {
      float* mine = mrg + (wave - 1) * MERGE_FLOATS;
#pragma unroll
      for (int a = 0; a < ACC; ++a) {
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[(a * 4 + i) * 64 + lane] = acc[a][i];
      }
      if (lane < GC) {
        mine[ACC * 4 * 64 + lane] = m_run;
        mine[ACC * 4 * 64 + GC + lane] = l_tot;
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
      for (int hf = 0; hf < NH; ++hf) acc[hp * NH + hf][i] *= f0;
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        const float* other = mrg + (w - 1) * MERGE_FLOATS;
        const float fw = fast_exp2(other[ACC * 4 * 64 + hr] - Ms);
        lsum += other[ACC * 4 * 64 + GC + hr] * fw;
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) acc[hp * NH + hf][i] += other[((hp * NH + hf) * 4 + i) * 64 + lane] * fw;
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
      for (int hf = 0; hf < NH; ++hf) po[64 * hf + lane] = acc[hp * NH + hf][i] * inv;
      if (lane == 0) {
        prm.part_m[prow] = m_h[r] == kNegInf ? kNegInf : m_h[r] * kLn2;
        prm.part_l[prow] = l_h[r];
      }
    } else {
      uint16_t* o = reinterpret_cast<uint16_t*>(prm.out) + (q_row0 + r) * D;
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) o[64 * hf + lane] = (uint16_t)f32_to_bf16_rne(acc[hp * NH + hf][i] * inv);
    }
  }
}

template <int D, int BS, int GC>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const DecodeParams prm = make_params(a, GC);
  const long long np = prm.part_blocks > 0 ? a.max_partitions : 1;
  const long long grid = (long long)a.batch * a.num_kv_heads * prm.chunks * np;
  // Wavefronts per work item: the most that keep the whole grid resident at once (4 per SIMD),
  // or 4 when the grid needs several rounds anyway (finer pieces even out the last round).
  const long long resident = 16LL * device_cu_count();
  int nw = 4;
  if (grid <= resident) nw = grid * 4 <= resident ? 4 : grid * 2 <= resident ? 2 : 1;
  const dim3 g3((unsigned)grid);
  switch (nw) {
    case 1: hipLaunchKernelGGL((paged_decode_mfma_kernel<D, BS, GC, 1>), g3, dim3(64), 0, stream, prm); break;
    case 2: hipLaunchKernelGGL((paged_decode_mfma_kernel<D, BS, GC, 2>), g3, dim3(128), 0, stream, prm); break;
    default: hipLaunchKernelGGL((paged_decode_mfma_kernel<D, BS, GC, 4>), g3, dim3(256), 0, stream, prm); break;
  }
  return hipGetLastError();
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
