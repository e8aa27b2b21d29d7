// Chunked prefill over the paged pool: the multi-token append, and causal GQA attention of a
// chunk of query positions against everything cached for the sequence.
//
// xserv compare phase10...cf1e9e41, attention.rs: `reshape_and_cache_bf16` writes a run of
// num_tokens K/V rows of one sequence starting at position start_pos (token i goes to position
// start_pos + i, through the block table); `flash_attention(q, k, v, causal)` is the prefill
// attention with native GQA. Here a chunk row i of sequence b sits at position p = start_pos[b] + i
// and sees the keys at positions 0..p (the causal mask aligned to the end of the cached range).
//
// Attention kernel. A workgroup of four wavefronts owns 64 consecutive "rows" of one
// (sequence, kv head): row rho = i * G + r is chunk position i of query head g * G + r (G query
// heads per kv head), so one K/V tile in LDS serves every head of the group. Each wavefront
// owns 16 rows (one per lane column) and walks the 32-token key tiles up to its last row's
// position:
//   scores  S^T[32 tokens x 16 rows] as two v_mfma_f32_16x16x32_bf16, half h taking the tokens
//           2m + h (m = 0..15). Lane l then holds the scores of tokens 8(l/16) .. 8(l/16)+7 of
//           row l%16: the row max and sum are a reduction over the lane's 8 values and the
//           four lanes l%16 + 16j. The accumulator rescale is per lane.
//   P.V     O^T[D x 16 rows] += V^T[D x 32] . P^T[32 x 16] with v_mfma_f32_16x16x32_bf16, D/16
//           of them. The B operand (P^T, rounded to bf16) is exactly what the score MFMAs left
//           in each lane. The A operand needs 8 tokens of one d per lane, so V is staged in
//           LDS transposed ([d][token], 64 bytes per d row, 16-byte slots XOR-swizzled by d)
//           and read back 16 bytes at a time.
// The next tile is loaded into registers while the current one is processed (double-buffered
// LDS, one barrier per tile). Tokens past the causal limit of a row get score -inf; tiles past
// the workgroup's last position are never loaded, and K/V of positions past it are zero.
#include <math.h>

#include "xs_internal.h"
#include "xs_mfma_tile.h"

namespace xs {
namespace {

// ---------------------------------------------------------------------------------------------
// Multi-token append: one thread per 16-byte piece of one K or V row (a bit copy).

__global__ __launch_bounds__(256) void kv_append_chunk_kernel(const uint4* __restrict__ k_src,
                                                              const uint4* __restrict__ v_src, uint4* __restrict__ k_cache,
                                                              uint4* __restrict__ v_cache,
                                                              const int32_t* __restrict__ block_tables,
                                                              const int32_t* __restrict__ start_pos,
                                                              const int32_t* __restrict__ chunk_lens, int batch,
                                                              int num_kv_heads, int chunk, int pieces_per_row,
                                                              int block_size, int max_blocks_per_seq, int num_blocks) {
  // Thread index -> (K or V, b, g, i, piece), source-contiguous.
  const long long per_seq = (long long)num_kv_heads * chunk * pieces_per_row;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= 2 * (long long)batch * per_seq) return;
  const bool is_v = idx >= (long long)batch * per_seq;
  const long long src = is_v ? idx - (long long)batch * per_seq : idx;
  const int b = (int)(src / per_seq);
  const int i = (int)((src / pieces_per_row) % chunk);
  const int g = (int)((src / ((long long)chunk * pieces_per_row)) % num_kv_heads);
  const int piece = (int)(src % pieces_per_row);
  const int s0 = start_pos[b], n = chunk_lens[b];
  if (s0 < 0 || n < 0 || n > chunk || (long long)s0 + n > (long long)max_blocks_per_seq * block_size) return;
  if (i >= n) return;
  const int pos = s0 + i;
  const int blk = block_tables[(long long)b * max_blocks_per_seq + pos / block_size];
  if (blk < 0 || blk >= num_blocks) return;
  const long long dst = (((long long)blk * num_kv_heads + g) * block_size + pos % block_size) * pieces_per_row + piece;
  if (is_v)
    v_cache[dst] = v_src[src];
  else
    k_cache[dst] = k_src[src];
}

// ---------------------------------------------------------------------------------------------
// Prefill attention.

struct PrefillParams {
  const uint4* q;
  const uint4* k_cache;
  const uint4* v_cache;
  const int32_t* block_tables;
  const int32_t* start_pos;
  const int32_t* chunk_lens;
  uint4* out;
  float scale_log2e;
  int batch, num_q_heads, num_kv_heads, group, chunk, row_blocks, bs_log2, max_blocks_per_seq, num_blocks;
};

constexpr int kTileTokens = 32;
constexpr int kRowsPerWave = 16;
constexpr int kWaves = 4;
constexpr int kRowsPerGroup = kRowsPerWave * kWaves;

template <int D>
struct PrefillLds {
  static constexpr int ND = D / 8;                       // 16-byte pieces per token row
  static constexpr int K_STRIDE = 2 * D + 16;            // padded K row (bytes)
  static constexpr int K_BYTES = kTileTokens * K_STRIDE;
  static constexpr int VT_STRIDE = 2 * kTileTokens;      // one d row of V^T (bytes)
  static constexpr int VT_BYTES = D * VT_STRIDE;
  static constexpr int BUF_BYTES = K_BYTES + VT_BYTES;
  static constexpr int LOADS = kTileTokens * ND / (64 * kWaves);  // 16-byte pieces per thread per tile
};

// LDS row of token t in the K tile: score half h = t % 2 reads rows 16h .. 16h+15 in order.
__device__ __forceinline__ int k_row(int t) { return 16 * (t & 1) + (t >> 1); }
// Column of token t in a V^T row: lane group j's 16-byte slot j holds tokens 8j .. 8j+7 in the
// order of its score registers (element 4h + i is token 8j + 2i + h).
__device__ __forceinline__ int vt_col(int t) { return 8 * (t >> 3) + 4 * (t & 1) + ((t & 7) >> 1); }
// Slot swizzle of V^T row d: conflict-free 16-byte reads of 8 consecutive d rows.
__device__ __forceinline__ int vt_swz(int d) { return ((d >> 1) ^ (d >> 3)) & 3; }

template <int D>
__global__ __launch_bounds__(256) void paged_prefill_kernel(PrefillParams prm) {
  using LD = PrefillLds<D>;
  constexpr int ND = LD::ND;
  constexpr int KK = D / 32;
  constexpr int MD = D / 16;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * LD::BUF_BYTES];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int j = lane >> 4, c = lane & 15;

  // Workgroup -> (row block, sequence, kv head); the last row blocks (most keys) go first, and
  // the workgroups of one (sequence, kv head) share blockIdx.x mod 8 (one XCD's L2) when the
  // number of pairs is a multiple of 8.
  const int pairs = prm.batch * prm.num_kv_heads;
  const int rb = prm.row_blocks - 1 - (int)(blockIdx.x / (unsigned)pairs);
  const int pair = (int)(blockIdx.x % (unsigned)pairs);
  const int g = pair % prm.num_kv_heads;
  const int b = pair / prm.num_kv_heads;
  const int G = prm.group;
  const int C = prm.chunk;
  const int BS = 1 << prm.bs_log2;

  int s0 = prm.start_pos[b], n = prm.chunk_lens[b];
  if (s0 < 0 || n < 0 || n > C || (long long)s0 + n > (long long)prm.max_blocks_per_seq * BS) {
    s0 = 0;
    n = 0;  // a sequence with an invalid range gets zero rows
  }
  const int rows_total = C * G;
  const int rho0_wg = rb * kRowsPerGroup;
  const int rho0 = rho0_wg + wave * kRowsPerWave;

  // This lane's row (column of the score tile).
  const int rho = rho0 + c;
  const int i_c = rho / G;
  const int h_c = g * G + rho % G;
  const bool row_exists = rho < rows_total;
  const bool row_valid = row_exists && i_c < n;
  const int pos_c = s0 + i_c;  // last key position of this row
  const size_t out_row = ((size_t)b * prm.num_q_heads + h_c) * C + i_c;

  // Last valid chunk position of the workgroup and of this wavefront.
  const int i_hi_wg = min((min(rho0_wg + kRowsPerGroup, rows_total) - 1) / G, n - 1);
  const int i_lo_wave = rho0 / G;
  const int i_hi_wave = min((min(rho0 + kRowsPerWave, rows_total) - 1) / G, n - 1);
  const bool wave_active = rho0 < rows_total && i_lo_wave < n;
  const int ntiles = i_hi_wg >= rho0_wg / G ? (s0 + i_hi_wg) / kTileTokens + 1 : 0;
  const int wave_tiles = wave_active ? (s0 + i_hi_wave) / kTileTokens + 1 : 0;
  const int kmax = s0 + i_hi_wg;  // last key position any row of the workgroup reads

  float4_t acc[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) acc[md] = float4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;

  if (ntiles > 0) {
    const int32_t* bt = prm.block_tables + (size_t)b * prm.max_blocks_per_seq;
    const int Hkv = prm.num_kv_heads;
    auto block_ok = [&](int blk) { return blk >= 0 && blk < prm.num_blocks; };

    // B operand of the scores: q[row][32kk + 8j .. +8].
    uint4 qop[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qop[kk] = row_valid ? prm.q[out_row * ND + 4 * kk + j] : make_uint4(0, 0, 0, 0);

    // Loader: piece r of this thread is token 16*th + c of the tile, 16-byte piece 4*dq + j.
    uint4 kr[LD::LOADS], vr[LD::LOADS];
    auto load_tile = [&](int tile) {
#pragma unroll
      for (int r = 0; r < LD::LOADS; ++r) {
        const int u = 4 * r + wave;
        const int t = 16 * (u & 1) + c, dp = 4 * (u >> 1) + j;
        const int pos = tile * kTileTokens + t;
        // Unconditional loads (a branch around them would make the compiler wait for all
        // loads in flight): positions past kmax and bad block ids read row 0 and become zeros.
        const bool in_range = pos <= kmax;
        const int blk = bt[in_range ? pos >> prm.bs_log2 : 0];
        const bool ok = in_range && block_ok(blk);
        const size_t row = ok ? ((size_t)blk * Hkv + g) * BS + (pos & (BS - 1)) : 0;
        const uint4 kv = prm.k_cache[row * ND + dp];
        const uint4 vv = prm.v_cache[row * ND + dp];
        const uint4 z = make_uint4(0, 0, 0, 0);
        kr[r] = ok ? kv : z;
        vr[r] = ok ? vv : z;
      }
    };
    auto store_tile = [&](int buf) {
      unsigned char* kl = lds + buf * LD::BUF_BYTES;
      unsigned char* vl = kl + LD::K_BYTES;
#pragma unroll
      for (int r = 0; r < LD::LOADS; ++r) {
        const int u = 4 * r + wave;
        const int t = 16 * (u & 1) + c, dp = 4 * (u >> 1) + j;
        *reinterpret_cast<uint4*>(kl + k_row(t) * LD::K_STRIDE + 16 * dp) = kr[r];
        const int col = vt_col(t);
        const uint32_t w[4] = {vr[r].x, vr[r].y, vr[r].z, vr[r].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = 8 * dp + e;
          const int off = d * LD::VT_STRIDE + 16 * ((col >> 3) ^ vt_swz(d)) + 2 * (col & 7);
          *reinterpret_cast<uint16_t*>(vl + off) = (uint16_t)(e & 1 ? w[e >> 1] >> 16 : w[e >> 1] & 0xffffu);
        }
      }
    };
    // Block id of the lane's 8 score tokens (8-aligned, so one block for block_size >= 8).
    auto lane_block = [&](int tile) {
      const int pos = tile * kTileTokens + 8 * j;
      const int blk = bt[pos <= kmax ? pos >> prm.bs_log2 : 0];
      return pos <= kmax ? blk : -1;
    };

    load_tile(0);
    int lb = lane_block(0);
    store_tile(0);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
      const int buf = it & 1;
      const bool has_next = it + 1 < ntiles;
      int lb_next = -1;
      if (has_next) {
        load_tile(it + 1);
        lb_next = lane_block(it + 1);
      }
      if (it < wave_tiles) {
        const unsigned char* kl = lds + buf * LD::BUF_BYTES;
        const unsigned char* vl = kl + LD::K_BYTES;
        float4_t s[2] = {float4_t{0.f, 0.f, 0.f, 0.f}, float4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint4 ka = *reinterpret_cast<const uint4*>(kl + (16 * h + c) * LD::K_STRIDE + 16 * (4 * kk + j));
            s[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka), as_bf16x8(qop[kk]), s[h], 0, 0, 0);
          }
        }
        // Lane's tokens: 8j + 2i + h of the tile (score s[h][i]).
        const int base = it * kTileTokens + 8 * j;
        const bool blk_ok = block_ok(lb);
        float sc[2][4];
        float mt = -INFINITY;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool ok = row_valid && blk_ok && base + 2 * i + h <= pos_c;
            sc[h][i] = ok ? s[h][i] * prm.scale_log2e : -INFINITY;
            mt = fmaxf(mt, sc[h][i]);
          }
        }
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float m_new = fmaxf(m_run, mt);
        const float ms = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - ms);
        const bool grew = m_new != m_run;
        m_run = m_new;
        bf16x8_t pb;
        float psum = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = fast_exp2(sc[h][i] - ms);
            psum += p;
            pb[4 * h + i] = (__bf16)p;
          }
        }
        l_part = l_part * alpha + psum;
        if (__any(grew)) {
#pragma unroll
          for (int md = 0; md < MD; ++md) acc[md] *= alpha;
        }
#pragma unroll
        for (int md = 0; md < MD; ++md) {
          const int d = 16 * md + c;
          const uint4 va = *reinterpret_cast<const uint4*>(vl + d * LD::VT_STRIDE + 16 * (j ^ vt_swz(d)));
          acc[md] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), pb, acc[md], 0, 0, 0);
        }
      }
      if (has_next) store_tile(buf ^ 1);
      __syncthreads();
      lb = lb_next;
    }
  }

  float l_tot = l_part + __shfl_xor(l_part, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (!row_exists) return;
  const float inv = row_valid && l_tot > 0.f ? 1.f / l_tot : 0.f;
  // acc[md][e] is O[row c][16md + 4j + e].
  uint2* orow = reinterpret_cast<uint2*>(prm.out + out_row * ND);
#pragma unroll
  for (int md = 0; md < MD; ++md) {
    const float4_t o = acc[md] * inv;
    orow[4 * md + j] = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
  }
}

template <int D>
hipError_t launch_prefill_d(const PrefillParams& p, hipStream_t stream) {
  const long long grid = (long long)p.batch * p.num_kv_heads * p.row_blocks;
  hipLaunchKernelGGL(paged_prefill_kernel<D>, dim3((unsigned)grid), dim3(64 * kWaves), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_append_chunk(const void* k_src, const void* v_src, void* k_cache, void* v_cache,
                                  const int32_t* block_tables, const int32_t* start_pos, const int32_t* chunk_lens,
                                  int batch, int num_kv_heads, int head_dim, int chunk, int block_size,
                                  int max_blocks_per_seq, int num_blocks, int elt_bytes, hipStream_t stream) {
  const int pieces_per_row = head_dim * elt_bytes / 16;
  const long long total = 2LL * batch * num_kv_heads * chunk * pieces_per_row;
  const int threads = 256;
  const long long blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(kv_append_chunk_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     static_cast<const uint4*>(k_src), static_cast<const uint4*>(v_src), static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), block_tables, start_pos, chunk_lens, batch, num_kv_heads, chunk,
                     pieces_per_row, block_size, max_blocks_per_seq, num_blocks);
  return hipGetLastError();
}

int prefill_row_blocks(int chunk, int group) { return (int)(((long long)chunk * group + kRowsPerGroup - 1) / kRowsPerGroup); }

hipError_t launch_paged_prefill(const PrefillArgs& a, hipStream_t stream) {
  PrefillParams p;
  p.q = static_cast<const uint4*>(a.q);
  p.k_cache = static_cast<const uint4*>(a.k_cache);
  p.v_cache = static_cast<const uint4*>(a.v_cache);
  p.block_tables = a.block_tables;
  p.start_pos = a.start_pos;
  p.chunk_lens = a.chunk_lens;
  p.out = static_cast<uint4*>(a.out);
  p.scale_log2e = a.scale * kLog2e;
  p.batch = a.batch;
  p.num_q_heads = a.num_q_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.group = a.num_q_heads / a.num_kv_heads;
  p.chunk = a.chunk;
  p.row_blocks = prefill_row_blocks(a.chunk, p.group);
  p.bs_log2 = a.block_size == 8 ? 3 : a.block_size == 16 ? 4 : 5;
  p.max_blocks_per_seq = a.max_blocks_per_seq;
  p.num_blocks = a.num_blocks;
  return a.head_dim == 64 ? launch_prefill_d<64>(p, stream) : launch_prefill_d<128>(p, stream);
}

}  // namespace xs
