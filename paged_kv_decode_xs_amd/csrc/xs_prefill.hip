// Chunked prefill over the paged pool: the multi-token append, and causal GQA attention of a
// chunk of query positions against everything cached for the sequence.
//
// xserv compare phase10...cf1e9e41, attention.rs: `reshape_and_cache_bf16` writes a run of
// num_tokens K/V rows of one sequence starting at position start_pos (token i goes to position
// start_pos + i, through the block table); `flash_attention(q, k, v, causal)` is the prefill
// attention with native GQA. Here a chunk row i of sequence b sits at position p = start_pos[b] + i
// and sees the keys at positions 0..p (the causal mask aligned to the end of the cached range).
//
// Attention kernel. A workgroup of eight wavefronts owns 256 consecutive "rows" of one
// (sequence, kv head): row rho = i * G + r is chunk position i of query head g * G + r (G query
// heads per kv head), so one K/V tile in LDS serves every head of the group. Each wavefront
// owns 32 rows (one per lane column n = lane % 32) and walks the 64-token key tiles up to its
// last row's position:
//   scores  S^T[64 tokens x 32 rows] = K . Q^T as two independent chains of
//           v_mfma_f32_32x32x16_bf16 (tokens 0-31 and 32-63, D/16 each, q in registers). Lane l
//           then holds 32 scores of row l%32: the row max and sum are a reduction over the
//           lane's values and one lane swap; the accumulator rescale is per lane.
//   P.V     O^T[D x 32 rows] += V^T[D x 16] . P^T[16 x 32] with v_mfma_f32_32x32x16_bf16, four
//           token quarters per 32-wide d block. The B operand (P^T, rounded to bf16) is exactly
//           what the score MFMAs left in each lane. The A operand needs 8 tokens of one d per
//           lane: V is staged in LDS token-major like K and read back with the transposing LDS
//           read (ds_read_b64_tr_b16).
// The next two tiles are loaded into registers while the current one is processed
// (double-buffered LDS, one barrier per tile). Tokens past the causal limit of a row get score
// -inf, and K/V of positions past the workgroup's last key or in a bad block are zero.
// Split-K (partition size P > 0): a workgroup takes one piece of P key positions of its row
// block; a row block with several pieces leaves each row's normalised output over the piece and
// its (max, sum) in the caller's partials, and the merge kernel combines them per row with the
// log-sum-exp identity (the same as the decode's partition merge). The device hands workgroups
// out in id order as CUs free up, so where the sizes differ and the grid is larger than one
// workgroup per CU the ids go to the pieces (or row blocks) largest first: longest-first list
// scheduling.
// SW instances add the sinks and sliding window of the gpt-oss prefill (same diff,
// `flash_attention_sinks`: one sink logit per query head that only enlarges the softmax
// denominator; window_size W > 0 keeps the last W positions up to the query's own). A row at
// position p sees keys max(0, p + 1 - W) .. p: the workgroup starts at the tile of its first
// row's window, each wavefront skips the tiles before its own rows' windows, and the window's
// lower edge joins the causal mask. The sink enters in the epilogue of an unsplit row, and in
// the merge of a split one (pieces carry none).
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
  float* part_o;    // split only: [B, Hq, C, NP, D] f32, each row's output over one piece of keys
  float2* part_ml;  // split only: [B, Hq, C, NP] (m, l) of those pieces (m in scaled log2 units)
  const uint16_t* sinks;  // SW only: [Hq] bf16 sink logits, or null
  int window;             // SW only: W > 0 keeps positions p + 1 - W .. p; 0 keeps 0 .. p
  float scale_log2e;
  int batch, num_q_heads, num_kv_heads, group, chunk, row_blocks, bs_log2, max_blocks_per_seq, num_blocks;
  int part_tiles;      // key tiles per piece (0: each workgroup takes its whole key range)
  int max_partitions;  // NP
  int rank_items;      // 1: workgroups take row blocks / pieces largest first (ranked_piece)
};

typedef float __attribute__((ext_vector_type(16))) float16_t;

constexpr int kTileTokens = 64;
constexpr int kRowsPerWave = 32;
constexpr int kWaves = 8;
constexpr int kRowsPerGroup = kRowsPerWave * kWaves;
constexpr float kRescaleLog2 = 8.f;  // weights stay below 2^8 between rescales

template <int D>
struct PrefillLds {
  static constexpr int ND = D / 8;                       // 16-byte pieces per token row
  static constexpr int K_STRIDE = 2 * D;                 // K row (bytes); pieces XOR-swizzled
  static constexpr int K_BYTES = kTileTokens * K_STRIDE;
  static constexpr int V_BYTES = kTileTokens * K_STRIDE;  // V rows like K rows (own swizzle)
  static constexpr int BUF_BYTES = K_BYTES + V_BYTES;
  static constexpr int LOADS = kTileTokens * ND / (64 * kWaves);  // 16-byte pieces per thread per tile
  static_assert(LOADS * 64 * kWaves == kTileTokens * ND, "loader");
  static_assert(2 * BUF_BYTES <= 65536, "LDS");
};

// (x in this lane, x in lane l ^ 32), in either order: one v_permlane32_swap, no LDS.
__device__ __forceinline__ float2 with_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ uint4 mask4(const uint4 v, uint32_t m) {
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

// 16-byte piece p of K row t sits at slot p ^ s(t). The LDS serves a 16-byte access of 16 lanes at a time from its 64 banks: the 16 rows that 16
// lanes read (or write) at one piece must land on 16 different 16-byte bank groups. With 256-byte
// rows (D = 128) every row starts at bank 0, so the piece is XORed with t % 16; with 128-byte
// rows (D = 64) rows t and t + 1 share a bank line, so with (t / 2) % 8.
template <int D>
__device__ __forceinline__ int k_off(int t, int p) {
  return t * (2 * D) + 16 * (p ^ (D == 128 ? (t & 15) : ((t >> 1) & 7)));
}
// Score register r of chain h2 and lane half hl holds token 32h2 + 8(r/4) + 4hl + r%4 of the tile.
// V rows are stored like K rows (token-major, 2D bytes), 16-byte piece p of row t at slot
// p ^ v_swz(t): eight consecutive rows written at one piece hit eight bank groups, and the four
// rows of a transposing read (below) hit four different 32-byte ranges.
__device__ __forceinline__ int v_swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes, lane i receives
// element i % 4 of the 8-byte chunks addressed by lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4. With
// lane j of the group addressing row t0 + j/4 at column c0 + 4 (j % 4), lane i receives rows
// t0 .. t0+3 at column c0 + i.
typedef short __attribute__((ext_vector_type(4))) short4_lds_t;
typedef __attribute__((address_space(3))) unsigned char lds_byte;
__device__ __forceinline__ short4_lds_t lds_read_tr16(lds_byte* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_lds_t*)p);
}

// Key tiles of row block rb (256 rows) of sequence b: up to its last valid row's position (0 when
// the row block holds no valid row or the sequence's range is invalid).
__device__ __forceinline__ int row_block_tiles(const PrefillParams& prm, int b, int rb) {
  const int BS = 1 << prm.bs_log2;
  int s0 = prm.start_pos[b], nlen = prm.chunk_lens[b];
  if (s0 < 0 || nlen < 0 || nlen > prm.chunk || (long long)s0 + nlen > (long long)prm.max_blocks_per_seq * BS) return 0;
  const int rows_total = prm.chunk * prm.group;
  const int rho0 = rb * kRowsPerGroup;
  const int i_hi = min((min(rho0 + kRowsPerGroup, rows_total) - 1) / prm.group, nlen - 1);
  return i_hi >= rho0 / prm.group ? (s0 + i_hi) / kTileTokens + 1 : 0;
}

// Item of rank k (per kv head), largest first: with split-K the full pieces (PT tiles) of every
// row block, then each row block's last piece (fewer tiles, or none: a row block without keys
// still has its piece 0, which writes its zero rows) by decreasing size, ties by row block;
// without split-K the row blocks themselves by decreasing size. Row block
// x = b * row_blocks + (row_blocks - 1 - rb). One wavefront holds the row blocks' sizes, 64 to a
// register (up to kRankMax row blocks), and finds the size of rank k by a binary search on
// ballot counts. Sets b = -1 past the last item.
constexpr int kRankMax = 256;
__device__ __forceinline__ void ranked_piece(const PrefillParams& prm, int k, int& b, int& rb, int& piece) {
  const int lane = threadIdx.x & 63;
  const int PT = prm.part_tiles > 0 ? prm.part_tiles : 1 << 24, RBN = prm.row_blocks;
  const int nx = prm.batch * RBN;
  constexpr int kChunks = kRankMax / 64;
  int nfull[kChunks], last[kChunks];  // full pieces; size of the last piece (-1: none)
  int F = 0;
#pragma unroll
  for (int ch = 0; ch < kChunks; ++ch) {
    nfull[ch] = 0;
    last[ch] = -1;
    const int x = 64 * ch + lane;
    if (x < nx) {
      const int nt = row_block_tiles(prm, x / RBN, RBN - 1 - x % RBN);
      nfull[ch] = nt / PT;
      last[ch] = nt % PT != 0 || nt == 0 ? nt % PT : -1;
    }
    int f = nfull[ch];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) f += __shfl_xor(f, off, 64);
    F += f;
  }
  b = -1;
  rb = 0;
  piece = 0;
  int x = -1;
  if (k < F) {
    // The k-th full piece, row block major.
    int base = 0;
#pragma unroll
    for (int ch = 0; ch < kChunks; ++ch) {
      int incl = nfull[ch];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      const unsigned long long hit = __ballot(base + incl > k);
      if (x < 0 && hit) {
        const int first = __builtin_ctzll(hit);
        x = 64 * ch + first;
        piece = k - base - __shfl(incl - nfull[ch], first, 64);
      }
      base += __shfl(incl, 63, 64);
    }
  } else {
    const int r = k - F;
    auto count_ge = [&](int sz) {
      int cnt = 0;
#pragma unroll
      for (int ch = 0; ch < kChunks; ++ch) cnt += __builtin_popcountll(__ballot(last[ch] >= sz));
      return cnt;
    };
    int top = 0;  // largest last-piece size
#pragma unroll
    for (int ch = 0; ch < kChunks; ++ch) top = max(top, last[ch]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) top = max(top, __shfl_xor(top, off, 64));
    if (r < count_ge(0)) {
      int lo = 0, hi = top;  // the size of rank r lies in [lo, hi]
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (count_ge(mid) > r) lo = mid;
        else hi = mid - 1;
      }
      int jth = r - count_ge(lo + 1);
#pragma unroll
      for (int ch = 0; ch < kChunks; ++ch) {
        const unsigned long long m = __ballot(last[ch] == lo);
        const int cnt = __builtin_popcountll(m);
        if (x < 0 && jth < cnt) {
          const unsigned long long below = lane ? m & ((~0ull) >> (64 - lane)) : 0ull;
          const unsigned long long hit = __ballot(((m >> lane) & 1ull) && __builtin_popcountll(below) == jth);
          const int first = __builtin_ctzll(hit);
          x = 64 * ch + first;
          piece = __shfl(nfull[ch], first, 64);
        }
        jth -= cnt;
      }
    }
  }
  if (x >= 0) {
    b = x / RBN;
    rb = RBN - 1 - x % RBN;
  }
  b = __builtin_amdgcn_readfirstlane(b);
  rb = __builtin_amdgcn_readfirstlane(rb);
  piece = __builtin_amdgcn_readfirstlane(piece);
}

template <int D, bool SW>
__global__ __launch_bounds__(64 * kWaves) void paged_prefill_kernel(PrefillParams prm) {
  using LD = PrefillLds<D>;
  constexpr int ND = LD::ND;
  constexpr int KS = D / 16;  // score steps (16 d each)
  constexpr int MD = D / 32;  // 32-wide d blocks of the output
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * LD::BUF_BYTES];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, hl = lane >> 5;  // score column (row of the chunk) and lane half
  const int j = lane >> 4, c = lane & 15;   // loader coordinates

  // Workgroup -> (piece, sequence, row block, kv head), kv head fastest, then row block (the last
  // ones, with the most keys, first), sequence, piece. The device hands workgroup i to XCD i % 8,
  // and within an XCD deals consecutive workgroups to its shader engines in turn, from one
  // in-order queue that waits whenever the next workgroup's engine is full. With this order the
  // engines of an XCD take row blocks of every sequence and piece alike (similar work, no engine
  // holding up the queue), and the workgroups of one kv head share an XCD's L2 when the number of
  // kv heads is a multiple of 8.
  // With rank_items (set by the launcher) the row blocks or split-K pieces go largest first
  // (ranked_piece), kv head still fastest.
  const int Hkv_ = prm.num_kv_heads;
  const int g = (int)(blockIdx.x % (unsigned)Hkv_);
  const int r1 = (int)(blockIdx.x / (unsigned)Hkv_);
  int rb, b, piece;
  if (prm.rank_items) {
    ranked_piece(prm, r1, b, rb, piece);
    if (b < 0) return;
  } else {
    rb = prm.row_blocks - 1 - r1 % prm.row_blocks;
    const int r2 = r1 / prm.row_blocks;
    b = r2 % prm.batch;
    piece = r2 / prm.batch;
  }
  const int G = prm.group;
  const int C = prm.chunk;
  const int BS = 1 << prm.bs_log2;

  int s0 = prm.start_pos[b], nlen = prm.chunk_lens[b];
  if (s0 < 0 || nlen < 0 || nlen > C || (long long)s0 + nlen > (long long)prm.max_blocks_per_seq * BS) {
    s0 = 0;
    nlen = 0;  // a sequence with an invalid range gets zero rows
  }
  const int rows_total = C * G;
  const int rho0_wg = rb * kRowsPerGroup;
  const int rho0 = rho0_wg + wave * kRowsPerWave;

  // This lane's row (column n of the score tile).
  const int rho = rho0 + n;
  const int i_c = rho / G;
  const int h_c = g * G + rho % G;
  const bool row_exists = rho < rows_total;
  const bool row_valid = row_exists && i_c < nlen;
  const int pos_c = s0 + i_c;  // last key position of this row
  const size_t out_row = ((size_t)b * prm.num_q_heads + h_c) * C + i_c;
  // The row's sink logit in log2 units, loaded now so that its latency is hidden by the loop.
  const float sink_l2 = SW && prm.sinks && row_exists ? bf16lo_to_f32(prm.sinks[h_c]) * kLog2e : 0.f;

  // Last valid chunk position of the workgroup and of this wavefront.
  const int i_hi_wg = min((min(rho0_wg + kRowsPerGroup, rows_total) - 1) / G, nlen - 1);
  const int i_lo_wave = rho0 / G;
  const int i_hi_wave = min((min(rho0 + kRowsPerWave, rows_total) - 1) / G, nlen - 1);
  const bool wave_active = rho0 < rows_total && i_lo_wave < nlen;
  const int ntiles = i_hi_wg >= rho0_wg / G ? (s0 + i_hi_wg) / kTileTokens + 1 : 0;
  const int wave_tiles = wave_active ? (s0 + i_hi_wave) / kTileTokens + 1 : 0;
  const int kmax = s0 + i_hi_wg;  // last key position any row of the workgroup reads
  // Split-K: this workgroup takes key tiles [t_lo, t_hi) of its row block. Pieces past the row
  // block's keys leave at once; piece 0 always runs (it writes the zero rows).
  const int PT = prm.part_tiles;
  const int npieces = PT > 0 ? (ntiles + PT - 1) / PT : 1;
  if (piece > 0 && piece >= npieces) return;
  // Sliding window: the first tile that the workgroup's first row, and this wavefront's first
  // row, see.
  const int W = SW ? prm.window : 0;
  const int tile_first = W > 0 ? max(0, s0 + rho0_wg / G + 1 - W) / kTileTokens : 0;
  const int wave_first = W > 0 ? max(0, s0 + i_lo_wave + 1 - W) / kTileTokens : 0;
  // Pieces wholly before the window leave at once (the merge starts each row at the piece of its
  // window's first key, never earlier than this); piece 0 still writes its rows.
  if (SW && piece > 0 && (piece + 1) * PT <= tile_first) return;
  const int t_lo = SW ? max(PT > 0 ? piece * PT : 0, tile_first) : PT > 0 ? piece * PT : 0;
  const int t_hi = PT > 0 ? min(piece * PT + PT, ntiles) : ntiles;

  float16_t acc[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) acc[md] = float16_t{};
  float m_run = -INFINITY, l_part = 0.f;

  if (t_hi > t_lo) {
    const int32_t* bt = prm.block_tables + (size_t)b * prm.max_blocks_per_seq;
    const int Hkv = prm.num_kv_heads;
    auto block_ok = [&](int blk) { return blk >= 0 && blk < prm.num_blocks; };

    // B operand of the scores: q[row][16ks + 8hl .. +8] (rows outside the chunk read row 0 and
    // become zeros; selects are per word, so nothing goes through private memory).
    // A negative scale is taken as |scale| with q negated (a sign-bit flip, exact), so scores
    // are always scaled by a positive factor and their max can be taken before scaling.
    const uint32_t qmask = row_valid ? 0xffffffffu : 0u;
    const uint32_t qsign = prm.scale_log2e < 0.f ? 0x80008000u : 0u;
    // At least FLT_MIN, so a masked -inf score stays -inf (scale 0 gives uniform weights).
    const float sl2 = fmaxf(fabsf(prm.scale_log2e), 1.17549435e-38f);
    const size_t q_row = row_valid ? out_row : 0;
    uint4 qop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 qv = mask4(prm.q[q_row * ND + 2 * ks + hl], qmask);
      qop[ks] = make_uint4(qv.x ^ (qsign & qmask), qv.y ^ (qsign & qmask), qv.z ^ (qsign & qmask),
                           qv.w ^ (qsign & qmask));
    }

    // The block ids of a tile (at most 8: 64 tokens, block_size >= 8) sit in one VGPR, lane x
    // holding block 64 tile / BS + x % 8, and are read as scalars (readlane). They are loaded one
    // step before the tile's own loads, and every step issues the same loads (tiles past the
    // workgroup's keys read row 0 and are masked), so the waits for one tile never drain the
    // loads of the next.
    const int last_blk = kmax >> prm.bs_log2;
    auto tile_ids = [&](int tile) {
      const int x = ((tile * kTileTokens) >> prm.bs_log2) + (lane & 7);
      return bt[x <= last_blk ? x : 0];
    };

    // Loader: piece r of this thread is token 16*th + c of the tile, 16-byte piece 4*dq + j.
    // Loads are unconditional (positions past kmax and bad block ids read row 0); the mask is
    // applied when the tile goes to LDS, so the loads stay in flight meanwhile. Two tiles are in
    // flight at once (register sets ra and rb, the loop unrolled by two).
    struct TileRegs {
      uint4 k[LD::LOADS], v[LD::LOADS];
      uint32_t mask[LD::LOADS];
      uint64_t vbits;  // bit t: token t is at or before kmax and its block id is valid
    };
    auto load_tile = [&](int tile, int ids, TileRegs& R) {
      auto block_id = [&](int k) { return __builtin_amdgcn_readlane(ids, k); };
      const int t0 = tile * kTileTokens;
#pragma unroll
      for (int r = 0; r < LD::LOADS; ++r) {
        const int u = kWaves * r + wave;
        const int th = u & 3, dp = 4 * (u >> 2) + j;
        const int t = 16 * th + c;
        const int pos = t0 + t;
        // The 16 tokens of this piece row lie in one block, or two for block_size 8.
        const int bi = (16 * th) >> prm.bs_log2;
        const int blk = prm.bs_log2 == 3 && c >= 8 ? block_id(bi + 1) : block_id(bi);
        const bool ok = pos <= kmax && block_ok(blk);
        const size_t row = ok ? (((size_t)blk * Hkv + g) * BS + (pos & (BS - 1))) * ND + dp : 0;
        R.mask[r] = ok ? 0xffffffffu : 0u;
        R.k[r] = prm.k_cache[row];
        R.v[r] = prm.v_cache[row];
      }
      // Validity bits of the tile, computed on the scalar unit.
      uint64_t bits = 0;
      const int nb = kTileTokens >> prm.bs_log2;
      const uint64_t one_block = (1ull << BS) - 1ull;
      for (int k = 0; k < nb; ++k)
        if (block_ok(block_id(k))) bits |= one_block << (k * BS);
      const int lim = kmax - t0 + 1;
      R.vbits = lim >= 64 ? bits : lim <= 0 ? 0ull : bits & ((1ull << lim) - 1ull);
    };
    auto store_tile = [&](int buf, const TileRegs& R) {
      unsigned char* kl = lds + buf * LD::BUF_BYTES;
      unsigned char* vl = kl + LD::K_BYTES;
#pragma unroll
      for (int r = 0; r < LD::LOADS; ++r) {
        const int u = kWaves * r + wave;
        const int t = 16 * (u & 3) + c, dp = 4 * (u >> 2) + j;
        *reinterpret_cast<uint4*>(kl + k_off<D>(t, dp)) = mask4(R.k[r], R.mask[r]);
        *reinterpret_cast<uint4*>(vl + t * LD::K_STRIDE + 16 * (dp ^ v_swz(t))) = mask4(R.v[r], R.mask[r]);
      }
    };

    auto compute = [&](int it, uint64_t vbits) {
      const unsigned char* kl = lds + (it & 1) * LD::BUF_BYTES;
      const unsigned char* vl = kl + LD::K_BYTES;
      // S^T[64 tokens x 32 rows] = K . Q^T as two independent chains (tokens 0-31 and 32-63;
      // back-to-back MFMAs on the same accumulator are forwarded).
      float16_t sa0 = {}, sa1 = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 k0 = *reinterpret_cast<const uint4*>(kl + k_off<D>(n, 2 * ks + hl));
        const uint4 k1 = *reinterpret_cast<const uint4*>(kl + k_off<D>(32 + n, 2 * ks + hl));
        sa0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(k0), as_bf16x8(qop[ks]), sa0, 0, 0, 0);
        sa1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(k1), as_bf16x8(qop[ks]), sa1, 0, 0, 0);
      }
      // Tokens this row may see in the tile, as a bit mask (no per-score branches): valid
      // positions (vbits) up to the row's own position, none for rows outside the chunk. Tiles
      // that every row of the wavefront sees whole skip the masking.
      const int lim = pos_c - it * kTileTokens + 1;  // tokens 0 .. lim-1 are causal for this row
      uint64_t causal = lim >= 64 ? ~0ull : lim <= 0 ? 0ull : (1ull << lim) - 1ull;
      if (W > 0) {
        const int lo = lim - W;  // tokens before lo are outside this row's window
        causal &= lo <= 0 ? ~0ull : lo >= 64 ? 0ull : ~((1ull << lo) - 1ull);
      }
      const uint64_t allowed = row_valid ? vbits & causal : 0ull;
      float sc[32];
      if (__all(allowed == ~0ull)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sc[r] = sa0[r];
          sc[16 + r] = sa1[r];
        }
      } else {
        const uint32_t a0 = (uint32_t)allowed >> (4 * hl), a1 = (uint32_t)(allowed >> 32) >> (4 * hl);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = 8 * (r >> 2) + (r & 3);  // token of register r, less 4 hl (and 32 h2)
          sc[r] = (a0 >> t) & 1u ? sa0[r] : -INFINITY;
          sc[16 + r] = (a1 >> t) & 1u ? sa1[r] : -INFINITY;
        }
      }
      // Max of the raw scores, then in scaled log2 units (the factor is positive).
      float mt = -INFINITY;
#pragma unroll
      for (int r = 0; r < 32; ++r) mt = fmaxf(mt, sc[r]);
      const float2 mp = with_other_half(mt);
      mt = fmaxf(mp.x, mp.y) * sl2;
      // Lazy rescale: the reference max of a row moves only when the tile max exceeds it by
      // more than kRescaleLog2 (or on the row's first finite score). Weights are then at most
      // 2^kRescaleLog2, and the common factor cancels in the final division by l.
      const bool bump = mt > m_run + kRescaleLog2;
      if (__any(bump)) {
        // 0 on a row's first finite max; 1 for rows that keep theirs (also those still at
        // -inf, where m_run - m_run would be NaN).
        const float alpha = bump ? fast_exp2(m_run - mt) : 1.f;
        l_part *= alpha;
#pragma unroll
        for (int md = 0; md < MD; ++md) acc[md] *= alpha;
        m_run = bump ? mt : m_run;
      }
      const float ms = m_run == -INFINITY ? 0.f : m_run;
      bf16x8_t pb[4];
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        const float p = fast_exp2(fmaf(sc[r], sl2, -ms));
        psum += p;
        pb[r >> 3][r & 7] = (__bf16)p;
      }
      l_part += psum;
      // O^T[32 d x 32 rows] += V^T[32 d x 16 tokens] . P^T[16 tokens x 32 rows], four token
      // quarters u per d block. The A operand of lane (n, hl) is V at d = 32md + n for the tokens
      // of its weights: 16u + 4hl + 0..3 and 16u + 8 + 4hl + 0..3 (two transposing reads; lane j
      // of each 16-lane group addresses row j/4 of the four, at d 32md + 16((lane/16)%2) + 4(j%4)).
      // All rows a lane reads are 4hl + j/4 plus a multiple of 8, so they share one swizzle: the
      // address is one per-lane base per d block plus a constant row offset.
      const int jg = lane & 15;
      const int dcol = 16 * ((lane >> 4) & 1) + 4 * (jg & 3);  // d within the 32-wide block
      const int row_l = 4 * hl + (jg >> 2);
      const int swz_l = v_swz(row_l);
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const int d = 32 * md + dcol;
        lds_byte* vb = (lds_byte*)vl + (row_l * LD::K_STRIDE + 16 * ((d >> 3) ^ swz_l) + (d & 7) * 2);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const short4_lds_t lo = lds_read_tr16(vb + 16 * u * LD::K_STRIDE);
          const short4_lds_t hi = lds_read_tr16(vb + (16 * u + 8) * LD::K_STRIDE);
          const short4_t lo4 = __builtin_bit_cast(short4_t, lo), hi4 = __builtin_bit_cast(short4_t, hi);
          const bf16x8_t va = __builtin_bit_cast(
              bf16x8_t, make_uint4((uint16_t)lo4[0] | ((uint32_t)(uint16_t)lo4[1] << 16),
                                   (uint16_t)lo4[2] | ((uint32_t)(uint16_t)lo4[3] << 16),
                                   (uint16_t)hi4[0] | ((uint32_t)(uint16_t)hi4[1] << 16),
                                   (uint16_t)hi4[2] | ((uint32_t)(uint16_t)hi4[3] << 16)));
          acc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[u], acc[md], 0, 0, 0);
        }
      }
    };

    // One step: the ids of tile it+3 and tile it+2 itself (into `fut`) start loading, tile it is
    // processed from LDS, tile it+1 (loaded one step earlier into `nxt`) goes to the other LDS
    // buffer.
    uint64_t vbits = 0;
    auto step = [&](int it, TileRegs& nxt, TileRegs& fut, int& ids_now, int& ids_next) {
      ids_next = tile_ids(it + 3);
      load_tile(it + 2, ids_now, fut);
      if (it < wave_tiles && (!SW || it >= wave_first)) compute(it, vbits);
      store_tile((it + 1) & 1, nxt);
      __syncthreads();
      vbits = nxt.vbits;
    };

    TileRegs ra, rb;
    int ida = tile_ids(t_lo), idb;
    load_tile(t_lo, ida, ra);
    store_tile(t_lo & 1, ra);
    vbits = ra.vbits;
    // Same order of loads as in a step: the ids of tile t_lo+2 before the loads of tile t_lo+1.
    idb = tile_ids(t_lo + 1);
    ida = tile_ids(t_lo + 2);
    load_tile(t_lo + 1, idb, ra);
    __syncthreads();
    for (int it = t_lo; it < t_hi; it += 2) {
      step(it, ra, rb, ida, idb);
      if (it + 1 >= t_hi) break;
      step(it + 1, rb, ra, idb, ida);
    }
  }

  const float2 lp = with_other_half(l_part);
  const float l_tot = lp.x + lp.y;
  // The sink of an unsplit row: e^(sigma - m) more in the denominator (in log2 units; a row with
  // no keys keeps its zeros).
  float den = l_tot;
  if (SW && prm.sinks && npieces <= 1 && m_run != -INFINITY) den += fast_exp2(sink_l2 - m_run);
  const float inv = row_valid && den > 0.f ? 1.f / den : 0.f;
  // acc[md][r] is O[row n][32md + 8(r/4) + 4hl + r%4]: four runs of 4 values per d block.
  if (row_exists && npieces > 1 && row_valid) {
    // A piece of a split row block: this row's output over the piece's keys, and its (m, l)
    // (m = -inf, l = 0 and a zero output for a row with no keys in the piece).
    const size_t prow = out_row * prm.max_partitions + piece;
    float4* po = reinterpret_cast<float4*>(prm.part_o + prow * D);
#pragma unroll
    for (int md = 0; md < MD; ++md) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float* o = reinterpret_cast<const float*>(&acc[md]) + 4 * q4;
        po[8 * md + 2 * q4 + hl] = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
      }
    }
    if (hl == 0) prm.part_ml[prow] = make_float2(m_run, l_tot);
  }
  if (piece > 0) return;  // rows past chunk_lens get their zeros from piece 0 (uniform: the whole workgroup)
  // Output rows. A lane's row is one head of one chunk position, and the rows of a wavefront
  // belong to several heads, whose rows lie C * D * 2 bytes apart in `out`: written straight from
  // the accumulators, every store would scatter 16-byte pieces over 32 rows. The bf16 rows are
  // staged in LDS instead (the tile buffers are free once every wavefront is past its last tile;
  // 256 rows of 2D bytes fill them exactly, laid out like K rows), then written with ND
  // consecutive lanes per row, whole rows of 128 or 256 bytes.
  __syncthreads();
  if (row_exists) {
    const int lr = wave * kRowsPerWave + n;
#pragma unroll
    for (int md = 0; md < MD; ++md) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float* o = reinterpret_cast<const float*>(&acc[md]) + 4 * q4;
        *reinterpret_cast<uint2*>(lds + k_off<D>(lr, 4 * md + q4) + 8 * hl) =
            make_uint2(pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv));
      }
    }
  }
  __syncthreads();
  const int nrows = min(kRowsPerGroup, rows_total - rho0_wg);
  for (int x = tid; x < nrows * ND; x += 64 * kWaves) {
    const int lr = x / ND, p = x % ND;
    const int rho = rho0_wg + lr;
    const int i = rho / G;
    if (npieces > 1 && i < nlen) continue;  // split rows: the merge writes them
    const size_t orow = ((size_t)b * prm.num_q_heads + g * G + rho % G) * C + i;
    prm.out[orow * ND + p] = *reinterpret_cast<const uint4*>(lds + k_off<D>(lr, p));
  }
}

// Split-K merge of the rows of split row blocks (the others were written by the attention
// kernel): D/E lanes per row, E consecutive d each (E = 4 or 8). Row (b, h, i) combines the pieces
// that hold keys it sees (pieces 0 .. pos / (64 PT)): M = max_j m_j, w_j = l_j 2^(m_j - M),
// out = sum_j w_j o_j / sum_j w_j, taken four pieces at a time (their loads in flight together)
// with a running maximum. SW: the pieces start at the one holding the row's first window key,
// and the sink enters as one more term of weight 2^(sigma - M) with no value row.
// The merge is a chain of dependent loads (the lengths, then the partials). E = 8 halves the
// wavefronts at the cost of a longer chain per lane: it pays where the E = 4 grid would take
// several rounds of resident workgroups (measured: 14.6 -> 10.6 us on the Qwen3 batch's rows),
// not where one round holds it (the 16K chunk: 204 -> 209 us per call).
constexpr int kMergeThreads = 256;
template <int D, bool SW, int E>
__global__ __launch_bounds__(kMergeThreads) void prefill_merge_kernel(PrefillParams prm) {
  static_assert(E == 4 || E == 8, "four or eight d per lane");
  constexpr int NV = E / 4;                 // float4 pieces of a partial row per lane
  constexpr int LPR = D / E;                // lanes per row
  constexpr int RPB = kMergeThreads / LPR;  // rows per workgroup
  const int sub = threadIdx.x % LPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;  // (b * Hq + h) * C + i
  const int C = prm.chunk, G = prm.group;
  if (row >= (long long)prm.batch * prm.num_q_heads * C) return;
  const int i = (int)(row % C);
  const int h = (int)((row / C) % prm.num_q_heads);
  const int b = (int)(row / ((long long)C * prm.num_q_heads));
  const int BS = 1 << prm.bs_log2;
  const int s0 = prm.start_pos[b], nlen = prm.chunk_lens[b];
  if (s0 < 0 || nlen < 0 || nlen > C || (long long)s0 + nlen > (long long)prm.max_blocks_per_seq * BS) return;
  if (i >= nlen) return;
  // The row's row block and whether it was split (the same arithmetic as the attention kernel).
  const int rb = (i * G + h % G) / kRowsPerGroup;
  const int i_hi_wg = min((min((rb + 1) * kRowsPerGroup, C * G) - 1) / G, nlen - 1);
  const int ntiles = (s0 + i_hi_wg) / kTileTokens + 1;
  const int PT = prm.part_tiles;
  if ((ntiles + PT - 1) / PT <= 1) return;
  const int nrow = (s0 + i) / (kTileTokens * PT) + 1;  // pieces holding keys 0 .. s0 + i
  const size_t prow0 = (size_t)row * prm.max_partitions;
  float M = -INFINITY, wsum = 0.f;
  int jfirst = 0;
  if (SW) {
    if (prm.window > 0) jfirst = max(0, s0 + i + 1 - prm.window) / (kTileTokens * PT);
    if (prm.sinks) {
      M = bf16lo_to_f32(prm.sinks[h]) * kLog2e;  // the sink's term, 2^(sigma - M) = 1
      wsum = 1.f;
    }
  }
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int j0 = jfirst; j0 < nrow; j0 += 4) {
    float2 ml[4];
    float4 o[4][NV];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool in = j0 + u < nrow;
      const size_t pr = prow0 + (in ? j0 + u : 0);
      ml[u] = prm.part_ml[pr];
      const float4* src = reinterpret_cast<const float4*>(prm.part_o + pr * D) + NV * sub;
#pragma unroll
      for (int v = 0; v < NV; ++v) o[u][v] = src[v];
      if (!in) ml[u] = make_float2(-INFINITY, 0.f);
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < 4; ++u) Mn = fmaxf(Mn, ml[u].x);
    if (Mn == -INFINITY) continue;  // no keys yet
    const float f = fast_exp2(M - Mn);  // 0 while M is still -inf
    wsum *= f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] *= f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = ml[u].y * fast_exp2(ml[u].x - Mn);  // 0 for a piece with none of the row's keys
      wsum += w;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        acc[4 * v] = fmaf(w, o[u][v].x, acc[4 * v]);
        acc[4 * v + 1] = fmaf(w, o[u][v].y, acc[4 * v + 1]);
        acc[4 * v + 2] = fmaf(w, o[u][v].z, acc[4 * v + 2]);
        acc[4 * v + 3] = fmaf(w, o[u][v].w, acc[4 * v + 3]);
      }
    }
    M = Mn;
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  uint2* dst = reinterpret_cast<uint2*>(prm.out) + (size_t)row * (D / 4) + NV * sub;
#pragma unroll
  for (int v = 0; v < NV; ++v)
    dst[v] = make_uint2(pack_bf16x2(acc[4 * v] * inv, acc[4 * v + 1] * inv),
                        pack_bf16x2(acc[4 * v + 2] * inv, acc[4 * v + 3] * inv));
}

template <int D, bool SW>
hipError_t launch_prefill_d(const PrefillParams& p, hipStream_t stream) {
  const long long pieces = p.part_tiles > 0 ? p.max_partitions : 1;
  const long long grid = (long long)p.batch * p.num_kv_heads * p.row_blocks * pieces;
  hipLaunchKernelGGL((paged_prefill_kernel<D, SW>), dim3((unsigned)grid), dim3(64 * kWaves), 0, stream, p);
  if (p.part_tiles > 0) {
    const long long rows = (long long)p.batch * p.num_q_heads * p.chunk;
    // Eight d per lane when four would need more workgroups than one resident round (eight
    // 256-thread workgroups per CU).
    constexpr int rpb4 = kMergeThreads / (D / 4), rpb8 = kMergeThreads / (D / 8);
    if ((rows + rpb4 - 1) / rpb4 > 8LL * device_cu_count())
      hipLaunchKernelGGL((prefill_merge_kernel<D, SW, 8>), dim3((unsigned)((rows + rpb8 - 1) / rpb8)),
                         dim3(kMergeThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((prefill_merge_kernel<D, SW, 4>), dim3((unsigned)((rows + rpb4 - 1) / rpb4)),
                         dim3(kMergeThreads), 0, stream, p);
  }
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
  p.part_o = a.part_o;
  p.part_ml = reinterpret_cast<float2*>(a.part_ml);
  p.part_tiles = a.partition_size / kTileTokens;
  p.max_partitions = a.max_partitions;
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
  p.sinks = static_cast<const uint16_t*>(a.sinks);
  p.window = a.window;
  // Largest first where the order matters and the sizes differ: split-K pieces (always more
  // workgroups than CUs' worth of work at once), or unsplit row blocks when the grid exceeds
  // one workgroup per CU (the resident limit at these register counts) and there is no window
  // (windowed row blocks are all alike, and the ranking would only add latency). The ranking
  // covers up to kRankMax row blocks per kv head.
  const long long rbs = (long long)p.batch * p.row_blocks;
  p.rank_items = rbs <= kRankMax && (p.part_tiles > 0 || (rbs * p.num_kv_heads > device_cu_count() && p.window == 0));
  if (a.sinks || a.window > 0)
    return a.head_dim == 64 ? launch_prefill_d<64, true>(p, stream) : launch_prefill_d<128, true>(p, stream);
  return a.head_dim == 64 ? launch_prefill_d<64, false>(p, stream) : launch_prefill_d<128, false>(p, stream);
}

}  // namespace xs
