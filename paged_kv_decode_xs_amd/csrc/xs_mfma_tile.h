// One wavefront's online-softmax attention over 16-token tiles on the matrix cores (bf16 K/V,
// head_dim 64/128, GC <= 8 query heads sharing one kv head). Shared by the decode kernels.
//
// What a tile adds (xserv compare phase10...cf1e9e41, attention.rs, `paged_decode_attention`;
// GQA by `repeat_kv` in xserv compare phase8...phase13): for the GC heads h and tokens t of the
// tile, s_t = scale * q_h . K_t, and the running (m, l, o) of each head absorbs the tile:
//   m' = max(m, max_t s_t),  l' = l e^(m-m') + sum_t e^(s_t-m'),  o' = o e^(m-m') + sum_t e^(s_t-m') V_t.
//
//   QK  C[16 tokens x 16] = K_tile[16 x D] . Q^T[D x 16] with v_mfma_f32_16x16x32_bf16 (D/32 of
//       them). The 16 columns hold the GC heads repeated, so lane l ends with the scores of
//       tokens 4(l/16)+i (i = 0..3) for head (l%16) % GC. The A operand (K) needs lane l to hold
//       16 bytes of token l%16, so each K load moves four 64-byte runs per token row.
//   softmax  The running max is kept per head and shared by the whole wavefront: a tile max
//       over the lane's 4 scores, then across the four lane rows. p = 2^(s*log2e*scale - m).
//       The accumulators are rescaled only when some head's max moved.
//   PV  O[4 heads x D] += P[4 heads x 4 tokens] . V[4 tokens x D] per group of 4 tokens, with
//       v_mfma_f32_4x4x4_16b_bf16: its 16 blocks each take 4 columns of d, and all of them use
//       the P operand of one block (CBSZ/ABID broadcast). That operand (P, rounded to bf16) is
//       exactly what the QK output left in lanes 16kg..16kg+3. The B operand needs 4 tokens of
//       one d per lane, so V goes through the wavefront's own LDS slice and comes back 2 bytes
//       at a time; lane l reads column d = 64h + l, 128 consecutive bytes per wavefront.
//       The accumulator is O[head][64h + lane]: D/16 registers per 4 heads.
// Tokens outside the tile's valid range get score -inf and a zeroed V, so pool tails (NaN
// included) and positions before a sliding window never reach the result.
#pragma once

#include <math.h>

#include <type_traits>
#include <utility>

#include "xs_device.h"

namespace xs {

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

template <int D, int GC>
struct TileAttn {
  static constexpr int KK = D / 32;                // QK matrix ops per tile
  static constexpr int NH = D / 64;                // 64-wide d halves of the PV output
  static constexpr int HP = (GC + 3) / 4;          // PV passes of 4 heads
  static constexpr int ROW16 = D / 8;              // 16-byte pieces per token row
  static constexpr int VL = 16 * ROW16 / 64;       // V loads per lane per tile
  static constexpr int STRIDE = 2 * D;             // LDS bytes per token row
  static constexpr int STAGE_BYTES = 16 * STRIDE;  // one wavefront's V tile
  static constexpr int ACC = HP * NH;              // 4-float accumulators per lane
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(GC == 1 || GC == 2 || GC == 4 || GC == 8, "heads per wavefront");

  uint4 qop[KK];       // B operand of QK: q[h0 + c%GC][32kk + 8j .. +8]
  float4_t acc[ACC];   // acc[hp*NH + hf][i] = O[head 4hp+i][64hf + lane] (rows past GC repeat)
  float m_run;         // running max of head c%GC, the same in every lane of that head
  float l_part;        // this lane's share of the softmax sum of head c%GC

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int a = 0; a < ACC; ++a) acc[a] = float4_t{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_part = 0.f;
  }

  // q rows q_row0 .. q_row0+GC-1 (16-byte pieces, ROW16 per row).
  __device__ __forceinline__ void load_q(const uint4* q, size_t q_row0, int lane) {
    const int j = lane >> 4, c = lane & 15;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qop[kk] = q[(q_row0 + c % GC) * ROW16 + 4 * kk + j];
  }

  // Loads one tile. `kpool`/`vpool` point at the tile's first token row of one kv head; token
  // `new_tok` of the tile (or -1) comes from `knew`/`vnew` (one row each) instead.
  __device__ __forceinline__ static void load_tile(const uint4* kpool, const uint4* vpool, int new_tok,
                                                   const uint4* knew, const uint4* vnew, int lane, uint4 (&kr)[KK],
                                                   uint4 (&vr)[VL]) {
    const int j = lane >> 4, c = lane & 15;
    const uint4* ks = c == new_tok ? knew : kpool + c * ROW16;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) kr[kk] = load_stream(ks + 4 * kk + j);
#pragma unroll
    for (int r = 0; r < VL; ++r) {
      const int piece = r * 64 + lane;
      const uint4* vs = piece / ROW16 == new_tok ? vnew + piece % ROW16 : vpool + piece;
      vr[r] = load_stream(vs);
    }
  }

  // Adds the tile's tokens 0 .. nvalid-1.
  __device__ __forceinline__ void process(const uint4 (&kr)[KK], const uint4 (&vr)[VL], int nvalid,
                                          unsigned char* vlds, float scale_log2e, int lane) {
    process_range(kr, vr, 0, nvalid, vlds, scale_log2e, lane);
  }

  // Adds the tile's tokens lo .. hi-1 (a sliding window can start inside a tile).
  __device__ __forceinline__ void process_range(const uint4 (&kr)[KK], const uint4 (&vr)[VL], int lo, int hi,
                                                unsigned char* vlds, float scale_log2e, int lane) {
    constexpr float kNegInf = -INFINITY;
    const int j = lane >> 4;
    // Stage V in LDS (rows of 2D bytes); tokens outside [lo, hi) become zeros.
#pragma unroll
    for (int r = 0; r < VL; ++r) {
      const int piece = r * 64 + lane;
      uint4 v = vr[r];
      if (piece / ROW16 >= hi || piece / ROW16 < lo) v = make_uint4(0, 0, 0, 0);
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
      sc[i] = s[i] * scale_log2e;
      if (4 * j + i >= hi || 4 * j + i < lo) sc[i] = kNegInf;
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
  }

  // Per-head (m, l) over this wavefront's tokens, as wave-uniform values: head r's are held by
  // lane r. Every lane must call this (it shuffles).
  __device__ __forceinline__ void head_stats(float (&m_h)[HP * 4], float (&l_h)[HP * 4]) const {
    float l_tot = l_part + __shfl_xor(l_part, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
#pragma unroll
    for (int r = 0; r < HP * 4; ++r) {
      m_h[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_run), r));
      l_h[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l_tot), r));
    }
  }
};

}  // namespace xs
