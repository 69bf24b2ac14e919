// gqa_tile.h -- one wave's share of group attention: tiles of 16 tokens whose
// two products run on the matrix cores ([GQA] section 4: the G query heads of
// a group read the same K/V rows; [DS] "online forward computation", step 3:
// exact softmax attention over the selected tokens' full K/V rows; [LeanK]
// section 2.2: K stored as d_k kept columns, the query read at keep[c]).
//
// Per tile, with 16x16x16 fp16 inputs and fp32 accumulation, every operand in
// registers:
//
//   scores   S[t][h] = sum_c K[t][c] q_h[keep[c]]: eight products over the
//            128 stored channels (rows: tokens, columns: heads padded to 16);
//   softmax  online per head in fp32 (exp2 domain), the tile maximum and sum
//            taken across the four lane groups with permlane swaps;
//   output   O^T[c][h] += sum_t V[t][c] P[t][h]: eight products of 16
//            channels each; P is the score tile itself (the score product
//            leaves S[4 kg + j][h] in lane (h, kg), which is the B operand of
//            the output product), rounded to fp16.
//
// Operand layout of v_mfma_f32_16x16x16_f16 (wave of 64): lane l supplies
// A[l % 16][4 (l / 16) + j] and B[4 (l / 16) + j][l % 16] for j = 0..3 and
// receives D[4 (l / 16) + j][l % 16].  Contraction orders are free:
//   scores: lane group kg = l / 16 takes channels [32 kg, 32 kg + 32), step s
//     channels 32 kg + 4 s + j: the lane's K operand for all eight steps is
//     one contiguous 64-byte piece of its token's row;
//   output: row i of step s is channel 8 i + s, so lane (i, kg) needs
//     channels [8 i, 8 i + 8) of tokens 4 kg .. 4 kg + 3: four 16-byte loads,
//     and its accumulators hold channels [32 kg, 32 kg + 32) of head i.
#pragma once

#include "attn_common.h"

namespace ds {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kGqaTile = 16;  // tokens per tile

struct GqaTile {
  uint4 k[4];  // K: 64 bytes of the row of token m16
  uint4 v[4];  // V: channels [8 m16, 8 m16 + 8) of tokens 4 kg + j
};

// The wave's online-softmax state: o[s][jj] = O[head m16][8 (4 kg + jj) + s]
// (unnormalised), m and l of head m16.
struct GqaState {
  float4_t o[8];
  float m, l;
};

__device__ __forceinline__ void gqa_init(GqaState& st) {
#pragma unroll
  for (int s = 0; s < 8; ++s) st.o[s] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  st.m = kNegInf;
  st.l = 0.0f;
}

// Lane roles and row bases: m16 = lane % 16 (K token of the tile; head of
// the score and output columns), kg = lane / 16.
struct GqaLane {
  const __half* Kb;  // K of the (batch, KV head) row
  const __half* Vr;  // V of the row, at channel 8 m16
  int m16, kg;
  // paged: the bases exclude the batch row (tokens are physical ids)
  __device__ __forceinline__ GqaLane(const AttnArgs& a, int b, int g, bool paged) {
    const int lane = threadIdx.x & 63;
    m16 = lane & 15;
    kg = lane >> 4;
    Kb = a.K + (paged ? 0 : (int64_t)b * a.ks0) + (int64_t)g * a.ks1;
    Vr = a.V + (paged ? 0 : (int64_t)b * a.vs0) + (int64_t)g * a.vs1 + 8 * m16;
  }
};

// Query operand: q of head m16 (zero for m16 >= ng) at the stored K columns'
// channels 32 kg + 4 s + j, from rows staged in LDS (row h: d_k halves at the
// query channels of the stored columns, zero past d_k, 16-byte aligned).
__device__ __forceinline__ void gqa_query(const __half* qk, int ng, const GqaLane& ln,
                                          half4_t (&qb)[8]) {
  const bool hv = ln.m16 < ng;
  const uint4* qr = reinterpret_cast<const uint4*>(qk + (hv ? ln.m16 : 0) * kDv + 32 * ln.kg);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint4 x = hv ? qr[u] : make_uint4(0, 0, 0, 0);
    qb[2 * u] = __builtin_bit_cast(half4_t, u32x2_t{x.x, x.y});
    qb[2 * u + 1] = __builtin_bit_cast(half4_t, u32x2_t{x.z, x.w});
  }
}

// Loads of the tile at list positions [i0, i0 + 16) of nb (nb >= 1); tok(i)
// is the token at position i.  Every load is issued, without a branch:
// positions past nb read the token at nb - 1 and K columns past d_k read
// the last stored column.  Their values never count: the scores of such
// positions are set to -inf (so P = 0) and the query is zero past d_k.
// Branch-free loads let the compiler wait for one tile while later tiles are
// still in flight.
template <bool PAGED, typename TokFn>
__device__ __forceinline__ void gqa_load(const AttnArgs& a, const GqaLane& ln, int i0, int nb,
                                         TokFn tok, GqaTile& T) {
  const int64_t tk = tok(min(i0 + ln.m16, nb - 1));
  const __half* kr = ln.Kb + k_off<PAGED>(a, tk);
#pragma unroll
  for (int u = 0; u < 4; ++u) T.k[u] = ld_stream(kr + min(32 * ln.kg + 8 * u, a.d_k - 8));
#pragma unroll
  for (int j = 0; j < 4; ++j)
    T.v[j] = ld_stream(ln.Vr + v_off<PAGED>(a, tok(min(i0 + 4 * ln.kg + j, nb - 1))));
}

// Half s (0..7) of the four 16-byte pieces x[0..3], as the A operand.
__device__ __forceinline__ half4_t pick_half(const uint4 (&x)[4], int s) {
  const int wsel = s >> 1;
  auto word = [&](const uint4& v) {
    return wsel == 0 ? v.x : wsel == 1 ? v.y : wsel == 2 ? v.z : v.w;
  };
  // v_perm_b32: bytes {0,1} (low half) or {2,3} (high half) of each source
  const uint32_t sel = (s & 1) ? 0x07060302u : 0x05040100u;
  const uint32_t lo = __builtin_amdgcn_perm(word(x[1]), word(x[0]), sel);
  const uint32_t hi = __builtin_amdgcn_perm(word(x[3]), word(x[2]), sel);
  return __builtin_bit_cast(half4_t, u32x2_t{lo, hi});
}

// One tile (positions [i0, i0 + 16) of nb, i0 < nb) into the state.
__device__ __forceinline__ void gqa_tile(const GqaTile& cur, const half4_t (&qb)[8], int i0, int nb,
                                         float scale_log2, int kg, GqaState& st) {
  // scores of the tile: lane holds S[token 4 kg + j][head m16]
  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const uint4 kv = cur.k[s >> 1];
    const u32x2_t pr = (s & 1) ? u32x2_t{kv.z, kv.w} : u32x2_t{kv.x, kv.y};
    acc = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, pr), qb[s], acc, 0, 0,
                                                0);
  }
  float sv[4];
  float tm = kNegInf;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sv[j] = i0 + 4 * kg + j < nb ? acc[j] * scale_log2 : kNegInf;
    tm = fmaxf(tm, sv[j]);
  }
  LanePair pr = xchg16(tm);  // over the four lane groups
  tm = fmaxf(pr.lo, pr.hi);
  pr = xchg32(tm);
  tm = fmaxf(pr.lo, pr.hi);
  const float mnew = fmaxf(st.m, tm);  // finite: token i0 of the tile is real
  const float al = st.m == kNegInf ? 0.0f : exp2f(st.m - mnew);
  float p[4], ps = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    p[j] = sv[j] == kNegInf ? 0.0f : exp2f(sv[j] - mnew);
    ps += p[j];
  }
  pr = xchg16(ps);
  ps = pr.lo + pr.hi;
  pr = xchg32(ps);
  ps = pr.lo + pr.hi;
  st.l = st.l * al + ps;
  st.m = mnew;
  const half4_t pb = {(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
#pragma unroll
  for (int s = 0; s < 8; ++s)
    st.o[s] = __builtin_amdgcn_mfma_f32_16x16x16f16(pick_half(cur.v, s), pb, st.o[s] * al, 0, 0, 0);
}

// The wave's state into slot w of `red` (heads m16 < ng).
template <int G, int NW>
__device__ __forceinline__ void gqa_to_red(const GqaState& st, const GqaLane& ln, int ng, int w,
                                           AttnRed<G, NW>& red) {
  if (ln.m16 < ng) {
    float* dst = &red.v[w][ln.m16][0];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float4* d4 = reinterpret_cast<float4*>(dst + 8 * (4 * ln.kg + jj));
      d4[0] = make_float4(st.o[0][jj], st.o[1][jj], st.o[2][jj], st.o[3][jj]);
      d4[1] = make_float4(st.o[4][jj], st.o[5][jj], st.o[6][jj], st.o[7][jj]);
    }
    if (ln.kg == 0) {
      dst[kDv] = st.m;
      dst[kDv + 1] = st.l;
    }
  }
}

// The wave states merged per head and channel by threads (h, c), h < ng,
// and the fp16 output written (one channel per thread).
template <int NW>
__device__ __forceinline__ void gqa_merge_out(const AttnArgs& a, const AttnRed<kMaxGroup, NW>& red,
                                              int b, int g, int ng) {
  const int tid = threadIdx.x;
  if (tid >= ng * kDv) return;
  const int h = tid / kDv, c = tid - h * kDv;
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, red.v[w][h][kDv]);
  float L = 0.0f, O = 0.0f;
  if (M != kNegInf) {
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = red.v[w][h][kDv];
      if (mw == kNegInf) continue;
      const float sc = exp2f(mw - M);
      L += sc * red.v[w][h][kDv + 1];
      O += sc * red.v[w][h][c];
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  a.out[((int64_t)b * a.Hq + (int64_t)g * ng + h) * kDv + c] = __float2half_rn(O * inv);
}

}  // namespace ds
