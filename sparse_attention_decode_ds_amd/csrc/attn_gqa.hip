// attn_gqa.hip -- attention pass for query groups of G >= 2 heads that share
// one K/V head ([GQA] section 4; [DS] "online forward computation", step 3:
// exact softmax attention over the selected tokens' full K/V rows; [LeanK]
// section 2.2: K stored as d_k kept columns, the query read at keep[c]).
//
// Each selected K/V row is loaded once for the whole group, and both
// products of a tile of 16 tokens run on the matrix cores (16x16x16 fp16
// inputs, fp32 accumulation), with every operand in registers:
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
#include "attn_common.h"

namespace ds {
namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kGT = 256;  // threads per workgroup (4 waves)
constexpr int kTile = 16;  // tokens per tile

template <int G>
struct GqaLds {
  alignas(16) __half q[G][kDv];  // the query rows at the stored K columns' channels
  int32_t lidx[kMaxTokensPerSplit];
  AttnRed<G> red;  // per wave: final (o, m, l) of each head
};

struct GqaTile {
  uint4 k[4];  // K: 64 bytes of the row of token m16
  uint4 v[4];  // V: channels [8 m16, 8 m16 + 8) of tokens 4 kg + j
};

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

template <int G, bool FINAL>
__global__ __launch_bounds__(kGT) void k_attn_gqa(AttnArgs a) {
  __shared__ GqaLds<G> f;
  const int row = blockIdx.x / a.n_split;
  const int split = blockIdx.x - row * a.n_split;
  const int b = row / a.Hkv;
  const int g = row - b * a.Hkv;
  const int S = min(max(a.seq_lens[b], 0), a.max_seq);
  const int n_tok = a.sparse ? min(a.count[row], S) : S;
  const int t0 = split * a.tps;
  const int n_here = max(0, min(n_tok - t0, a.tps));
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_id();
  const int m16 = lane & 15;  // K token of the tile; head of the score and output columns
  const int kg = lane >> 4;   // K channels [32 kg, 32 kg + 32); V tokens 4 kg .. 4 kg + 3

  // The first batch of the token list and the query rows are fetched
  // together (one round trip, one barrier).
  const int32_t* src0 = a.idx + (int64_t)row * a.idx_stride + t0;
  if (a.sparse)
    for (int i = tid; i < min(n_here, kMaxTokensPerSplit); i += kGT) f.lidx[i] = src0[i];
  // Query operand: q of head m16 (zero past G) at the query channel of each
  // stored K column 32 kg + 4 s + j, staged in LDS per stored column.
  for (int i = tid; i < G * kDv; i += kGT) {
    const int h = i / kDv, c = i - h * kDv;
    __half v = __float2half(0.0f);
    if (c < a.d_k) {
      const __half* qh = a.q + ((int64_t)b * a.Hq + (int64_t)g * G + h) * a.d_q;
      v = qh[a.keep ? a.keep[(int64_t)g * a.d_k + c] : c];
    }
    f.q[h][c] = v;
  }
  __syncthreads();
  half4_t qb[8];
  {
    const bool hv = m16 < G;
    const uint4* qr = reinterpret_cast<const uint4*>(&f.q[hv ? m16 : 0][32 * kg]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint4 x = hv ? qr[u] : make_uint4(0, 0, 0, 0);
      qb[2 * u] = __builtin_bit_cast(half4_t, u32x2_t{x.x, x.y});
      qb[2 * u + 1] = __builtin_bit_cast(half4_t, u32x2_t{x.z, x.w});
    }
  }

  const __half* Kr = a.K + (int64_t)b * a.ks0 + (int64_t)g * a.ks1 + 32 * kg;
  const __half* Vr = a.V + (int64_t)b * a.vs0 + (int64_t)g * a.vs1 + 8 * m16;
  float4_t oacc[8];  // oacc[s][jj] = O[head m16][8 (4 kg + jj) + s]
#pragma unroll
  for (int s = 0; s < 8; ++s) oacc[s] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = kNegInf, l_run = 0.0f;  // head m16

  for (int bat = 0; bat < n_here; bat += kMaxTokensPerSplit) {
    const int nb = min(kMaxTokensPerSplit, n_here - bat);
    if (a.sparse && bat > 0) {
      __syncthreads();
      for (int i = tid; i < nb; i += kGT) f.lidx[i] = src0[bat + i];
      __syncthreads();
    }
    auto tok = [&](int i) -> int64_t {
      return a.sparse ? (int64_t)f.lidx[i] : (int64_t)(t0 + bat + i);
    };
    auto load = [&](int i0, GqaTile& T) {
      const int ik = i0 + m16;
      const bool kv_ok = ik < nb;
      const int64_t tk = kv_ok ? tok(ik) : 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        T.k[u] = make_uint4(0, 0, 0, 0);
        if (kv_ok && 32 * kg + 8 * u < a.d_k) T.k[u] = ld_stream(Kr + tk * a.ks2 + 8 * u);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int iv = i0 + 4 * kg + j;
        T.v[j] = make_uint4(0, 0, 0, 0);
        if (iv < nb) T.v[j] = ld_stream(Vr + tok(iv) * a.vs2);
      }
    };
    GqaTile cur, nxt;
    int i0 = w * kTile;
    if (i0 < nb) load(i0, nxt);
    for (; i0 < nb; i0 += 4 * kTile) {
      cur = nxt;
      if (i0 + 4 * kTile < nb) load(i0 + 4 * kTile, nxt);
      // scores of the tile: lane holds S[token 4 kg + j][head m16]
      float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint4 kv = cur.k[s >> 1];
        const u32x2_t pr = (s & 1) ? u32x2_t{kv.z, kv.w} : u32x2_t{kv.x, kv.y};
        acc = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, pr), qb[s], acc,
                                                    0, 0, 0);
      }
      float sv[4];
      float tm = kNegInf;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sv[j] = i0 + 4 * kg + j < nb ? acc[j] * a.scale_log2 : kNegInf;
        tm = fmaxf(tm, sv[j]);
      }
      LanePair pr = xchg16(tm);  // over the four lane groups
      tm = fmaxf(pr.lo, pr.hi);
      pr = xchg32(tm);
      tm = fmaxf(pr.lo, pr.hi);
      const float mnew = fmaxf(m_run, tm);  // finite: token i0 of the tile is real
      const float al = m_run == kNegInf ? 0.0f : exp2f(m_run - mnew);
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
      l_run = l_run * al + ps;
      m_run = mnew;
      const half4_t pb = {(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
#pragma unroll
      for (int s = 0; s < 8; ++s)
        oacc[s] = __builtin_amdgcn_mfma_f32_16x16x16f16(pick_half(cur.v, s), pb, oacc[s] * al, 0, 0,
                                                        0);
    }
  }

  // The wave's state into LDS, then the four waves merged per head.
  if (m16 < G) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int s = 0; s < 8; ++s) f.red.v[w][m16][8 * (4 * kg + jj) + s] = oacc[s][jj];
    if (kg == 0) {
      f.red.v[w][m16][kDv] = m_run;
      f.red.v[w][m16][kDv + 1] = l_run;
    }
  }
  __syncthreads();
  attn_store<G, FINAL>(a, f.red, b, g, split);
}

template <int G>
hipError_t launch_g(const AttnArgs& a, int rows, bool final_out, hipStream_t s, const KEvents& ev) {
  const dim3 grid(rows * a.n_split);
  if (final_out) return launch_k(k_attn_gqa<G, true>, grid, dim3(kGT), s, ev, a);
  return launch_k(k_attn_gqa<G, false>, grid, dim3(kGT), s, ev, a);
}

}  // namespace

hipError_t launch_attn_gqa(const AttnArgs& a, int rows, int G, bool final_out, hipStream_t s,
                           const KEvents& ev) {
  if (rows <= 0) return hipSuccess;
  switch (G) {
    case 2: return launch_g<2>(a, rows, final_out, s, ev);
    case 3: return launch_g<3>(a, rows, final_out, s, ev);
    case 4: return launch_g<4>(a, rows, final_out, s, ev);
    case 5: return launch_g<5>(a, rows, final_out, s, ev);
    case 6: return launch_g<6>(a, rows, final_out, s, ev);
    case 7: return launch_g<7>(a, rows, final_out, s, ev);
    case 8: return launch_g<8>(a, rows, final_out, s, ev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ds
