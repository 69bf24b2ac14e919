// attn_gqa.hip -- attention pass for query groups of G >= 2 heads that share
// one K/V head ([GQA] section 4; [DS] "online forward computation", step 3:
// exact softmax attention over the selected tokens' full K/V rows; [LeanK]
// section 2.2: K stored as d_k kept columns, the query read at keep[c]).
//
// Each selected K row is loaded once for the whole group.  Per tile of 16
// tokens the scores S[t][h] = sum_c K[t][c] q_h[keep[c]] are one chain of
// eight 16x16x16 fp16 matrix-core products with fp32 accumulation (rows:
// tokens, columns: heads padded to 16, contraction: 128 stored channels in
// eight steps of 16).  The softmax runs in fp32 per head (online, exp2
// domain), and P.V accumulates in fp32 on the vector units with each lane
// owning two output channels of every head; the tile's probabilities reach
// every lane through LDS.
//
// Operand layout of v_mfma_f32_16x16x16_f16 (wave of 64): lane l supplies
// A[l % 16][4 (l / 16) + j] and B[4 (l / 16) + j][l % 16] for j = 0..3 and
// receives D[4 (l / 16) + j][l % 16].  The contraction order is free, so lane
// group kg = l / 16 takes channels [32 kg, 32 kg + 32) and step s of the
// chain uses channels 32 kg + 4 s + j: the lane's K operand for all eight
// steps is one contiguous 64-byte piece of the token's row.
#include "attn_common.h"

namespace ds {
namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kGT = 256;  // threads per workgroup (4 waves)
constexpr int kTile = 16;  // tokens per score tile

template <int G>
struct GqaLds {
  alignas(16) __half q[G][kDv];  // the query rows at the stored K columns' channels
  int32_t lidx[kMaxTokensPerSplit];
  float p[4][kTile][16];  // per wave: probabilities of the current tile, [token][head]
  float alpha[4][16];     // per wave: rescale of each head's state for the current tile
  AttnRed<G> red;         // per wave: final (o, m, l) of each head
};

struct GqaTile {
  uint4 k[4];      // K operand: 64 bytes of the lane's token row
  uint32_t v[16];  // V channels 2 lane, 2 lane + 1 of the tile's 16 tokens
};

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
  const int m16 = lane & 15;  // token of the K operand; head of the query operand and scores
  const int kg = lane >> 4;   // channel group [32 kg, 32 kg + 32)

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
  const __half* Vr = a.V + (int64_t)b * a.vs0 + (int64_t)g * a.vs1 + 2 * lane;
  float o[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) o[h][0] = o[h][1] = 0.0f;
  float m_run = kNegInf, l_run = 0.0f;  // head m16

  for (int bat = 0; bat < n_here; bat += kMaxTokensPerSplit) {
    const int nb = min(kMaxTokensPerSplit, n_here - bat);
    if (a.sparse) {
      __syncthreads();
      const int32_t* src = a.idx + (int64_t)row * a.idx_stride + t0 + bat;
      for (int i = tid; i < nb; i += kGT) f.lidx[i] = src[i];
      __syncthreads();
    }
    auto tok = [&](int i) -> int64_t { return a.sparse ? (int64_t)f.lidx[i] : (int64_t)(t0 + bat + i); };
    auto load = [&](int i0, GqaTile& T) {
      const int i = i0 + m16;
      const bool tv = i < nb;
      const int64_t t = tv ? tok(i) : 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        T.k[u] = make_uint4(0, 0, 0, 0);
        if (tv && 32 * kg + 8 * u < a.d_k) T.k[u] = ld_stream(Kr + t * a.ks2 + 8 * u);
      }
#pragma unroll
      for (int r = 0; r < kTile; ++r) {
        T.v[r] = 0u;
        if (i0 + r < nb) T.v[r] = *reinterpret_cast<const uint32_t*>(Vr + tok(i0 + r) * a.vs2);
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
        acc = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, pr), qb[s], acc, 0, 0,
                                                    0);
      }
      float sv[4];
      float tm = kNegInf;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sv[j] = i0 + 4 * kg + j < nb ? acc[j] * a.scale_log2 : kNegInf;
        tm = fmaxf(tm, sv[j]);
      }
      LanePair pr = xchg16(tm);  // over the four lane groups (tokens 4 kg + j)
      tm = fmaxf(pr.lo, pr.hi);
      pr = xchg32(tm);
      tm = fmaxf(pr.lo, pr.hi);
      const float mnew = fmaxf(m_run, tm);  // finite: token i0 of the tile is real
      const float al = m_run == kNegInf ? 0.0f : exp2f(m_run - mnew);
      float ps = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pj = sv[j] == kNegInf ? 0.0f : exp2f(sv[j] - mnew);
        f.p[w][4 * kg + j][m16] = pj;
        ps += pj;
      }
      pr = xchg16(ps);
      ps = pr.lo + pr.hi;
      pr = xchg32(ps);
      ps = pr.lo + pr.hi;
      l_run = l_run * al + ps;
      m_run = mnew;
      if (kg == 0) f.alpha[w][m16] = al;
      __builtin_amdgcn_wave_barrier();
      // P.V for channels 2 lane, 2 lane + 1 of every head
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float alh = f.alpha[w][h];
        o[h][0] *= alh;
        o[h][1] *= alh;
      }
#pragma unroll
      for (int r = 0; r < kTile; ++r) {
        const float2 vf = __half22float2(*reinterpret_cast<const __half2*>(&cur.v[r]));
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float ph = f.p[w][r][h];
          o[h][0] = fmaf(ph, vf.x, o[h][0]);
          o[h][1] = fmaf(ph, vf.y, o[h][1]);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }

  // The wave's state into LDS, then the four waves merged per head.
#pragma unroll
  for (int h = 0; h < G; ++h) {
    f.red.v[w][h][2 * lane] = o[h][0];
    f.red.v[w][h][2 * lane + 1] = o[h][1];
  }
  if (kg == 0 && m16 < G) {
    f.red.v[w][m16][kDv] = m_run;
    f.red.v[w][m16][kDv + 1] = l_run;
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
