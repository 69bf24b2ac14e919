// attn_gqa.hip -- attention pass for query groups of G >= 2 heads that share
// one K/V head ([GQA] section 4; [DS] "online forward computation", step 3:
// exact softmax attention over the selected tokens' full K/V rows; [LeanK]
// section 2.2: K stored as d_k kept columns, the query read at keep[c]).
//
// One workgroup of four waves per (row, split); each wave takes every fourth
// 16-token tile of the split's token list, with the loads of its next tile
// (splits of up to four tiles per wave) or next two tiles in flight while one
// is consumed (gqa_tile.h: both products of a tile on the matrix cores).  The
// four wave states are merged through LDS.
#include "gqa_tile.h"

namespace ds {
namespace {

constexpr int kGT = 256;  // threads per workgroup (4 waves)

template <int G>
struct GqaLds {
  alignas(16) __half q[G][kDv];  // the query rows at the stored K columns' channels
  int32_t lidx[kMaxTokensPerSplit];
  AttnRed<G> red;  // per wave: final (o, m, l) of each head
};

// RING: splits of more than four tiles per wave (the ring measured faster on
// long runs, the single prefetch on short ones).
template <int G, bool FINAL, bool RING>
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
  const int w = wave_id();
  const GqaLane ln(a, b, g);

  // The first batch of the token list and the query rows are fetched
  // together (one round trip, one barrier).
  const int32_t* src0 = a.idx + (int64_t)row * a.idx_stride + t0;
  if (a.sparse)
    for (int i = tid; i < min(n_here, kMaxTokensPerSplit); i += kGT) f.lidx[i] = src0[i];
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
  gqa_query(&f.q[0][0], G, ln, qb);

  GqaState st;
  gqa_init(st);
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
    constexpr int D = 4 * kGqaTile;  // the wave's tiles are D positions apart
    const int i_first = w * kGqaTile;
    if (i_first >= nb) continue;
    if (!RING) {
      // The next tile's loads in flight while one is consumed.
      GqaTile cur, nxt;
      gqa_load(a, ln, i_first, nb, tok, nxt);
      for (int i0 = i_first; i0 < nb; i0 += D) {
        cur = nxt;
        if (i0 + D < nb) gqa_load(a, ln, i0 + D, nb, tok, nxt);
        gqa_tile(cur, qb, i0, nb, a.scale_log2, ln.kg, st);
      }
    } else {
      // A ring of three tiles: two in flight while one is consumed.  Every
      // load is issued (up to two past the end read the last token again),
      // so each wait covers exactly one tile.
      GqaTile t0, t1, t2;
      gqa_load(a, ln, i_first, nb, tok, t0);
      gqa_load(a, ln, i_first + D, nb, tok, t1);
      for (int i0 = i_first; i0 < nb; i0 += 3 * D) {
        gqa_load(a, ln, i0 + 2 * D, nb, tok, t2);
        gqa_tile(t0, qb, i0, nb, a.scale_log2, ln.kg, st);
        if (i0 + D >= nb) break;
        gqa_load(a, ln, i0 + 3 * D, nb, tok, t0);
        gqa_tile(t1, qb, i0 + D, nb, a.scale_log2, ln.kg, st);
        if (i0 + 2 * D >= nb) break;
        gqa_load(a, ln, i0 + 4 * D, nb, tok, t1);
        gqa_tile(t2, qb, i0 + 2 * D, nb, a.scale_log2, ln.kg, st);
      }
    }
  }

  // The wave's state into LDS, then the four waves merged per head.
  gqa_to_red(st, ln, G, w, f.red);
  __syncthreads();
  attn_store<G, FINAL>(a, f.red, b, g, split);
}

template <int G>
hipError_t launch_g(const AttnArgs& a, int rows, bool final_out, hipStream_t s, const KEvents& ev) {
  const dim3 grid(rows * a.n_split);
  const bool ring = a.tps > 16 * kGqaTile;  // more than four tiles per wave
  if (final_out)
    return ring ? launch_k(k_attn_gqa<G, true, true>, grid, dim3(kGT), s, ev, a)
                : launch_k(k_attn_gqa<G, true, false>, grid, dim3(kGT), s, ev, a);
  return ring ? launch_k(k_attn_gqa<G, false, true>, grid, dim3(kGT), s, ev, a)
              : launch_k(k_attn_gqa<G, false, false>, grid, dim3(kGT), s, ev, a);
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
