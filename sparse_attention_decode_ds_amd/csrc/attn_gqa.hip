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
// long runs, the single prefetch on short ones).  PAGED: K/V in a paged pool;
// the staged list holds physical token ids (the dense path stages its
// positions too).
template <int G, bool FINAL, bool RING, bool PAGED>
__global__ __launch_bounds__(kGT) void k_attn_gqa(AttnArgs a_in) {
  __shared__ GqaLds<G> f;
  const SplitItem it = split_item(a_in, blockIdx.x);
  if (it.n == 0) return;  // every head pruned: the combine writes zeros
  const int b = it.b, g = it.g;
  const int row = b * a_in.Hkv + g;
  const AttnArgs a = with_head(a_in, g);
  const int tid = threadIdx.x;
  // With plain splits the first batch of the split's token list depends on
  // the kernel arguments only: its loads go out before the row's length and
  // count arrive (entries past the count are read but never used).
  constexpr int kPre = kMaxTokensPerSplit / kGT;
  const bool early = a.sparse && !split_by_bytes(a);
  int32_t pre[kPre];
  if (early) {
    const int te = it.split * a.tps;
    const int32_t* src = a.idx + (int64_t)row * a.idx_stride + te;
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int i = u * kGT + tid;
      pre[u] = (i < a.tps && te + i < a.idx_stride) ? src[i] : 0;
    }
  }
  const int S = min(max(a.seq_lens[b], 0), a.max_seq);
  // a fully pruned head (no K columns) attends nothing: zero output
  const int n_tok = a.d_k == 0 ? 0 : (a.sparse ? min(a.count[row], S) : S);
  const int tps = split_tokens(a, it, n_tok);
  const int t0 = it.split * tps;
  const int n_here = max(0, min(n_tok - t0, tps));
  const int w = wave_id();
  const GqaLane ln(a, b, g, PAGED);
  const int32_t* ptab = PAGED ? a.ptab + (int64_t)b * a.max_pages : nullptr;
  // list position -> token (physical id in a paged pool), staged in LDS
  auto stage = [&](int pos) -> int32_t {
    const int t = a.sparse ? a.idx[(int64_t)row * a.idx_stride + pos] : pos;
    return PAGED ? phys_tok(ptab, a.pshift, t) : t;
  };
  constexpr bool kStaged = PAGED;  // dense positions are staged too when paged

  // The first batch of the token list and the query rows are fetched
  // together (one round trip, one barrier).
  if (early) {
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int i = u * kGT + tid;
      if (i < min(n_here, kMaxTokensPerSplit))
        f.lidx[i] = PAGED ? phys_tok(ptab, a.pshift, pre[u]) : pre[u];
    }
  } else if (a.sparse || kStaged) {
    for (int i = tid; i < min(n_here, kMaxTokensPerSplit); i += kGT) f.lidx[i] = stage(t0 + i);
  }
  // The query rows at the stored K columns' channels into registers: thread
  // tid holds channel c = tid mod 128 of heads tid / 128, + 2, + 4, + 6.
  constexpr int kQPer = kMaxGroup * kDv / kGT;
  static_assert(kGT % kDv == 0, "one channel per thread");
  const int qc = tid & (kDv - 1);
  __half qv[kQPer];
  {
    const int kc = qc < a.d_k ? (a.keep ? a.keep[(int64_t)g * a.keep_ld + qc] : qc) : 0;
    const __half* qh = a.q + ((int64_t)b * a.Hq + (int64_t)g * G) * a.d_q + kc;
#pragma unroll
    for (int m = 0; m < kQPer; ++m) {
      const int h = tid / kDv + m * (kGT / kDv);
      qv[m] = (h < G && qc < a.d_k) ? qh[(int64_t)h * a.d_q] : __float2half(0.0f);
    }
  }
  auto stage_query = [&]() {
#pragma unroll
    for (int m = 0; m < kQPer; ++m) {
      const int h = tid / kDv + m * (kGT / kDv);
      if (h < G) f.q[h][qc] = qv[m];
    }
  };
  constexpr int D = 4 * kGqaTile;  // the wave's tiles are D positions apart
  const int i_first = w * kGqaTile;
  const int nb0 = min(kMaxTokensPerSplit, n_here);
  GqaTile nxt;
  if (RING) {
    stage_query();
    __syncthreads();
  } else {
    // The first tile's loads go out before the query (behind the keep
    // table, a second round trip) is staged.
    __syncthreads();
    auto tok0 = [&](int i) -> int64_t {
      return (a.sparse || kStaged) ? (int64_t)f.lidx[i] : (int64_t)(t0 + i);
    };
    if (i_first < nb0) gqa_load<PAGED>(a, ln, i_first, nb0, tok0, nxt);
    stage_query();
    __syncthreads();
  }
  half4_t qb[8];
  gqa_query(&f.q[0][0], G, ln, qb);

  GqaState st;
  gqa_init(st);
  for (int bat = 0; bat < n_here; bat += kMaxTokensPerSplit) {
    const int nb = min(kMaxTokensPerSplit, n_here - bat);
    if ((a.sparse || kStaged) && bat > 0) {
      __syncthreads();
      for (int i = tid; i < nb; i += kGT) f.lidx[i] = stage(t0 + bat + i);
      __syncthreads();
    }
    auto tok = [&](int i) -> int64_t {
      return (a.sparse || kStaged) ? (int64_t)f.lidx[i] : (int64_t)(t0 + bat + i);
    };
    if (i_first >= nb) continue;
    if (!RING) {
      // The next tile's loads in flight while one is consumed (the first
      // batch's first tile was issued in the prologue).
      GqaTile cur;
      if (bat > 0) gqa_load<PAGED>(a, ln, i_first, nb, tok, nxt);
      for (int i0 = i_first; i0 < nb; i0 += D) {
        cur = nxt;
        if (i0 + D < nb) gqa_load<PAGED>(a, ln, i0 + D, nb, tok, nxt);
        gqa_tile(cur, qb, i0, nb, a.scale_log2, ln.kg, st);
      }
    } else {
      // A ring of three tiles: two in flight while one is consumed.  Every
      // load is issued (up to two past the end read the last token again),
      // so each wait covers exactly one tile.
      GqaTile t0, t1, t2;
      gqa_load<PAGED>(a, ln, i_first, nb, tok, t0);
      gqa_load<PAGED>(a, ln, i_first + D, nb, tok, t1);
      for (int i0 = i_first; i0 < nb; i0 += 3 * D) {
        gqa_load<PAGED>(a, ln, i0 + 2 * D, nb, tok, t2);
        gqa_tile(t0, qb, i0, nb, a.scale_log2, ln.kg, st);
        if (i0 + D >= nb) break;
        gqa_load<PAGED>(a, ln, i0 + 3 * D, nb, tok, t0);
        gqa_tile(t1, qb, i0 + D, nb, a.scale_log2, ln.kg, st);
        if (i0 + 2 * D >= nb) break;
        gqa_load<PAGED>(a, ln, i0 + 4 * D, nb, tok, t1);
        gqa_tile(t2, qb, i0 + 2 * D, nb, a.scale_log2, ln.kg, st);
      }
    }
  }

  // The wave's state into LDS, then the four waves merged per head.
  gqa_to_red(st, ln, G, w, f.red);
  __syncthreads();
  attn_store<G, FINAL>(a, f.red, b, g, it.split);
}

template <int G, bool PAGED>
hipError_t launch_gp(const AttnArgs& a, int rows, bool final_out, hipStream_t s, const KEvents& ev) {
  const dim3 grid(rows * a.n_split);
  const bool ring = a.tps > 16 * kGqaTile;  // more than four tiles per wave
  if (final_out)
    return ring ? launch_k(k_attn_gqa<G, true, true, PAGED>, grid, dim3(kGT), s, ev, a)
                : launch_k(k_attn_gqa<G, true, false, PAGED>, grid, dim3(kGT), s, ev, a);
  return ring ? launch_k(k_attn_gqa<G, false, true, PAGED>, grid, dim3(kGT), s, ev, a)
              : launch_k(k_attn_gqa<G, false, false, PAGED>, grid, dim3(kGT), s, ev, a);
}

template <int G>
hipError_t launch_g(const AttnArgs& a, int rows, bool final_out, hipStream_t s, const KEvents& ev) {
  return a.ptab ? launch_gp<G, true>(a, rows, final_out, s, ev)
                : launch_gp<G, false>(a, rows, final_out, s, ev);
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
