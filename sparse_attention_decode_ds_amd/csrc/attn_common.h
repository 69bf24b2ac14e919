// attn_common.h -- device code for step 3b of a Double Sparsity decode step:
// exact softmax attention over a set of tokens' full K/V rows.
//
// [DS] "online forward computation", step 3: attention over the top-k tokens
// uses the full query, K and V (not the channel-sparse ones).  [GQA] section
// 4: the G query heads of a group read the same K/V rows, so each selected row
// is loaded once and applied to all G heads.  [LeanK] section 2.2: K may be
// stored compacted to d_k kept columns; the query is read at those channels.
//
// Layout: a workgroup of 4 waves = 16 rows of 16 lanes ("slots").  Each slot
// walks its own tokens; lane c holds K and V channels [8c, 8c+8) as one
// 16-byte load each and keeps an online-softmax state per head (running max m
// in the log2 domain, sum l, unnormalised output o).  Loads of the next group
// of tokens are in flight while the current group is consumed (two register
// buffers in ping-pong).  The 16 states are merged with shuffles and LDS.
#pragma once

#include "ds_internal.h"

namespace ds {

constexpr int kAttnThreads = 256;
constexpr int kSlots = 16;
constexpr int kUnroll = 4;  // tokens per slot and group
constexpr float kNegInf = -__builtin_huge_valf();

template <int G>
struct AttnAcc {
  float o[G][8];
  float m[G];
  float l[G];
};

// Per wave: final (o, m, l) of each head.
template <int G, int NW = 4>
struct AttnRed {
  alignas(16) float v[NW][G][kDv + 4];  // o[0 .. kDv), m, l, 2 floats of padding
};

// ---- Work items of the split attention pass ----
// Plain layouts (and one split per row): workgroup blk takes split
// blk % n_split of row blk / n_split, each split `tps` tokens long.
// Per-head layouts with several splits (up to 64 KV heads): the heads differ
// in bytes per token (kept K columns plus the V row; none for a pruned head),
// so the R = Hkv * n_split workgroups of a batch row are dealt to its heads by
// those bytes w_g, keeping the largest bytes per workgroup, max w_g / n_g,
// low.  Every storing head first gets 1 + floor((R - live) * w_g / wtot)
// (live: the storing heads, wtot: the sum of their w_g), which leaves
// u < live workgroups over; those go one each to the u heads with the most
// bytes per workgroup so far (ties to the lower head).  A pruned head gets
// none, and a head's splits share its token list evenly.  Head g takes the
// row's work items [cum(g - 1), cum(g)).  Partial results: plain layouts keep
// the splits of a query head together (slot (row * G + h) * n_split +
// split); byte-dealt work items write slots blk * G + h.
struct SplitItem {
  int b, g, split, n;  // batch row, KV head, split of n (n == 0: no work)
};

constexpr int kMaxByteSplitHeads = 64;  // one lane per head

__device__ __forceinline__ bool split_by_bytes(const AttnArgs& a) {
  return a.heads != nullptr && a.n_split > 1 && a.Hkv <= kMaxByteSplitHeads;
}

// cum(g) for the head g = lane of the calling lane (lanes past the last head:
// R, or 0 when no head stores anything).  Every lane of the wave calls it.
__device__ __forceinline__ uint32_t head_cum(const AttnArgs& a) {
  const int lane = threadIdx.x & 63;
  uint32_t w = 0;
  if (lane < a.Hkv) {
    const uint32_t kc = (uint32_t)a.heads[lane].k_cols;
    w = kc ? kc + (uint32_t)kDv : 0u;
  }
  const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(w), 63);
  const uint32_t live = (uint32_t)__popcll(__ballot(w != 0u));
  if (live == 0) return 0u;
  const uint32_t R = (uint32_t)(a.Hkv * a.n_split);
  uint32_t n = w ? 1u + (R - live) * w / wtot : 0u;
  const uint32_t u = R - (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(n), 63);
  // bytes per workgroup as a fixed-point key, made unique by the lane
  const uint32_t key = w ? (((w << 16) / n) << 6) | (uint32_t)(63 - lane) : 0u;
  uint32_t rank = 0;
  for (int j = 0; j < a.Hkv; ++j) rank += (uint32_t)__builtin_amdgcn_readlane((int)key, j) > key;
  n += (w && rank < u) ? 1u : 0u;
  return wave_incl_scan(n);
}

// The work item of attention workgroup blk (uniform over the workgroup).
__device__ __forceinline__ SplitItem split_item(const AttnArgs& a, int blk) {
  SplitItem it;
  if (!split_by_bytes(a)) {
    const int row = blk / a.n_split;
    it.split = blk - row * a.n_split;
    it.b = row / a.Hkv;
    it.g = row - it.b * a.Hkv;
    it.n = a.n_split;
    return it;
  }
  const int R = a.Hkv * a.n_split;
  it.b = blk / R;
  const uint32_t r = (uint32_t)(blk - it.b * R);
  const uint32_t c = head_cum(a);
  const int lane = threadIdx.x & 63;
  // cum is non-decreasing over the heads: the first k end at or before r
  const int k = __popcll(__ballot(lane < a.Hkv && c <= r));
  if (k >= a.Hkv) {  // no head stores anything
    it.g = 0;
    it.split = 0;
    it.n = 0;
    return it;
  }
  const uint32_t lo = k ? (uint32_t)__builtin_amdgcn_readlane((int)c, k - 1) : 0u;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)c, k);
  it.g = k;
  it.split = (int)(r - lo);
  it.n = (int)(hi - lo);
  return it;
}

// Tokens per split of a work item whose head attends n_tok tokens.
__device__ __forceinline__ int split_tokens(const AttnArgs& a, const SplitItem& it, int n_tok) {
  if (!split_by_bytes(a)) return a.tps;
  return max(16, (((n_tok + it.n - 1) / it.n + 15) / 16) * 16);
}

// The work items [base, base + n) of head g (each lane its own g < Hkv)
// within its batch row, for byte-dealt splits.  Every lane of the wave calls it.
__device__ __forceinline__ void head_items(const AttnArgs& a, int g, int& base, int& n) {
  const uint32_t c = head_cum(a);
  const uint32_t hi = (uint32_t)__shfl((int)c, g);
  const uint32_t lo = (uint32_t)__shfl((int)c, max(g - 1, 0));
  base = g ? (int)lo : 0;
  n = (int)(hi - (uint32_t)base);
}

// Merge weights of two online-softmax states; either may be empty (m = -inf).
__device__ __forceinline__ void merge_weights(float m, float m2, float& w1, float& w2, float& mx) {
  mx = fmaxf(m, m2);
  w1 = (m == kNegInf) ? 0.0f : exp2f(m - mx);
  w2 = (m2 == kNegInf) ? 0.0f : exp2f(m2 - mx);
}

// Query of each head at stored-K channels [8c, 8c+8), scaled so that exp2 of
// the dot product is exp of the logit; zero for lanes past d_k.
template <int G>
__device__ __forceinline__ void load_query(const AttnArgs& a, int b, int g, int c, bool kl,
                                           float (&qf)[G][8]) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const __half* qh = a.q + ((int64_t)b * a.Hq + (int64_t)g * G + h) * a.d_q;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v = 0.0f;
      if (kl) {
        const int ch = c * 8 + i;
        const int qc = a.keep ? a.keep[(int64_t)g * a.keep_ld + ch] : ch;
        v = h2f(qh[qc]) * a.scale_log2;
      }
      qf[h][i] = v;
    }
  }
}

template <int G>
__device__ __forceinline__ void acc_init(AttnAcc<G>& acc) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    acc.m[h] = kNegInf;
    acc.l[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc.o[h][i] = 0.0f;
  }
}

// Token loads of one slot in flight: two groups of kUnroll tokens (list
// positions base + 16 u), consumed alternately.
struct AttnLoads {
  uint4 ka[kUnroll], va[kUnroll], kb[kUnroll], vb[kUnroll];
};

// Element offsets of token t's K and V rows from the row's base pointers:
// t * stride for contiguous rows; for a paged pool t is a physical id
// (page << pshift | slot) and the base pointers exclude the batch row.
template <bool PAGED>
__device__ __forceinline__ int64_t k_off(const AttnArgs& a, int64_t t) {
  return PAGED ? (t >> a.pshift) * a.ks0 + (t & a.pmask) * a.ks2 : t * a.ks2;
}
template <bool PAGED>
__device__ __forceinline__ int64_t v_off(const AttnArgs& a, int64_t t) {
  return PAGED ? (t >> a.pshift) * a.vs0 + (t & a.pmask) * a.vs2 : t * a.vs2;
}

// Loads of the tokens tok(i), i = base + 16 u, into kk/vv.  Positions at or
// past hi load the list's first token tok(0) instead (the row's token 0 if
// the list is still empty): every load is issued unconditionally, so no
// register holding a load in flight is ever merged or cleared; the consumer
// masks those positions out, and their values are finite wherever the
// selected rows are.  Kr, Vr point at the lane's 16-byte piece of the row's
// token 0 (lanes past the stored K width read a valid column; their query
// weights are zero); for a paged pool, at page 0's and tok gives physical
// ids.
template <bool PAGED, typename TokFn>
__device__ __forceinline__ void attn_issue(const AttnArgs& a, const __half* Kr, const __half* Vr,
                                           int base, int hi, TokFn tok, uint4* kk, uint4* vv) {
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int i = base + u * kSlots;
    const int64_t t = hi > 0 ? tok(i < hi ? i : 0) : 0;  // (paged: page 0, slot 0)
    kk[u] = ld_stream(Kr + k_off<PAGED>(a, t));
    vv[u] = ld_stream(Vr + v_off<PAGED>(a, t));
  }
}

// The first two groups of slot `slot`, positions [0, n).
template <bool PAGED, typename TokFn>
__device__ __forceinline__ void attend_prime(const AttnArgs& a, const __half* Kr, const __half* Vr,
                                             int slot, int n, TokFn tok, AttnLoads& L) {
  constexpr int kStep = kSlots * kUnroll;
  attn_issue<PAGED>(a, Kr, Vr, slot, n, tok, L.ka, L.va);
  attn_issue<PAGED>(a, Kr, Vr, slot + kStep, n, tok, L.kb, L.vb);
}

// Accumulate tokens tok(i), i in [0, n), slot `slot` taking i = slot, slot+16, ...,
// with the first two groups already in L (attend_prime); each group is
// reloaded with the group after next as soon as it is consumed.
template <int G, bool PAGED, typename TokFn>
__device__ __forceinline__ void attend_run(const AttnArgs& a, const __half* Kr, const __half* Vr,
                                           int slot, int n, TokFn tok, const float (&qf)[G][8],
                                           AttnAcc<G>& acc, AttnLoads& L) {
  constexpr int kStep = kSlots * kUnroll;
  auto consume = [&](int base, const uint4* kk, const uint4* vv) {
    float s[kUnroll][G];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float kf[8];
      unpack8(kk[u], kf);
      const bool valid = base + u * kSlots < n;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) d += qf[h][i] * kf[i];
        d = row16_sum(d);
        s[u][h] = valid ? d : kNegInf;
      }
    }
    float vf[kUnroll][8];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) unpack8(vv[u], vf[u]);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = acc.m[h];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) mx = fmaxf(mx, s[u][h]);
      if (mx == kNegInf) continue;
      const float alpha = exp2f(acc.m[h] - mx);
      float p[kUnroll];
      float ps = 0.0f;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        p[u] = exp2f(s[u][h] - mx);
        ps += p[u];
      }
      acc.l[h] = acc.l[h] * alpha + ps;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float o = acc.o[h][i] * alpha;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) o += p[u] * vf[u][i];
        acc.o[h][i] = o;
      }
      acc.m[h] = mx;
    }
  };
  for (int base = slot; base < n; base += 2 * kStep) {
    consume(base, L.ka, L.va);
    if (base + 2 * kStep < n) attn_issue<PAGED>(a, Kr, Vr, base + 2 * kStep, n, tok, L.ka, L.va);
    if (base + kStep >= n) break;
    consume(base + kStep, L.kb, L.vb);
    if (base + 3 * kStep < n) attn_issue<PAGED>(a, Kr, Vr, base + 3 * kStep, n, tok, L.kb, L.vb);
  }
}

template <int G, bool PAGED, typename TokFn>
__device__ __forceinline__ void attend(const AttnArgs& a, const __half* Kr, const __half* Vr,
                                       int slot, int n, TokFn tok, const float (&qf)[G][8],
                                       AttnAcc<G>& acc) {
  if (n <= 0) return;
  AttnLoads L;
  attend_prime<PAGED>(a, Kr, Vr, slot, n, tok, L);
  attend_run<G, PAGED>(a, Kr, Vr, slot, n, tok, qf, acc, L);
}

template <int G, bool FINAL, int NW = 4>
__device__ __forceinline__ void attn_store(const AttnArgs& a, AttnRed<G, NW>& red, int b, int g,
                                           int split, int ng = G);

// Merge the 16 slot states and write either the fp16 output (FINAL) or the
// (o, m, l) partial of split `split`.  Every thread of the workgroup calls it.
template <int G, bool FINAL>
__device__ __forceinline__ void attn_finish(const AttnArgs& a, AttnAcc<G>& acc, AttnRed<G>& red,
                                            int b, int g, int split) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_id();
  const int c = lane & 15;
  // slots 4w + s merge with slot 4w + (s ^ 1), then with 4w + (s ^ 2): the
  // lanes 16 and 32 apart (both lanes of a pair compute the same state)
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
    auto xchg = [&](float x) { return off == 16 ? xchg16(x) : xchg32(x); };
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const LanePair pm = xchg(acc.m[h]);
      const LanePair pl = xchg(acc.l[h]);
      float w1, w2, mx;
      merge_weights(pm.lo, pm.hi, w1, w2, mx);
      acc.l[h] = pl.lo * w1 + pl.hi * w2;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const LanePair po = xchg(acc.o[h][i]);
        acc.o[h][i] = po.lo * w1 + po.hi * w2;
      }
      acc.m[h] = mx;
    }
  }
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int i = 0; i < 8; ++i) red.v[w][h][c * 8 + i] = acc.o[h][i];
      if (c == 0) {
        red.v[w][h][kDv] = acc.m[h];
        red.v[w][h][kDv + 1] = acc.l[h];
      }
    }
  }
  __syncthreads();
  if (tid >= G * 16) return;
  attn_store<G, FINAL>(a, red, b, g, split);
}

// Workgroup merge of the NW wave states in `red` and the store, by threads
// (h, c) with h < ng (the others do nothing); ng <= G heads in the group.
// Partial slots as split_item describes (blockIdx.x is the work item).
template <int G, bool FINAL, int NW>
__device__ __forceinline__ void attn_store(const AttnArgs& a, AttnRed<G, NW>& red, int b, int g,
                                           int split, int ng) {
  const int tid = threadIdx.x;
  if (tid >= ng * 16) return;
  const int h = tid >> 4;
  const int cc = tid & 15;
  float M = kNegInf;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, red.v[ww][h][kDv]);
  float L = 0.0f, O[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) O[i] = 0.0f;
  if (M != kNegInf) {
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float mw = red.v[ww][h][kDv];
      if (mw == kNegInf) continue;
      const float sc = exp2f(mw - M);
      L += sc * red.v[ww][h][kDv + 1];
#pragma unroll
      for (int i = 0; i < 8; ++i) O[i] += sc * red.v[ww][h][cc * 8 + i];
    }
  }
  const int64_t bh = (int64_t)b * a.Hq + (int64_t)g * ng + h;
  if (FINAL) {
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    __half2 r2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) r2[i] = __floats2half2_rn(O[2 * i] * inv, O[2 * i + 1] * inv);
    *reinterpret_cast<uint4*>(a.out + bh * kDv + cc * 8) = *reinterpret_cast<const uint4*>(r2);
  } else {
    const int64_t slot =
        split_by_bytes(a) ? (int64_t)blockIdx.x * ng + h : bh * a.n_split + split;
    float* dst = a.part + slot * kPartStride;
    *reinterpret_cast<float4*>(dst + cc * 8) = make_float4(O[0], O[1], O[2], O[3]);
    *reinterpret_cast<float4*>(dst + cc * 8 + 4) = make_float4(O[4], O[5], O[6], O[7]);
    if (cc == 0) {
      dst[kDv] = M;
      dst[kDv + 1] = L;
    }
  }
}

// Log-sum-exp merge of the n partials at p, p + stride, ... of one query
// head row (16 lanes, lane c covers channels [8c, 8c+8)) into its fp16
// output row `out`.  The partials are read in groups of 8 whose loads are all
// in flight together, and merged into a running (max, sum, output) state.
__device__ __forceinline__ void merge_partials(const float* p, int n, int64_t stride, __half* out,
                                               int c) {
  constexpr int kB = 8;
  float M = kNegInf, L = 0.0f, O[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) O[i] = 0.0f;
  for (int s0 = 0; s0 < n; s0 += kB) {
    float4 x0[kB], x1[kB];
    float m[kB], l[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      m[u] = kNegInf;
      l[u] = 0.0f;
      x0[u] = x1[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (s0 + u < n) {
        const float* q = p + (int64_t)(s0 + u) * stride;
        x0[u] = *reinterpret_cast<const float4*>(q + c * 8);
        x1[u] = *reinterpret_cast<const float4*>(q + c * 8 + 4);
        const float2 ml = *reinterpret_cast<const float2*>(q + kDv);
        m[u] = ml.x;
        l[u] = ml.y;
      }
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < kB; ++u) Mn = fmaxf(Mn, m[u]);
    if (Mn == kNegInf) continue;  // every partial so far is empty
    const float al = M == kNegInf ? 0.0f : exp2f(M - Mn);
    L *= al;
#pragma unroll
    for (int i = 0; i < 8; ++i) O[i] *= al;
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const float w = m[u] == kNegInf ? 0.0f : exp2f(m[u] - Mn);
      L += w * l[u];
      O[0] += w * x0[u].x;
      O[1] += w * x0[u].y;
      O[2] += w * x0[u].z;
      O[3] += w * x0[u].w;
      O[4] += w * x1[u].x;
      O[5] += w * x1[u].y;
      O[6] += w * x1[u].z;
      O[7] += w * x1[u].w;
    }
    M = Mn;
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  __half2 r2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) r2[i] = __floats2half2_rn(O[2 * i] * inv, O[2 * i + 1] * inv);
  *reinterpret_cast<uint4*>(out + c * 8) = *reinterpret_cast<const uint4*>(r2);
}

}  // namespace ds
