// score_common.h -- device code shared by the score/select kernels: the
// query gather (step 1), the approximate score over the label cache (step 2)
// and the exact top-k select (step 3a) of a Double Sparsity decode step.
//
// [DS] "online forward computation": step 1 takes the query at the heavy
// channels into a contiguous vector, step 2 scores every cached token from
// that vector and the contiguous label cache, step 3 keeps the k tokens with
// the largest scores.  Under GQA ([GQA] section 4) one token set serves the
// group of query heads; its score is the sum of the heads' scores, i.e. the
// gathered queries are summed first.
//
// Selection (exact, ties to the lower token index).  Scores become
// order-preserving uint32 keys.  A first histogram uses 2048 linear bins
// between the row's smallest and largest score; the bin index is a monotone
// function of the score, so every key in a higher bin is larger than every key
// in a lower one.  The bin that holds the k-th largest key is then resolved
// exactly: by counting ranks when it holds at most kRankMax keys (the usual
// case), otherwise by radix passes over the key bits restricted to that bin.
// The result is a class per key: taken, not taken, or "equal" (taken lowest
// index first up to a quota), and an ordered output pass writes the set in
// ascending token order.
#pragma once

#include "ds_internal.h"

namespace ds {

constexpr int kHistBins = 2048;
constexpr int kRankMax = 256;

struct RowPtrs {
  const __half* lab16;
  const uint8_t* codes;
  const __half* scales;
};

__device__ __forceinline__ RowPtrs row_ptrs(const ScoreArgs& a, int row) {
  RowPtrs p;
  const int64_t base = (int64_t)row * a.slots;
  p.lab16 = a.lab16 ? a.lab16 + base * a.r : nullptr;
  p.codes = a.codes ? a.codes + base * (a.r >> 1) : nullptr;
  p.scales = a.scales ? a.scales + base : nullptr;
  return p;
}

// ---------------------------------------------------------------------------
// Step 1: the gathered query, kept in LDS in two forms.
// ---------------------------------------------------------------------------
// qg[j] (fp32) for every label dtype.  For int4 labels with r <= 16 also a
// fixed-point copy: with e the exponent such that max_j |qg[j]| < 2^e,
// qi[j] = rint(qg[j] * 2^(kQBits - e)) is split into kQDigits balanced
// base-16 digits in [-8, 7] (five digits hold any |qi| <= 2^18: their range
// is [-559240, 489335]); dig[w][d] packs digit d of channels 8w .. 8w + 7
// (nibble i = channel 8w + i, the order of the int4 codes).  Then
// sum_j qi[j] * c[j] = sum_d 16^d * (4-bit dot products of dig[.][d] with the
// code words), exactly in int32 (|qi| <= 2^18, |c| <= 7, r <= 16), and the
// score is that integer times the token's scale.  The row's common factor
// 2^(e - kQBits) is left out: an exact power of two that scales every score
// of the row alike, it changes no comparison, so no selected set.  The
// query's rounding, at most 2^-18 of max|qg| per channel, lies far below the
// 4-bit labels' own (a code step is 1/7 of the token's largest label).
constexpr int kQBits = 18;
constexpr int kQDigits = 5;
struct QueryLds {
  float qg[128];
  uint32_t dig[2][kQDigits];
};

// Reductions over lanes 0 .. 15 of a wave with DPP row shifts (lanes with no
// source read 0, so the inputs must be >= 0 for the max): after the call
// lane 15 holds the result over lanes 0 .. 15, and for the OR lane 7 holds
// the OR over lanes 0 .. 7.
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, true)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, true)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, true)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, true)));
  return x;
}
__device__ __forceinline__ uint32_t row_or8(uint32_t x) {
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);  // row_shr:4
  return x;
}

// Fixed-point digits of the query (one whole wave; lane j < r <= 16 holds
// qg[j]).
__device__ __forceinline__ void make_qdig(float qgv, int r, QueryLds& q) {
  const int lane = threadIdx.x & 63;
  const bool on = lane < r;
  const float amax =
      __int_as_float(__builtin_amdgcn_readlane(__float_as_int(row_max16(on ? fabsf(qgv) : 0.0f)), 15));
  const int e = amax > 0.0f ? ilogbf(amax) + 1 : 0;
  int x = on ? (int)rintf(ldexpf(qgv, kQBits - e)) : 0;
#pragma unroll
  for (int d = 0; d < kQDigits; ++d) {
    const int dg = ((x + 8) & 15) - 8;
    x = (x - dg) / 16;  // exact: x - dg is a multiple of 16
    const uint32_t wd = row_or8(on ? (uint32_t)(dg & 15) << (4 * (lane & 7)) : 0u);
    if (lane == 7) q.dig[0][d] = wd;
    if (lane == 15) q.dig[1][d] = wd;
  }
}

// Thread tid < r holds qg[tid] in qgv: store it, and for int4 labels with
// r <= 16 let wave 0 derive the digits.  The caller synchronises afterwards.
__device__ __forceinline__ void store_query(bool int4, int r, float qgv, QueryLds& q) {
  const int tid = threadIdx.x;
  if (tid < r) q.qg[tid] = qgv;
  if (int4 && r <= 16 && tid < 64) make_qdig(tid < r ? qgv : 0.0f, r, q);
}

// qg[j] = sum over the group's query heads of q[h][keep[chan[j]]], read from
// global memory (blockDim.x >= r).
__device__ __forceinline__ void gather_query(const ScoreArgs& a, int b, int g, QueryLds& q) {
  const int j = threadIdx.x;
  float acc = 0.0f;
  if (j < a.r) {
    const int col = a.chan[(int64_t)g * a.r + j];
    const int qc = a.keep ? a.keep[(int64_t)g * a.keep_ld + col] : col;
    const __half* qh = a.q + ((int64_t)b * a.Hq + (int64_t)g * a.G) * a.d_q + qc;
    for (int h = 0; h < a.G; ++h) acc += h2f(qh[(int64_t)h * a.d_q]);
  }
  store_query(a.is_int4 != 0, a.r, acc, q);
}

// Query operands in registers, one type per label vector.
template <int R>
struct QFloat {
  float v[R];
  __device__ __forceinline__ void load(const QueryLds& l) {
#pragma unroll
    for (int j = 0; j < R; ++j) v[j] = l.qg[j];
  }
};
template <int W>
struct QDig {
  uint32_t d[W][kQDigits];
  __device__ __forceinline__ void load(const QueryLds& l) {
#pragma unroll
    for (int w = 0; w < W; ++w)
#pragma unroll
      for (int i = 0; i < kQDigits; ++i) d[w][i] = l.dig[w][i];
  }
};
struct QPtr {
  const float* qg;
  __device__ __forceinline__ void load(const QueryLds& l) { qg = l.qg; }
};

// sum_j qi[j] * c[j] for the code words w[0 .. W-1] (8 channels each).
template <int W>
__device__ __forceinline__ int dot_dig(const QDig<W>& q, const uint32_t* w) {
  int acc = 0;
#pragma unroll
  for (int d = kQDigits - 1; d >= 0; --d) {
    acc *= 16;
#pragma unroll
    for (int i = 0; i < W; ++i) acc = __builtin_amdgcn_sdot8((int)q.d[i][d], (int)w[i], acc, false);
  }
  return acc;
}

// The same for N tokens at once (token n's code words at w + n * W), the N
// integer chains interleaved digit by digit so that their instructions fill
// each other's dependency stalls; every result equals dot_dig's.
template <int W, int N>
__device__ __forceinline__ void dot_dig_n(const QDig<W>& q, const uint32_t* w, int* acc) {
#pragma unroll
  for (int n = 0; n < N; ++n) acc[n] = 0;
#pragma unroll
  for (int d = kQDigits - 1; d >= 0; --d) {
#pragma unroll
    for (int n = 0; n < N; ++n) acc[n] *= 16;
#pragma unroll
    for (int i = 0; i < W; ++i)
#pragma unroll
      for (int n = 0; n < N; ++n)
        acc[n] = __builtin_amdgcn_sdot8((int)q.d[i][d], (int)w[n * W + i], acc[n], false);
  }
}

__device__ __forceinline__ int nib(uint32_t w, int j) {
  return (int)(w << (28 - 4 * j)) >> 28;  // signed nibble j
}

// Step 2 for one vector of VT consecutive tokens.  R = 0 is the generic
// path (any r, scalar loads, fmaf over j in order).  int4 labels with r = 8
// or 16 use the exact integer dot products of the fixed-point query; fp16
// labels accumulate fmaf(qg[j], label[j], acc) over j in order.  The label
// append computes the new token's score the same way, so a token's score
// does not depend on which kernel computes it.
template <int R, bool INT4>
struct LabelVec;

template <>
struct LabelVec<8, true> {  // 4 tokens: 16 B of codes + 8 B of scales
  static constexpr int VT = 4;
  using Q = QDig<1>;
  uint4 c;
  uint2 s;
  __device__ __forceinline__ void load(const RowPtrs& p, int v) {
    c = ld_stream(reinterpret_cast<const uint4*>(p.codes) + v);
    s = reinterpret_cast<const uint2*>(p.scales)[v];
  }
  __device__ __forceinline__ void score(const Q& q, int, float* out) const {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    const __half2 s01 = *reinterpret_cast<const __half2*>(&s.x);
    const __half2 s23 = *reinterpret_cast<const __half2*>(&s.y);
    const float sc[4] = {__low2float(s01), __high2float(s01), __low2float(s23), __high2float(s23)};
    int acc[4];
    dot_dig_n<1, 4>(q, w, acc);
#pragma unroll
    for (int u = 0; u < 4; ++u) out[u] = (float)acc[u] * sc[u];
  }
};

template <>
struct LabelVec<16, true> {  // 2 tokens: 16 B of codes + 4 B of scales
  static constexpr int VT = 2;
  using Q = QDig<2>;
  uint4 c;
  uint32_t s;
  __device__ __forceinline__ void load(const RowPtrs& p, int v) {
    c = ld_stream(reinterpret_cast<const uint4*>(p.codes) + v);
    s = reinterpret_cast<const uint32_t*>(p.scales)[v];
  }
  __device__ __forceinline__ void score(const Q& q, int, float* out) const {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    const __half2 s01 = *reinterpret_cast<const __half2*>(&s);
    const float sc[2] = {__low2float(s01), __high2float(s01)};
    int acc[2];
    dot_dig_n<2, 2>(q, w, acc);
#pragma unroll
    for (int u = 0; u < 2; ++u) out[u] = (float)acc[u] * sc[u];
  }
};

template <>
struct LabelVec<8, false> {  // 1 token: 8 fp16 labels
  static constexpr int VT = 1;
  using Q = QFloat<8>;
  uint4 c;
  __device__ __forceinline__ void load(const RowPtrs& p, int v) {
    c = ld_stream(reinterpret_cast<const uint4*>(p.lab16) + v);
  }
  __device__ __forceinline__ void score(const Q& q, int, float* out) const {
    float f[8];
    unpack8(c, f);
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = fmaf(q.v[j], f[j], acc);
    out[0] = acc;
  }
};

template <>
struct LabelVec<16, false> {  // 1 token: 16 fp16 labels
  static constexpr int VT = 1;
  using Q = QFloat<16>;
  uint4 c0, c1;
  __device__ __forceinline__ void load(const RowPtrs& p, int v) {
    c0 = ld_stream(reinterpret_cast<const uint4*>(p.lab16) + 2 * v);
    c1 = ld_stream(reinterpret_cast<const uint4*>(p.lab16) + 2 * v + 1);
  }
  __device__ __forceinline__ void score(const Q& q, int, float* out) const {
    float f[16];
    unpack8(c0, f);
    unpack8(c1, f + 8);
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc = fmaf(q.v[j], f[j], acc);
    out[0] = acc;
  }
};

template <bool INT4>
struct LabelVec0 {  // generic r: 1 token, scalar loads, qg read from LDS
  static constexpr int VT = 1;
  using Q = QPtr;
  RowPtrs p;  // by value: the caller's RowPtrs may go out of scope before score()
  int t;
  __device__ __forceinline__ void load(const RowPtrs& pp, int v) {
    p = pp;
    t = v;
  }
  __device__ __forceinline__ void score(const Q& q, int r, float* out) const {
    float acc = 0.0f;
    if (INT4) {
      const uint8_t* c = p.codes + (int64_t)t * (r >> 1);
      for (int j = 0; j < r; ++j) {
        const int byte = c[j >> 1];
        const int v = (j & 1) ? (byte >> 4) : (byte & 0xF);
        acc = fmaf(q.qg[j], (float)(v >= 8 ? v - 16 : v), acc);
      }
      out[0] = h2f(p.scales[t]) * acc;
    } else {
      const __half* c = p.lab16 + (int64_t)t * r;
      for (int j = 0; j < r; ++j) acc = fmaf(q.qg[j], h2f(c[j]), acc);
      out[0] = acc;
    }
  }
};

template <int R, bool INT4>
struct VecSel {
  using type = LabelVec<R, INT4>;
};
template <bool INT4>
struct VecSel<0, INT4> {
  using type = LabelVec0<INT4>;
};

struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};

// Scores of tokens [t_beg, t_end) (t_beg a multiple of the vector width) as
// keys: store(t, score, key).  The first batch of label loads is issued
// before `hook` runs (every thread calls it exactly once; it fills ql and
// synchronises the workgroup), so the label latency overlaps the query
// gather.
template <int NT, int R, bool INT4, typename Store, typename Hook>
__device__ __forceinline__ void score_range(const ScoreArgs& a, const RowPtrs& p,
                                            const QueryLds& ql, int t_beg, int t_end,
                                            Store store, Hook hook) {
  using Vec = typename VecSel<R, INT4>::type;
  constexpr int VT = Vec::VT;
  constexpr int UNR = 4;
  const int v_beg = t_beg / VT;
  const int v_end = (t_end + VT - 1) / VT;
  Vec vec[UNR];
  int v0 = v_beg + (int)threadIdx.x;
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const int v = v0 + u * NT;
    if (v < v_end) vec[u].load(p, v);
  }
  hook();
  typename Vec::Q q;
  q.load(ql);
  for (;;) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int v = v0 + u * NT;
      if (v < v_end) {
        float s[VT];
        vec[u].score(q, a.r, s);
#pragma unroll
        for (int e = 0; e < VT; ++e) {
          const int t = v * VT + e;
          if (t < t_end) store(t, s[e], score_key(s[e]));
        }
      }
    }
    v0 += NT * UNR;
    if (v0 >= v_end) break;
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int v = v0 + u * NT;
      if (v < v_end) vec[u].load(p, v);
    }
  }
}

// Workgroup min and max (two barriers); tmp holds 2 * NT / 64 floats.
template <int NT>
__device__ __forceinline__ void block_minmax(float& mn, float& mx, float* tmp) {
  mn = wave_min(mn);
  mx = wave_max(mx);
  const int w = wave_id();
  if ((threadIdx.x & 63) == 0) {
    tmp[w] = mn;
    tmp[NT / 64 + w] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    mn = fminf(mn, tmp[i]);
    mx = fmaxf(mx, tmp[NT / 64 + i]);
  }
  __syncthreads();
}

// Bin (of 2048, descending order) holding the need-th largest key: writes
// sel[0] = bin, sel[1] = keys in higher bins, sel[2] = keys in that bin.
// Two barriers: wave totals of the per-thread bin sums, then the result.
template <int NT>
__device__ __forceinline__ void find_digit(const uint32_t* hist, uint32_t need, uint32_t* sel,
                                           uint32_t* scan_tmp) {
  constexpr int BPT = kHistBins / NT;
  const int hi = kHistBins - 1 - (int)threadIdx.x * BPT;
  const int w = wave_id();
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) local += hist[hi - i];
  const uint32_t incl = wave_incl_scan(local);
  if ((threadIdx.x & 63) == 63) scan_tmp[w] = incl;
  __syncthreads();
  uint32_t excl = incl - local;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) excl += i < w ? scan_tmp[i] : 0u;
  if (excl < need && need <= excl + local) {
    uint32_t acc = excl;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const uint32_t h = hist[hi - i];
      if (acc + h >= need) {
        sel[0] = (uint32_t)(hi - i);
        sel[1] = acc;
        sel[2] = h;
        break;
      }
      acc += h;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Exact selection.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float key_float(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return __uint_as_float(u);
}

// Linear bins between the smallest and largest valid score mn <= mx:
// bin(s) = trunc(clamp((s - mn) * scale + 1.5, 0, 2047.5)), a monotone
// function of s that puts every valid score in bins 1 .. 2047 and -inf (the
// marker of an empty slot) in bin 0; all valid scores share bin 1 when
// mn == mx.  Since k never exceeds the number of valid items, the k-th
// largest never lies in bin 0.
struct LinBins {
  float mn, scale;
  __device__ __forceinline__ LinBins(float lo, float hi) : mn(lo), scale(1.0f) {
    const float span = hi - lo;
    if (span > 0.0f && span <= 3.402823466e38f) scale = fminf(2046.0f / span, 3.402823466e38f);
  }
  __device__ __forceinline__ uint32_t operator()(float s) const {
    return (uint32_t)__builtin_amdgcn_fmed3f(fmaf(s - mn, scale, 1.5f), 0.0f, 2047.5f);
  }
};

struct SelScratch {
  uint32_t hist[kHistBins];
  alignas(16) uint32_t cand_key[kRankMax];
  alignas(16) int32_t cand_idx[kRankMax];
  uint32_t misc[12];
};

// Exact selection of the k largest of n keys (k < n) in LDS, ties to the
// lower index.  mn, mx: smallest and largest score of the row.
// ---------------------------------------------------------------------------
// Plain radix select over keys in memory (rows too long for LDS).
// ---------------------------------------------------------------------------
struct Threshold {
  uint32_t prefix, pmask, need;
};

template <int NT>
__device__ Threshold radix_select_global(const uint32_t* keys, int n, uint32_t k, uint32_t* hist,
                                         uint32_t* scan_tmp, uint32_t* sel) {
  Threshold th{0u, 0u, k};
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
    for (int i = threadIdx.x; i < kHistBins; i += NT) hist[i] = 0u;
    __syncthreads();
    const uint4* k4 = reinterpret_cast<const uint4*>(keys);
    const int nv = (n + 3) >> 2;
    for (int v = threadIdx.x; v < nv; v += NT) {
      const uint4 kv = k4[v];
      const uint32_t w[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * v + e < n && (w[e] & th.pmask) == th.prefix)
          atomicAdd(&hist[(w[e] >> shift) & dmask], 1u);
    }
    __syncthreads();
    find_digit<NT>(hist, th.need, sel, scan_tmp);
    const uint32_t d = sel[0], above = sel[1], cnt = sel[2];
    th.prefix |= d << shift;
    th.pmask |= dmask << shift;
    th.need -= above;
    if (cnt == th.need) break;  // the whole bin is taken
  }
  return th;
}

// Output pass over keys in memory, in rounds of 4*NT tokens.
template <int NT>
__device__ void emit_global(const uint32_t* keys, int n, Threshold th, int32_t* out,
                            uint32_t* scan_tmp) {
  uint32_t run_a = 0, run_e = 0;
  const uint4* k4 = reinterpret_cast<const uint4*>(keys);
  for (int base = 0; base < n; base += 4 * NT) {
    const int t0 = base + 4 * (int)threadIdx.x;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (t0 < n) {
      const uint4 kv = k4[t0 >> 2];
      w[0] = kv.x;
      w[1] = kv.y;
      w[2] = kv.z;
      w[3] = kv.w;
    }
    uint32_t na = 0, ne = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (t0 + e < n) {
        const uint32_t km = w[e] & th.pmask;
        na += km > th.prefix;
        ne += km == th.prefix;
      }
    }
    uint32_t total;
    const uint32_t ex = block_excl_scan<NT>(na | (ne << 16), scan_tmp, &total);
    uint32_t ab = run_a + (ex & 0xFFFFu), eb = run_e + (ex >> 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (t0 + e < n) {
        const uint32_t km = w[e] & th.pmask;
        const bool A = km > th.prefix, E = km == th.prefix;
        if (A || (E && eb < th.need)) out[ab + min(eb, th.need)] = t0 + e;
        ab += A;
        eb += E;
      }
    }
    run_a += total & 0xFFFFu;
    run_e += total >> 16;
  }
}

// ---------------------------------------------------------------------------
// Register-resident scores: the label append and the selection.
// ---------------------------------------------------------------------------
// Label of token t from the K row staged in LDS (one whole wave), written to
// the label cache exactly as the label kernel writes it.  With with_score its
// score goes to f.snew, computed as the label vector of type
// VecSel<R, INT4> scores a stored label (int4 r = 8 or 16: the fixed-point
// query in f.q; otherwise fmaf over j in order, then the int4 scale).
template <int R, bool INT4, typename F>
__device__ __forceinline__ void append_label(const LabelArgs& la, int row, int t, F& f, int r,
                                             bool with_score) {
  const int lane = threadIdx.x & 63;
  const int64_t slot = (int64_t)row * la.slots + t;
  float sf = 1.0f;
  if (!INT4) {
    for (int j = lane; j < r; j += 64) {
      const __half v = f.knew[f.chan[j]];
      la.lab16[slot * r + j] = v;
      f.lnew[j] = h2f(v);
    }
  } else {
    float amax = 0.0f;
    for (int j = lane; j < r; j += 64) amax = fmaxf(amax, fabsf(h2f(f.knew[f.chan[j]])));
    if (R == 8 || R == 16) {
      amax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(row_max16(amax)), 15));
    } else {
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    }
    const __half s16 = __float2half_rn(amax / 7.0f);  // IEEE division, round to nearest even
    sf = h2f(s16);
    for (int j = lane; j < r; j += 64) {
      float v = 0.0f;
      if (sf != 0.0f) v = fminf(fmaxf(rintf(h2f(f.knew[f.chan[j]]) / sf), -7.0f), 7.0f);
      f.lnew[j] = v;
    }
    __builtin_amdgcn_wave_barrier();
    for (int p = lane; p < (r >> 1); p += 64) {
      const int c0 = (int)f.lnew[2 * p], c1 = (int)f.lnew[2 * p + 1];
      la.codes[slot * (r >> 1) + p] = (uint8_t)((c0 & 0xF) | ((c1 & 0xF) << 4));
    }
    if (lane == 0) la.scales[slot] = s16;
  }
  __builtin_amdgcn_wave_barrier();
  if (INT4 && (R == 8 || R == 16)) {
    // the code words of the new token (nibble i of word w = channel 8w + i)
    const int c = lane < r ? (int)f.lnew[lane] : 0;
    const uint32_t wd = row_or8(lane < r ? (uint32_t)(c & 15) << (4 * (lane & 7)) : 0u);
    const uint32_t w[2] = {(uint32_t)__builtin_amdgcn_readlane((int)wd, 7),
                           (uint32_t)__builtin_amdgcn_readlane((int)wd, 15)};
    if (with_score && lane == 0) {
      QDig<(R == 16 ? 2 : 1)> qd;
      qd.load(f.q);
      f.snew = (float)dot_dig(qd, w) * sf;
    }
  } else if (with_score && lane == 0) {
    float acc = 0.0f;
    for (int j = 0; j < r; ++j) acc = fmaf(f.q.qg[j], f.lnew[j], acc);
    f.snew = INT4 ? sf * acc : acc;
  }
}

// Register-resident selection.  Thread tid holds items (j * NT + tid) * VT + e
// for rounds j < JMAX and elements e < VT in sc[j * VT + e]; a slot counts if
// valid(j, e) and its score is not -inf (the empty marker: such slots fall in
// bin 0, below every item, and never match a class), order(j, e) gives its
// position in the row (ties go to the lower position).  The k largest are characterised by two
// keys e_lo <= e_hi and a quota: items with key > e_hi are taken, items with
// key in [e_lo, e_hi] are taken lowest position first, `need` of them.  Items
// of the boundary linear bin span [kmin, kmax] and bins are monotone, so a key
// inside that span lies in the boundary bin.  mn, mx: smallest and largest
// valid score.  Bin 0 (empty slots) stays out of the histogram.
struct RegSel {
  uint32_t e_lo, e_hi, need;
};

struct NoBstarHook {
  __device__ __forceinline__ void operator()(uint32_t, const LinBins&) const {}
};

// on_bstar(bstar, bin) runs on every thread once the boundary bin is known:
// every valid item with bin(score) > bstar is among the k largest.
// Clears the histogram and the scalars of reg_select; a caller that runs
// it before one of its own barriers passes CLEARED = true to reg_select.
template <int NT>
__device__ __forceinline__ void sel_clear(SelScratch& ss) {
  for (int i = threadIdx.x; i < kHistBins; i += NT) ss.hist[i] = 0u;
  if (threadIdx.x < 12) ss.misc[threadIdx.x] = threadIdx.x == 3 ? 0xFFFFFFFFu : 0u;
}

// Radix passes over the key bits of the items in linear bin bstar (clustered
// or equal scores: too many for the rank count).  On entry r = (smallest key
// of the bin, largest key of the bin, items still to take from the bin); on
// return items of the bin with key > e_hi are taken and `need` of those with
// key in [e_lo, e_hi] (lowest position first).
template <int NT, int VT, int JMAX, typename Valid>
__device__ __forceinline__ void radix_in_bin(const float* sc, Valid valid, const LinBins& bin,
                                             uint32_t bstar, RegSel& r, SelScratch& ss,
                                             uint32_t* scan_tmp) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0u, pmask = 0u;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
    __syncthreads();
    for (int i = tid; i < kHistBins; i += NT) ss.hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < JMAX; ++j)
#pragma unroll
      for (int e = 0; e < VT; ++e) {
        if (!valid(j, e)) continue;
        const float sv = sc[j * VT + e];
        const uint32_t key = score_key(sv);
        if ((key & pmask) == prefix && bin(sv) == bstar)
          atomicAdd(&ss.hist[(key >> shift) & dmask], 1u);
      }
    __syncthreads();
    find_digit<NT>(ss.hist, r.need, ss.misc + 4, scan_tmp);
    const uint32_t d = ss.misc[4], ab = ss.misc[5], c2 = ss.misc[6];
    prefix |= d << shift;
    pmask |= dmask << shift;
    r.need -= ab;
    if (c2 == r.need) break;
  }
  __syncthreads();
  r.e_lo = max(r.e_lo, prefix);
  r.e_hi = min(r.e_hi, prefix | ~pmask);
}

template <int NT, int VT, int JMAX, bool CLEARED = false, typename Valid, typename Order,
          typename OnBstar = NoBstarHook>
__device__ __forceinline__ RegSel reg_select(const float* sc, Valid valid, Order order, uint32_t k,
                                             float mn, float mx, SelScratch& ss,
                                             uint32_t* scan_tmp, OnBstar on_bstar = OnBstar()) {
  const int tid = threadIdx.x;
  const LinBins bin(mn, mx);
  if (!CLEARED) {
    sel_clear<NT>(ss);
    __syncthreads();
  }
  // (empty slots are left out of the histogram: they would all hit bin 0)
#pragma unroll
  for (int j = 0; j < JMAX; ++j)
#pragma unroll
    for (int e = 0; e < VT; ++e) {
      const uint32_t bi = bin(sc[j * VT + e]);
      if (valid(j, e) && bi != 0u) atomicAdd(&ss.hist[bi], 1u);
    }
  __syncthreads();
  find_digit<NT>(ss.hist, k, ss.misc + 4, scan_tmp);
  const uint32_t bstar = ss.misc[4];
  const uint32_t cnt = ss.misc[6];
  on_bstar(bstar, bin);
  RegSel r;
  r.need = k - ss.misc[5];
  const bool few = cnt <= (uint32_t)kRankMax;
#pragma unroll
  for (int j = 0; j < JMAX; ++j)
#pragma unroll
    for (int e = 0; e < VT; ++e)
      if (valid(j, e) && bin(sc[j * VT + e]) == bstar) {
        const uint32_t key = score_key(sc[j * VT + e]);
        atomicMin(&ss.misc[3], key);
        atomicMax(&ss.misc[7], key);
        if (few) {
          const uint32_t pos = atomicAdd(&ss.misc[0], 1u);
          ss.cand_key[pos] = key;
          ss.cand_idx[pos] = order(j, e);
        }
      }
  __syncthreads();
  r.e_lo = ss.misc[3];
  r.e_hi = ss.misc[7];
  if (cnt == r.need) return r;  // the whole boundary bin is taken
  if (few) {
    for (int i = tid; i < (int)cnt; i += NT) {
      const uint32_t ki = ss.cand_key[i];
      const int ti = ss.cand_idx[i];
      uint32_t rank = 0;
      for (int m = 0; m < (int)cnt; ++m) {
        const uint32_t km = ss.cand_key[m];
        rank += (km > ki) || (km == ki && ss.cand_idx[m] < ti);
      }
      if (rank == r.need - 1) ss.misc[1] = ki;  // the last key taken
    }
    __syncthreads();
    const uint32_t T = ss.misc[1];
    for (int i = tid; i < (int)cnt; i += NT)
      if (ss.cand_key[i] > T) atomicAdd(&ss.misc[2], 1u);
    __syncthreads();
    r.e_lo = r.e_hi = T;
    r.need -= ss.misc[2];
    return r;
  }
  // Many keys in the boundary bin (clustered or equal scores): radix passes
  // over the key bits inside it.
  radix_in_bin<NT, VT, JMAX>(sc, valid, bin, bstar, r, ss, scan_tmp);
  return r;
}

// Ordered emission of the items taken by `r`: put(pos, j, e) with pos the
// item's rank among the taken items in position order.  tot holds
// JMAX * (NT / 64) words of LDS.  One barrier (two for more than 64 words).
// The classes are decided on the scores: key(s) > e_hi iff s > f_hi and
// key(s) >= e_lo iff s >= f_lo, with f_hi the largest float whose key is at
// most e_hi and f_lo the smallest float whose key is at least e_lo.  Both
// keys lie between the smallest and largest key of the row, so the floats are
// finite; every such key is a float's key except 0x7FFFFFFF, which lies
// between the keys of -denorm_min and of +-0.
template <int NT, int VT, int JMAX, typename Valid, typename Put>
__device__ __forceinline__ void reg_emit(const float* sc, Valid valid, const RegSel& r,
                                         uint32_t* tot, Put put) {
  constexpr int W = NT / 64;
  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const float f_lo = key_float(r.e_lo == 0x7FFFFFFFu ? 0x80000000u : r.e_lo);
  const float f_hi = key_float(r.e_hi == 0x7FFFFFFFu ? 0x7FFFFFFEu : r.e_hi);
  uint32_t ex[JMAX];
#pragma unroll
  for (int j = 0; j < JMAX; ++j) {
    uint32_t packed = 0u;
#pragma unroll
    for (int e = 0; e < VT; ++e) {
      if (!valid(j, e)) continue;
      const float sv = sc[j * VT + e];
      packed += sv > f_hi ? 1u : (sv >= f_lo ? 0x10000u : 0u);
    }
    const uint32_t incl = wave_incl_scan(packed);
    ex[j] = incl - packed;
    if (lane == 63) tot[j * W + w] = incl;
  }
  __syncthreads();
  // Position of each (round, wave) group among all groups in item order:
  // small tables are summed by every thread; large ones are turned into
  // exclusive prefixes in place by wave 0 first (one more barrier).
  constexpr int N = JMAX * W;
  constexpr bool kScan = N > 64;
  if (kScan) {
    constexpr int E = (N + 63) / 64;
    if (w == 0) {
      uint32_t v[E];
      uint32_t sum = 0u;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const int at = lane * E + i;
        v[i] = at < N ? tot[at] : 0u;
        sum += v[i];
      }
      uint32_t run0 = wave_incl_scan(sum) - sum;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const int at = lane * E + i;
        if (at < N) tot[at] = run0;
        run0 += v[i];
      }
    }
    __syncthreads();
  }
  uint32_t run = 0u;
#pragma unroll
  for (int j = 0; j < JMAX; ++j) {
    uint32_t base;
    if (kScan) {
      base = tot[j * W + w] + ex[j];
    } else {
      uint32_t pre = 0u, rowt = 0u;
#pragma unroll
      for (int ww = 0; ww < W; ++ww) {
        const uint32_t t = tot[j * W + ww];
        pre += ww < w ? t : 0u;
        rowt += t;
      }
      base = run + pre + ex[j];
      run += rowt;
    }
    uint32_t ab = base & 0xFFFFu, eb = base >> 16;
#pragma unroll
    for (int e = 0; e < VT; ++e) {
      if (!valid(j, e)) continue;
      const float sv = sc[j * VT + e];
      const bool A = sv > f_hi, E = !A && sv >= f_lo;
      if (A || (E && eb < r.need)) put(ab + min(eb, r.need), j, e);
      ab += A;
      eb += E;
    }
  }
}

// ---------------------------------------------------------------------------
// Register-resident selection into an unordered token list (for attention,
// which does not depend on the order of its tokens).  Same item layout,
// valid/order conventions and result as reg_select; the list holds the
// positions of the k largest.  Two halves, so that the caller can start
// reading the first part of the list while the boundary is resolved.
// ---------------------------------------------------------------------------
struct ListSel {
  uint32_t bstar;  // boundary linear bin
  uint32_t n_a;    // items in higher bins: list[0 .. n_a), all taken
  uint32_t need;   // items still to take from the boundary bin (>= 1)
  uint32_t cnt;    // items in the boundary bin
};

// First half.  The histogram of the linear bins gives the boundary bin b*
// (the scratch was cleared before one of the caller's barriers); every item
// of a higher bin is written to list[0 .. n_a) and, when there are at most
// kRankMax of them, the items of b* to the candidate arrays (key, position),
// both ordered by (wave, lane, round, element) through one exchange of wave
// totals.  Ends with a barrier, after which list[0 .. n_a) is complete.
// JUNK (a list in LDS with 64 spare words at `junk`): every item is written
// without a branch, the ones below b* into the lane's own spare word.
template <int NT, int VT, int JMAX, bool JUNK = false, typename Valid, typename Order>
__device__ __forceinline__ ListSel list_select_a(const float* sc, Valid valid, Order order,
                                                 uint32_t k, const LinBins& bin, SelScratch& ss,
                                                 uint32_t* scan_tmp, int32_t* list,
                                                 int32_t* junk = nullptr) {
  constexpr int N = JMAX * VT;
  static_assert(N <= 32, "one bit per item");
  const int lane = threadIdx.x & 63;
  // the items' bins, two 16-bit halves per word, computed once
  uint32_t bp[(N + 1) / 2];
#pragma unroll
  for (int i = 0; i < (N + 1) / 2; ++i) bp[i] = 0u;
#pragma unroll
  for (int j = 0; j < JMAX; ++j)
#pragma unroll
    for (int e = 0; e < VT; ++e) {
      const int i = j * VT + e;
      const uint32_t bi = bin(sc[i]);
      bp[i >> 1] |= bi << (16 * (i & 1));
      if (valid(j, e) && bi != 0u) atomicAdd(&ss.hist[bi], 1u);
    }
  __syncthreads();
  find_digit<NT>(ss.hist, k, ss.misc + 4, scan_tmp);
  ListSel ls;
  ls.bstar = ss.misc[4];
  ls.n_a = ss.misc[5];
  ls.cnt = ss.misc[6];
  ls.need = k - ls.n_a;
  const bool few = ls.cnt <= (uint32_t)kRankMax;
  // per thread: items above b* and in b* (bit i: item i); positions in
  // (wave, lane, round, element) order, so the list and hence the
  // attention's summation order are the same on every run
  uint32_t above = 0u, equal = 0u;
#pragma unroll
  for (int j = 0; j < JMAX; ++j)
#pragma unroll
    for (int e = 0; e < VT; ++e) {
      const int i = j * VT + e;
      const uint32_t bi = (bp[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      if (valid(j, e)) {
        above |= (bi > ls.bstar ? 1u : 0u) << i;
        equal |= (bi == ls.bstar ? 1u : 0u) << i;
      }
    }
  const uint32_t mine = (uint32_t)__builtin_popcount(above) |
                        ((uint32_t)__builtin_popcount(equal) << 16);
  const int w = wave_id();
  const uint32_t incl = wave_incl_scan(mine);
  if (lane == 63) scan_tmp[w] = incl;  // find_digit's reads of scan_tmp are behind its last barrier
  __syncthreads();
  uint32_t pos = incl - mine;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) pos += i < w ? scan_tmp[i] : 0u;
  uint32_t pa = pos & 0xFFFFu, pb = pos >> 16;
  if (JUNK) {
#pragma unroll
    for (int j = 0; j < JMAX; ++j)
#pragma unroll
      for (int e = 0; e < VT; ++e) {
        const uint32_t a = (above >> (j * VT + e)) & 1u;
        *(a ? list + pa : junk + lane) = order(j, e);
        pa += a;
      }
    if (few && equal) {  // the few items of b*: most threads have none
#pragma unroll
      for (int j = 0; j < JMAX; ++j)
#pragma unroll
        for (int e = 0; e < VT; ++e)
          if ((equal >> (j * VT + e)) & 1u) {
            ss.cand_key[pb] = score_key(sc[j * VT + e]);
            ss.cand_idx[pb] = order(j, e);
            ++pb;
          }
    }
  } else {
#pragma unroll
    for (int j = 0; j < JMAX; ++j)
#pragma unroll
      for (int e = 0; e < VT; ++e) {
        const int i = j * VT + e;
        if ((above >> i) & 1u) {
          list[pa++] = order(j, e);
        } else if ((equal >> i) & 1u) {
          if (few) {
            ss.cand_key[pb] = score_key(sc[i]);
            ss.cand_idx[pb] = order(j, e);
          }
          ++pb;
        }
      }
  }
  __syncthreads();
  return ls;
}

// Second half with at most kRankMax candidates (collected by list_select_a):
// each one's rank (key descending, then position ascending) is counted and
// the first `need` ranks go to list[n_a .. k).  Ends with a barrier; returns
// the whole selection characterised as by reg_select (for reg_emit).
static_assert(kRankMax % 8 == 0, "list_rank reads candidates in groups of eight");
template <int NT>
__device__ __forceinline__ RegSel list_rank(const ListSel& ls, SelScratch& ss, int32_t* list) {
  const int cnt = (int)ls.cnt;
  for (int i = threadIdx.x; i < cnt; i += NT) {
    const uint32_t ki = ss.cand_key[i];
    const int ti = ss.cand_idx[i];
    uint32_t above = 0, tied = 0;
    // eight candidates per step in four 16-byte LDS reads, all in flight
    // together: the reads are unconditional (m + 8 <= kRankMax, as
    // cnt <= kRankMax), and slots past cnt do not count
    for (int m = 0; m < cnt; m += 8) {
      const uint4 k0 = *reinterpret_cast<const uint4*>(&ss.cand_key[m]);
      const uint4 k1 = *reinterpret_cast<const uint4*>(&ss.cand_key[m + 4]);
      const int4 t0 = *reinterpret_cast<const int4*>(&ss.cand_idx[m]);
      const int4 t1 = *reinterpret_cast<const int4*>(&ss.cand_idx[m + 4]);
      const uint32_t km[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
      const int tm[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool in = m + u < cnt;
        above += (in && km[u] > ki) ? 1u : 0u;
        tied += (in && km[u] == ki && tm[u] < ti) ? 1u : 0u;
      }
    }
    const uint32_t rank = above + tied;
    if (rank < ls.need) list[ls.n_a + rank] = ti;
    if (rank == ls.need - 1) {  // the last item taken
      ss.misc[2] = ki;
      ss.misc[8] = above;
    }
  }
  __syncthreads();
  RegSel r;
  r.e_lo = r.e_hi = ss.misc[2];
  r.need = ls.need - ss.misc[8];
  return r;
}

// Second half: the `need` items taken from the boundary bin go to
// list[n_a .. k).  With few candidates each one's rank (key descending, then
// position ascending) is counted and the first `need` ranks are written;
// otherwise radix passes inside the bin and an ordered emission of its taken
// items.  Ends with a barrier (the list is complete) and returns the whole
// selection characterised as by reg_select, for reg_emit.
template <int NT, int VT, int JMAX, typename Valid, typename Order>
__device__ __forceinline__ RegSel list_select_b(const float* sc, Valid valid, Order order,
                                                const LinBins& bin, const ListSel& ls,
                                                SelScratch& ss, uint32_t* scan_tmp, uint32_t* tot,
                                                int32_t* list) {
  const int tid = threadIdx.x;
  RegSel r;
  if (ls.cnt <= (uint32_t)kRankMax) return list_rank<NT>(ls, ss, list);
  // smallest and largest key of the boundary bin
  const uint32_t bstar = ls.bstar;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < JMAX; ++j)
#pragma unroll
    for (int e = 0; e < VT; ++e)
      if (valid(j, e) && bin(sc[j * VT + e]) == bstar) {
        const uint32_t key = score_key(sc[j * VT + e]);
        kmin = min(kmin, key);
        kmax = max(kmax, key);
      }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
  }
  if ((tid & 63) == 0) {
    atomicMin(&ss.misc[3], kmin);
    atomicMax(&ss.misc[7], kmax);
  }
  __syncthreads();
  r.e_lo = ss.misc[3];
  r.e_hi = ss.misc[7];
  r.need = ls.need;
  if (ls.cnt != ls.need) radix_in_bin<NT, VT, JMAX>(sc, valid, bin, bstar, r, ss, scan_tmp);
  reg_emit<NT, VT, JMAX>(
      sc, [&](int j, int e) { return valid(j, e) && bin(sc[j * VT + e]) == bstar; }, r, tot,
      [&](uint32_t pos, int j, int e) { list[ls.n_a + pos] = order(j, e); });
  __syncthreads();
  return r;
}

__device__ __forceinline__ int row_len(const ScoreArgs& a, int b) {
  return min(max(a.seq_lens[b], 0), a.max_seq);
}

// A fully pruned KV head (no K columns) selects no token: its set is empty
// (all -1 when the caller asked for it) and its list length 0.  Returns true
// for such a row; every thread of the workgroup calls it.
template <int NT>
__device__ __forceinline__ bool pruned_row(const ScoreArgs& a, int row, int g) {
  if (!a.heads || a.heads[g].k_cols != 0) return false;
  if (a.pad_idx) {
    int32_t* out = a.idx + (int64_t)row * a.idx_stride;
    for (int t = threadIdx.x; t < a.idx_stride; t += NT) out[t] = -1;
  }
  if (threadIdx.x == 0) a.count[row] = 0;
  return true;
}

}  // namespace ds
