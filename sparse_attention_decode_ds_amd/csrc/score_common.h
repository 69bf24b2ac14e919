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

// Step 1: qg[j] = sum over the group's query heads of q[h][keep[chan[j]]].
__device__ __forceinline__ void gather_query(const ScoreArgs& a, int b, int g, float* qg) {
  for (int j = threadIdx.x; j < a.r; j += blockDim.x) {
    const int col = a.chan[(int64_t)g * a.r + j];
    const int qc = a.keep ? a.keep[(int64_t)g * a.d_k + col] : col;
    const __half* qh = a.q + ((int64_t)b * a.Hq + (int64_t)g * a.G) * a.d_q + qc;
    float acc = 0.0f;
    for (int h = 0; h < a.G; ++h) acc += h2f(qh[(int64_t)h * a.d_q]);
    qg[j] = acc;
  }
}

__device__ __forceinline__ int nib(uint32_t w, int j) {
  return (int)(w << (28 - 4 * j)) >> 28;  // signed nibble j
}

// Step 2 for one vector of VT consecutive tokens.  R = 0 is the generic
// path (any r, scalar loads); the others use 16-byte label loads.  Every
// variant accumulates fmaf(qg[j], label[j], acc) over j in order (then
// times the int4 scale), so a token's score does not depend on the path.
template <int R, bool INT4>
struct LabelVec;

template <>
struct LabelVec<8, true> {  // 4 tokens: 16 B of codes + 8 B of scales
  static constexpr int VT = 4;
  uint4 c;
  uint2 s;
  __device__ __forceinline__ void load(const RowPtrs& p, int v) {
    c = ld_stream(reinterpret_cast<const uint4*>(p.codes) + v);
    s = reinterpret_cast<const uint2*>(p.scales)[v];
  }
  __device__ __forceinline__ void score(const float* qg, int, float* out) const {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    const __half2 s01 = *reinterpret_cast<const __half2*>(&s.x);
    const __half2 s23 = *reinterpret_cast<const __half2*>(&s.y);
    const float sc[4] = {__low2float(s01), __high2float(s01), __low2float(s23), __high2float(s23)};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc = fmaf(qg[j], (float)nib(w[u], j), acc);
      out[u] = sc[u] * acc;
    }
  }
};

template <>
struct LabelVec<16, true> {  // 2 tokens: 16 B of codes + 4 B of scales
  static constexpr int VT = 2;
  uint4 c;
  uint32_t s;
  __device__ __forceinline__ void load(const RowPtrs& p, int v) {
    c = ld_stream(reinterpret_cast<const uint4*>(p.codes) + v);
    s = reinterpret_cast<const uint32_t*>(p.scales)[v];
  }
  __device__ __forceinline__ void score(const float* qg, int, float* out) const {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    const __half2 s01 = *reinterpret_cast<const __half2*>(&s);
    const float sc[2] = {__low2float(s01), __high2float(s01)};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) acc = fmaf(qg[j], (float)nib(w[2 * u + (j >> 3)], j & 7), acc);
      out[u] = sc[u] * acc;
    }
  }
};

template <>
struct LabelVec<8, false> {  // 1 token: 8 fp16 labels
  static constexpr int VT = 1;
  uint4 c;
  __device__ __forceinline__ void load(const RowPtrs& p, int v) {
    c = ld_stream(reinterpret_cast<const uint4*>(p.lab16) + v);
  }
  __device__ __forceinline__ void score(const float* qg, int, float* out) const {
    float f[8];
    unpack8(c, f);
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = fmaf(qg[j], f[j], acc);
    out[0] = acc;
  }
};

template <>
struct LabelVec<16, false> {  // 1 token: 16 fp16 labels
  static constexpr int VT = 1;
  uint4 c0, c1;
  __device__ __forceinline__ void load(const RowPtrs& p, int v) {
    c0 = ld_stream(reinterpret_cast<const uint4*>(p.lab16) + 2 * v);
    c1 = ld_stream(reinterpret_cast<const uint4*>(p.lab16) + 2 * v + 1);
  }
  __device__ __forceinline__ void score(const float* qg, int, float* out) const {
    float f[16];
    unpack8(c0, f);
    unpack8(c1, f + 8);
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc = fmaf(qg[j], f[j], acc);
    out[0] = acc;
  }
};

template <bool INT4>
struct LabelVec0 {  // generic r: 1 token, scalar loads, qg read from LDS
  static constexpr int VT = 1;
  const RowPtrs* p;
  int t;
  __device__ __forceinline__ void load(const RowPtrs& pp, int v) {
    p = &pp;
    t = v;
  }
  __device__ __forceinline__ void score(const float* qg, int r, float* out) const {
    float acc = 0.0f;
    if (INT4) {
      const uint8_t* c = p->codes + (int64_t)t * (r >> 1);
      for (int j = 0; j < r; ++j) {
        const int byte = c[j >> 1];
        const int v = (j & 1) ? (byte >> 4) : (byte & 0xF);
        acc = fmaf(qg[j], (float)(v >= 8 ? v - 16 : v), acc);
      }
      out[0] = h2f(p->scales[t]) * acc;
    } else {
      const __half* c = p->lab16 + (int64_t)t * r;
      for (int j = 0; j < r; ++j) acc = fmaf(qg[j], h2f(c[j]), acc);
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
// before `hook` runs (every thread calls it exactly once; it fills qg_lds and
// may synchronise the workgroup), so the label latency overlaps the query
// gather.
template <int NT, int R, bool INT4, typename Store, typename Hook>
__device__ __forceinline__ void score_range(const ScoreArgs& a, const RowPtrs& p,
                                            const float* qg_lds, int t_beg, int t_end,
                                            Store store, Hook hook) {
  using Vec = typename VecSel<R, INT4>::type;
  constexpr int VT = Vec::VT;
  constexpr int UNR = 4;
  constexpr int QR = R > 0 ? R : 1;
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
  float qreg[QR];
  const float* qg = qg_lds;
  if (R > 0) {
#pragma unroll
    for (int j = 0; j < QR; ++j) qreg[j] = qg_lds[j];
    qg = qreg;
  }
  for (;;) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int v = v0 + u * NT;
      if (v < v_end) {
        float s[VT];
        vec[u].score(qg, a.r, s);
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
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o, 64));
    mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  }
  const int w = threadIdx.x >> 6;
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
template <int NT>
__device__ __forceinline__ void find_digit(const uint32_t* hist, uint32_t need, uint32_t* sel,
                                           uint32_t* scan_tmp) {
  constexpr int BPT = kHistBins / NT;
  const int hi = kHistBins - 1 - (int)threadIdx.x * BPT;
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) local += hist[hi - i];
  uint32_t total;
  const uint32_t excl = block_excl_scan<NT>(local, scan_tmp, &total);
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
// Linear-bin select over keys held in LDS.
// ---------------------------------------------------------------------------
struct Sel {
  float mn, scale;         // bin = clamp((score - mn) * scale, 0, 2047)
  uint32_t bstar;          // bin of the k-th largest key
  uint32_t prefix, pmask;  // refinement inside that bin
  uint32_t need;           // keys of the "equal" class to take, lowest index first
};

__device__ __forceinline__ float key_float(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint32_t lin_bin(uint32_t key, float mn, float scale) {
  float x = (key_float(key) - mn) * scale;
  x = fminf(fmaxf(x, 0.0f), 2047.0f);  // NaN (0 * inf) maps to 0
  return (uint32_t)x;
}

// 2: taken, 1: equal class, 0: not taken.
__device__ __forceinline__ int sel_class(uint32_t key, const Sel& s) {
  const uint32_t bin = lin_bin(key, s.mn, s.scale);
  if (bin != s.bstar) return bin > s.bstar ? 2 : 0;
  const uint32_t km = key & s.pmask;
  return km > s.prefix ? 2 : (km == s.prefix ? 1 : 0);
}

struct SelScratch {
  uint32_t hist[kHistBins];
  uint32_t cand_key[kRankMax];
  int32_t cand_idx[kRankMax];
  uint32_t misc[8];
};

// Exact selection of the k largest of n keys (k < n) in LDS, ties to the
// lower index.  mn, mx: smallest and largest score of the row.
template <int NT>
__device__ Sel select_lds(const uint32_t* keys, int n, uint32_t k, float mn, float mx,
                          SelScratch& sc, uint32_t* scan_tmp) {
  Sel s;
  s.mn = mn;
  s.scale = 2048.0f / (mx - mn);  // +inf when all scores are equal: every key in bin 0
  for (int i = threadIdx.x; i < kHistBins; i += NT) sc.hist[i] = 0u;
  if (threadIdx.x < 8) sc.misc[threadIdx.x] = 0u;
  __syncthreads();
  for (int t = threadIdx.x; t < n; t += NT) atomicAdd(&sc.hist[lin_bin(keys[t], s.mn, s.scale)], 1u);
  __syncthreads();
  find_digit<NT>(sc.hist, k, sc.misc + 4, scan_tmp);
  s.bstar = sc.misc[4];
  const uint32_t above = sc.misc[5], cnt = sc.misc[6];
  s.prefix = 0u;
  s.pmask = 0u;
  s.need = k - above;
  if (cnt == s.need) return s;  // the whole bin is taken

  if (cnt <= (uint32_t)kRankMax) {
    // gather the bin's keys, rank them exactly
    for (int t = threadIdx.x; t < n; t += NT) {
      const uint32_t key = keys[t];
      if (lin_bin(key, s.mn, s.scale) == s.bstar) {
        const uint32_t p = atomicAdd(&sc.misc[0], 1u);
        sc.cand_key[p] = key;
        sc.cand_idx[p] = t;
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < (int)cnt; i += NT) {
      const uint32_t ki = sc.cand_key[i];
      const int ti = sc.cand_idx[i];
      uint32_t rank = 0;
      for (int j = 0; j < (int)cnt; ++j) {
        const uint32_t kj = sc.cand_key[j];
        rank += (kj > ki) || (kj == ki && sc.cand_idx[j] < ti);
      }
      if (rank == s.need - 1) sc.misc[1] = ki;  // the last key taken
    }
    __syncthreads();
    const uint32_t T = sc.misc[1];
    for (int i = threadIdx.x; i < (int)cnt; i += NT)
      if (sc.cand_key[i] > T) atomicAdd(&sc.misc[2], 1u);
    __syncthreads();
    s.prefix = T;
    s.pmask = 0xFFFFFFFFu;
    s.need -= sc.misc[2];
    __syncthreads();
    return s;
  }

  // Many keys in one bin (clustered or equal scores): radix passes over the
  // key bits of that bin.
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
    for (int i = threadIdx.x; i < kHistBins; i += NT) sc.hist[i] = 0u;
    __syncthreads();
    for (int t = threadIdx.x; t < n; t += NT) {
      const uint32_t key = keys[t];
      if ((key & s.pmask) == s.prefix && lin_bin(key, s.mn, s.scale) == s.bstar)
        atomicAdd(&sc.hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    find_digit<NT>(sc.hist, s.need, sc.misc + 4, scan_tmp);
    const uint32_t d = sc.misc[4], ab = sc.misc[5], c2 = sc.misc[6];
    s.prefix |= d << shift;
    s.pmask |= dmask << shift;
    s.need -= ab;
    if (c2 == s.need) break;
  }
  __syncthreads();
  return s;
}

// Ordered output over LDS keys: each thread owns a contiguous segment (odd
// length, so the strided LDS reads spread over the banks).  n < 65536.
template <int NT, typename Out>
__device__ void emit_sel_lds(const uint32_t* keys, int n, const Sel& s, Out out,
                             uint32_t* scan_tmp) {
  int seg = (n + NT - 1) / NT;
  seg |= 1;
  const int beg = (int)threadIdx.x * seg;
  const int end = min(n, beg + seg);
  uint32_t na = 0, ne = 0;
  for (int t = beg; t < end; ++t) {
    const int c = sel_class(keys[t], s);
    na += c == 2;
    ne += c == 1;
  }
  uint32_t total;
  const uint32_t ex = block_excl_scan<NT>(na | (ne << 16), scan_tmp, &total);
  uint32_t ab = ex & 0xFFFFu, eb = ex >> 16;
  for (int t = beg; t < end; ++t) {
    const int c = sel_class(keys[t], s);
    if (c == 2 || (c == 1 && eb < s.need)) out(ab + min(eb, s.need), t);
    ab += c == 2;
    eb += c == 1;
  }
}

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
// Helpers for register-resident scores (one score per slot, tokens ordered
// round-major across the workgroup).
// ---------------------------------------------------------------------------
// Inclusive prefix sum over the 64 lanes of a wave (DPP: shifts within rows
// of 16, then row broadcasts).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false); // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false); // row_bcast:31
  return x;
}

__device__ __forceinline__ uint32_t bin_of(float s, float mn, float scale) {
  float x = (s - mn) * scale;
  x = fminf(fmaxf(x, 0.0f), 2047.0f);  // NaN (0 * inf) maps to 0
  return (uint32_t)x;
}

// Label of token t from the K row staged in LDS (wave 0), written to the
// label cache exactly as the label kernel writes it; its score (same
// operation order as the label-vector scores) goes to f.snew.
template <bool INT4, typename F>
__device__ __forceinline__ void append_label(const LabelArgs& la, int row, int t, F& f, int r,
                                             bool with_score) {
  const int lane = threadIdx.x & 63;  // one wave
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
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
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
  if (with_score && lane == 0) {
    float acc = 0.0f;
    for (int j = 0; j < r; ++j) acc = fmaf(f.qg[j], f.lnew[j], acc);
    f.snew = INT4 ? sf * acc : acc;
  }
}

// Register-resident selection.  Thread tid holds items (j * NT + tid) * VT + e
// for rounds j < JMAX and elements e < VT in sc[j * VT + e]; valid(j, e) says
// whether that slot holds an item, order(j, e) gives its position in the row
// (ties go to the lower position).  The k largest are characterised by two
// keys e_lo <= e_hi and a quota: items with key > e_hi are taken, items with
// key in [e_lo, e_hi] are taken lowest position first, `need` of them.  Items
// of the boundary linear bin span [kmin, kmax] and bins are monotone, so a key
// inside that span lies in the boundary bin.
struct RegSel {
  uint32_t e_lo, e_hi, need;
};

template <int NT, int VT, int JMAX, typename Valid, typename Order>
__device__ RegSel reg_select(const float* sc, Valid valid, Order order, uint32_t k, float mn,
                             float mx, SelScratch& ss, uint32_t* scan_tmp) {
  const int tid = threadIdx.x;
  const float bscale = 2048.0f / (mx - mn);  // +inf when all scores are equal: every key in bin 0
  for (int i = tid; i < kHistBins; i += NT) ss.hist[i] = 0u;
  if (tid < 8) ss.misc[tid] = tid == 3 ? 0xFFFFFFFFu : 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < JMAX; ++j)
#pragma unroll
    for (int e = 0; e < VT; ++e)
      if (valid(j, e)) atomicAdd(&ss.hist[bin_of(sc[j * VT + e], mn, bscale)], 1u);
  __syncthreads();
  find_digit<NT>(ss.hist, k, ss.misc + 4, scan_tmp);
  const uint32_t bstar = ss.misc[4];
  const uint32_t cnt = ss.misc[6];
  RegSel r;
  r.need = k - ss.misc[5];
  const bool few = cnt <= (uint32_t)kRankMax;
#pragma unroll
  for (int j = 0; j < JMAX; ++j)
#pragma unroll
    for (int e = 0; e < VT; ++e)
      if (valid(j, e) && bin_of(sc[j * VT + e], mn, bscale) == bstar) {
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
        if ((key & pmask) == prefix && bin_of(sv, mn, bscale) == bstar)
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
  return r;
}

// Ordered emission of the items taken by `r`: put(pos, j, e) with pos the
// item's rank among the taken items in position order.  tot holds
// JMAX * (NT / 64) words of LDS.  One barrier.
template <int NT, int VT, int JMAX, typename Valid, typename Put>
__device__ __forceinline__ void reg_emit(const float* sc, Valid valid, const RegSel& r,
                                         uint32_t* tot, Put put) {
  constexpr int W = NT / 64;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  auto cls = [&](float sv) {
    const uint32_t key = score_key(sv);
    return key > r.e_hi ? 2 : (key >= r.e_lo ? 1 : 0);
  };
  uint32_t ex[JMAX];
#pragma unroll
  for (int j = 0; j < JMAX; ++j) {
    uint32_t packed = 0u;
#pragma unroll
    for (int e = 0; e < VT; ++e) {
      if (!valid(j, e)) continue;
      const int cl = cls(sc[j * VT + e]);
      packed += cl == 2 ? 1u : (cl == 1 ? 0x10000u : 0u);
    }
    const uint32_t incl = wave_incl_scan(packed);
    ex[j] = incl - packed;
    if (lane == 63) tot[j * W + w] = incl;
  }
  __syncthreads();
  uint32_t run = 0u;
#pragma unroll
  for (int j = 0; j < JMAX; ++j) {
    uint32_t pre = 0u, rowt = 0u;
#pragma unroll
    for (int ww = 0; ww < W; ++ww) {
      const uint32_t t = tot[j * W + ww];
      pre += ww < w ? t : 0u;
      rowt += t;
    }
    const uint32_t base = run + pre + ex[j];
    uint32_t ab = base & 0xFFFFu, eb = base >> 16;
#pragma unroll
    for (int e = 0; e < VT; ++e) {
      if (!valid(j, e)) continue;
      const int cl = cls(sc[j * VT + e]);
      if (cl == 2 || (cl == 1 && eb < r.need)) put(ab + min(eb, r.need), j, e);
      ab += cl == 2;
      eb += cl == 1;
    }
    run += rowt;
  }
}

__device__ __forceinline__ int row_len(const ScoreArgs& a, int b) {
  return min(max(a.seq_lens[b], 0), a.max_seq);
}

}  // namespace ds
