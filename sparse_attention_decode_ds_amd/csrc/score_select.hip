// score_select.hip -- steps 1-2 (query gather, approximate scores) and step
// 3a (top-k token selection) of a Double Sparsity decode step.
//
// [DS] "online forward computation": step 1 takes the query at the heavy
// channels into a contiguous vector, step 2 scores every cached token from
// that vector and the contiguous label cache, step 3 keeps the k tokens with
// the largest scores.  Under GQA ([GQA] section 4) one token set serves the
// whole group of query heads; its score is the sum of the heads' scores,
// i.e. the gathered queries are summed first.
//
// Two variants:
//  * fused (S <= kFuseMaxTokens): one workgroup per (batch, KV head) row;
//    the row's scores become order-preserving uint32 keys in LDS and a radix
//    select runs on them in place;
//  * chunked: many workgroups per row write keys to the workspace, then one
//    1024-thread workgroup per row runs the same radix select streaming the
//    keys from memory (they are still cache resident).
// The select is exact: three radix passes (11, 11, 10 bits) narrow the
// threshold key down; the output pass keeps keys above it plus, among keys
// equal to it, the lowest token indices, and writes the set in ascending
// token order (deterministic, no atomics on the output).
#include "ds_internal.h"

namespace ds {
namespace {

constexpr int kHistBins = 2048;

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
// path (any r, scalar loads); the others use 16-byte label loads.
template <int R, bool INT4>
struct LabelVec;

template <>
struct LabelVec<8, true> {  // 4 tokens: 16 B of codes + 8 B of scales
  static constexpr int VT = 4;
  uint4 c;
  uint2 s;
  __device__ __forceinline__ void load(const RowPtrs& p, int v) {
    c = reinterpret_cast<const uint4*>(p.codes)[v];
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
      for (int j = 0; j < 8; ++j) acc += qg[j] * (float)nib(w[u], j);
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
    c = reinterpret_cast<const uint4*>(p.codes)[v];
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
      for (int j = 0; j < 16; ++j) acc += qg[j] * (float)nib(w[2 * u + (j >> 3)], j & 7);
      out[u] = sc[u] * acc;
    }
  }
};

template <>
struct LabelVec<8, false> {  // 1 token: 8 fp16 labels
  static constexpr int VT = 1;
  uint4 c;
  __device__ __forceinline__ void load(const RowPtrs& p, int v) {
    c = reinterpret_cast<const uint4*>(p.lab16)[v];
  }
  __device__ __forceinline__ void score(const float* qg, int, float* out) const {
    float f[8];
    unpack8(c, f);
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += qg[j] * f[j];
    out[0] = acc;
  }
};

template <>
struct LabelVec<16, false> {  // 1 token: 16 fp16 labels
  static constexpr int VT = 1;
  uint4 c0, c1;
  __device__ __forceinline__ void load(const RowPtrs& p, int v) {
    c0 = reinterpret_cast<const uint4*>(p.lab16)[2 * v];
    c1 = reinterpret_cast<const uint4*>(p.lab16)[2 * v + 1];
  }
  __device__ __forceinline__ void score(const float* qg, int, float* out) const {
    float f[16];
    unpack8(c0, f);
    unpack8(c1, f + 8);
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc += qg[j] * f[j];
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
        acc += qg[j] * (float)(v >= 8 ? v - 16 : v);
      }
      out[0] = h2f(p->scales[t]) * acc;
    } else {
      const __half* c = p->lab16 + (int64_t)t * r;
      for (int j = 0; j < r; ++j) acc += qg[j] * h2f(c[j]);
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

// Scores of tokens [t_beg, t_end) (t_beg a multiple of VT) as keys: store(t, key).
template <int NT, int R, bool INT4, typename Store>
__device__ __forceinline__ void score_range(const ScoreArgs& a, const RowPtrs& p,
                                            const float* qg_lds, int t_beg, int t_end,
                                            Store store) {
  using Vec = typename VecSel<R, INT4>::type;
  constexpr int VT = Vec::VT;
  constexpr int UNR = 4;
  constexpr int QR = R > 0 ? R : 1;
  float qreg[QR];
  const float* qg = qg_lds;
  if (R > 0) {
#pragma unroll
    for (int j = 0; j < QR; ++j) qreg[j] = qg_lds[j];
    qg = qreg;
  }
  const int v_beg = t_beg / VT;
  const int v_end = (t_end + VT - 1) / VT;
  for (int v0 = v_beg + (int)threadIdx.x; v0 < v_end; v0 += NT * UNR) {
    Vec vec[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int v = v0 + u * NT;
      if (v < v_end) vec[u].load(p, v);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int v = v0 + u * NT;
      if (v < v_end) {
        float s[VT];
        vec[u].score(qg, a.r, s);
#pragma unroll
        for (int e = 0; e < VT; ++e) {
          const int t = v * VT + e;
          if (t < t_end) store(t, score_key(s[e]));
        }
      }
    }
  }
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

struct Threshold {
  uint32_t prefix, pmask, need;
};

// Radix select over n keys (LDS array, or a global row read 4 keys at a time).
template <int NT, bool GLOBAL>
__device__ Threshold radix_select(const uint32_t* keys, int n, uint32_t k, uint32_t* hist,
                                  uint32_t* scan_tmp, uint32_t* sel) {
  Threshold th{0u, 0u, k};
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
    for (int i = threadIdx.x; i < kHistBins; i += NT) hist[i] = 0u;
    __syncthreads();
    if (GLOBAL) {
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
    } else {
      for (int t = threadIdx.x; t < n; t += NT) {
        const uint32_t key = keys[t];
        if ((key & th.pmask) == th.prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
      }
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

// Output pass over LDS keys: each thread owns a contiguous segment (odd
// length, so the strided LDS reads spread over the banks).
template <int NT>
__device__ void emit_lds(const uint32_t* keys, int n, Threshold th, int32_t* out,
                         uint32_t* scan_tmp) {
  int seg = (n + NT - 1) / NT;
  seg |= 1;
  const int beg = (int)threadIdx.x * seg;
  const int end = min(n, beg + seg);
  uint32_t na = 0, ne = 0;
  for (int t = beg; t < end; ++t) {
    const uint32_t km = keys[t] & th.pmask;
    na += km > th.prefix;
    ne += km == th.prefix;
  }
  uint32_t total;
  const uint32_t ex = block_excl_scan<NT>(na | (ne << 16), scan_tmp, &total);
  uint32_t ab = ex & 0xFFFFu, eb = ex >> 16;
  for (int t = beg; t < end; ++t) {
    const uint32_t km = keys[t] & th.pmask;
    const bool A = km > th.prefix, E = km == th.prefix;
    if (A || (E && eb < th.need)) out[ab + min(eb, th.need)] = t;
    ab += A;
    eb += E;
  }
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

__device__ __forceinline__ int row_len(const ScoreArgs& a, int b) {
  return min(max(a.seq_lens[b], 0), a.max_seq);
}

// Rows with S <= k (or k <= 0): every token, in order.  Returns true if so.
template <int NT>
__device__ __forceinline__ bool emit_all_if_short(const ScoreArgs& a, int row, int S) {
  if (a.k > 0 && S > a.k) return false;
  int32_t* out = a.idx + (int64_t)row * a.idx_stride;
  for (int t = threadIdx.x; t < S; t += NT) out[t] = t;
  if (a.pad_idx)
    for (int t = S + threadIdx.x; t < a.idx_stride; t += NT) out[t] = -1;
  if (threadIdx.x == 0) a.count[row] = S;
  return true;
}

template <int NT>
__device__ __forceinline__ void finish_row(const ScoreArgs& a, int row) {
  int32_t* out = a.idx + (int64_t)row * a.idx_stride;
  if (a.pad_idx)
    for (int t = a.k + threadIdx.x; t < a.idx_stride; t += NT) out[t] = -1;
  if (threadIdx.x == 0) a.count[row] = a.k;
}

// ---------------------------------------------------------------------------
// Fused: one workgroup per row, keys in LDS (dynamic, max_seq words).
// ---------------------------------------------------------------------------
template <int NT, int R, bool INT4>
__global__ __launch_bounds__(NT) void k_score_select_fused(ScoreArgs a) {
  extern __shared__ uint32_t keys[];
  __shared__ float qg[128];
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t scan_tmp[NT / 64];
  __shared__ uint32_t sel[4];

  const int row = blockIdx.x;
  const int b = row / a.Hkv;
  const int g = row - b * a.Hkv;
  const int S = row_len(a, b);
  if (emit_all_if_short<NT>(a, row, S)) return;

  gather_query(a, b, g, qg);
  __syncthreads();
  const RowPtrs p = row_ptrs(a, row);
  score_range<NT, R, INT4>(a, p, qg, 0, S, [&](int t, uint32_t key) { keys[t] = key; });
  __syncthreads();

  const Threshold th = radix_select<NT, false>(keys, S, (uint32_t)a.k, hist, scan_tmp, sel);
  emit_lds<NT>(keys, S, th, a.idx + (int64_t)row * a.idx_stride, scan_tmp);
  finish_row<NT>(a, row);
}

// ---------------------------------------------------------------------------
// Chunked: scores of `chunk` tokens per workgroup, written as keys.
// ---------------------------------------------------------------------------
template <int NT, int R, bool INT4>
__global__ __launch_bounds__(NT) void k_score_chunk(ScoreArgs a) {
  __shared__ float qg[128];
  const int row = blockIdx.x / a.n_chunks;
  const int c = blockIdx.x - row * a.n_chunks;
  const int b = row / a.Hkv;
  const int g = row - b * a.Hkv;
  const int S = row_len(a, b);
  if (a.k <= 0 || S <= a.k) return;
  const int t_beg = c * a.chunk;
  const int t_end = min(S, t_beg + a.chunk);
  if (t_beg >= t_end) return;
  gather_query(a, b, g, qg);
  __syncthreads();
  const RowPtrs p = row_ptrs(a, row);
  uint32_t* kr = a.keys + (int64_t)row * a.keys_stride;
  score_range<NT, R, INT4>(a, p, qg, t_beg, t_end, [&](int t, uint32_t key) { kr[t] = key; });
}

template <int NT>
__global__ __launch_bounds__(NT) void k_select_stream(ScoreArgs a) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t scan_tmp[NT / 64];
  __shared__ uint32_t sel[4];
  const int row = blockIdx.x;
  const int b = row / a.Hkv;
  const int S = row_len(a, b);
  if (emit_all_if_short<NT>(a, row, S)) return;
  const uint32_t* kr = a.keys + (int64_t)row * a.keys_stride;
  const Threshold th = radix_select<NT, true>(kr, S, (uint32_t)a.k, hist, scan_tmp, sel);
  emit_global<NT>(kr, S, th, a.idx + (int64_t)row * a.idx_stride, scan_tmp);
  finish_row<NT>(a, row);
}

constexpr int kFusedThreads = 256;
constexpr int kChunkThreads = 256;
constexpr int kSelectThreads = 1024;

template <template <int, int, bool> class KT, int NT>
struct Pick {
  static void* get(int r, bool int4) {
    if (int4) {
      if (r == 8) return (void*)KT<NT, 8, true>::fn;
      if (r == 16) return (void*)KT<NT, 16, true>::fn;
      return (void*)KT<NT, 0, true>::fn;
    }
    if (r == 8) return (void*)KT<NT, 8, false>::fn;
    if (r == 16) return (void*)KT<NT, 16, false>::fn;
    return (void*)KT<NT, 0, false>::fn;
  }
};

template <int NT, int R, bool INT4>
struct FusedK {
  static constexpr auto fn = k_score_select_fused<NT, R, INT4>;
};
template <int NT, int R, bool INT4>
struct ChunkK {
  static constexpr auto fn = k_score_chunk<NT, R, INT4>;
};

}  // namespace

hipError_t launch_score_select_fused(const ScoreArgs& a, int rows, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  void* fn = Pick<FusedK, kFusedThreads>::get(a.r, a.is_int4 != 0);
  const size_t lds = (size_t)max(a.max_seq, 1) * sizeof(uint32_t);
  void* args[] = {const_cast<ScoreArgs*>(&a)};
  return hipLaunchKernel(fn, dim3(rows), dim3(kFusedThreads), args, lds, s);
}

hipError_t launch_score_chunks(const ScoreArgs& a, int rows, hipStream_t s) {
  if (rows <= 0 || a.n_chunks <= 0) return hipSuccess;
  void* fn = Pick<ChunkK, kChunkThreads>::get(a.r, a.is_int4 != 0);
  void* args[] = {const_cast<ScoreArgs*>(&a)};
  return hipLaunchKernel(fn, dim3(rows * a.n_chunks), dim3(kChunkThreads), args, 0, s);
}

hipError_t launch_select_stream(const ScoreArgs& a, int rows, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_select_stream<kSelectThreads>, dim3(rows), dim3(kSelectThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ds
