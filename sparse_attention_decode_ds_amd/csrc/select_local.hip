// select_local.hip -- exact top-k for long rows in two kernels ([DS] "online
// forward computation", steps 1-3a), without writing every score to memory.
//
// k_score_local: one workgroup per (row, chunk of CH tokens).  It appends the
//   current token's label when the chunk holds it ([DS] "offline
//   calibration"), scores the chunk into registers and keeps a superset of
//   the chunk's share of the row's top k: with quota M, every token whose
//   linear bin (between the chunk's min and max score) is at or above the bin
//   of the chunk's M-th largest score.  Kept tokens (key, index) go to the
//   row's candidate area in ascending index order, together with the
//   smallest kept key theta (0 when the chunk is kept whole).
//
// k_select_merge: one workgroup per row gathers the candidates (chunk order,
//   so ascending token order), selects the k largest exactly (linear bins +
//   exact boundary resolution, score_common.h) and writes them to the token
//   list, in ascending order only when the caller asked for the selected set
//   (the attention pass does not depend on the order).  The
//   result is exact when every chunk that dropped tokens has theta <= the
//   smallest selected key (every dropped key is then strictly smaller).  If a
//   chunk overflowed its slots or that check fails, the workgroup re-scores
//   the whole row into the workspace and runs a plain radix select over it.
#include "score_common.h"

namespace ds {
namespace {

constexpr int kNTM = 1024;

__device__ __forceinline__ int chunks_of(int S, int CH) { return (S + CH - 1) / CH; }
// Quota and candidate slots per chunk.  The quota M is twice the chunk's
// expected share of the top k (at least 64, at most the chunk); a chunk owns
// `cap` slots: M with an eighth and 64 to spare for the boundary bin, within
// the row's slots.  Writer and reader compute the same numbers.
struct Quota {
  int M, cap;
  __device__ __forceinline__ Quota(int S, int k, int CH, int stride, int n_ch) {
    const float expected = (float)k * (float)CH / (float)max(S, 1);
    int m0 = max(64, (int)(2.0f * expected) + 1);
    m0 = min(m0, CH);
    cap = min(stride / max(n_ch, 1), m0 + m0 / 8 + 64);
    M = min(m0, cap - cap / 8);
  }
};

template <int NT, int TPT>
struct LocalScratch {
  __half qrows[kMaxGroup][256];
  int32_t chan[128];
  int32_t keep[128];
  __half knew[128];
  float lnew[128];
  QueryLds q;
  float snew;
  float mm_tmp[2 * (NT / 64)];
  uint32_t scan_tmp[NT / 64];
  SelScratch sel;
  uint32_t tot[TPT][NT / 64];
  uint32_t theta;
};

// NT threads score a chunk of at most NT * TPT tokens.  Empty slots (past
// the chunk, and the appended token until its score is known) hold -inf.
template <int NT, int TPT, int R, bool INT4>
__global__ __launch_bounds__(NT) void k_score_local(ScoreArgs sa, LabelArgs la, int append) {
  constexpr int kWavesL = NT / 64;
  using Vec = typename VecSel<R, INT4>::type;
  constexpr int VT = Vec::VT;
  constexpr int JMAX = TPT / VT;
  // label vectors in flight per thread: all of them when they fit in about
  // 40 registers (one round trip for the whole chunk), else 4 at a time
  constexpr int UNR = JMAX * (int)sizeof(Vec) <= 160 ? JMAX : 4;
  constexpr float kEmpty = -__builtin_huge_valf();
  __shared__ LocalScratch<NT, TPT> f;

  const int row = blockIdx.x / sa.n_chunks;
  const int c = blockIdx.x - row * sa.n_chunks;
  const int b = row / sa.Hkv;
  const int g = row - b * sa.Hkv;
  const int S = row_len(sa, b);
  const int CH = sa.chunk;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_id();
  const int r = sa.r;
  const int t_beg = c * CH;
  const int t_end = min(S, t_beg + CH);
  if (t_beg >= t_end) return;
  const int t_new = S - 1;
  const bool has_new = append && t_new >= t_beg && t_new < t_end;
  const bool sparse = S > sa.k;

  // --- setup: small loads first --------------------------------------------
  if (sparse) {
    const __half* qh = sa.q + ((int64_t)b * sa.Hq + (int64_t)g * sa.G) * sa.d_q;
    for (int i = tid; i < sa.G * sa.d_q; i += NT) f.qrows[i / sa.d_q][i % sa.d_q] = qh[i];
    if (sa.keep)
      for (int i = tid; i < sa.d_k; i += NT) f.keep[i] = sa.keep[(int64_t)g * sa.d_k + i];
  }
  for (int j = tid; j < r; j += NT) f.chan[j] = sa.chan[(int64_t)g * r + j];
  if (has_new && tid < (la.d_k >> 3)) {
    const __half* kr = la.K + (int64_t)b * la.ks0 + (int64_t)g * la.ks1 + (int64_t)t_new * la.ks2;
    *reinterpret_cast<uint4*>(&f.knew[tid * 8]) = *reinterpret_cast<const uint4*>(kr + tid * 8);
  }
  if (!sparse) {  // the row attends every token; only the label append is due
    __syncthreads();
    if (has_new && tid < 64) append_label<R, INT4>(la, row, t_new, f, r, false);
    return;
  }

  const RowPtrs p = row_ptrs(sa, row);
  const int n_vec = (t_end - t_beg + VT - 1) / VT;
  const int v_last = n_vec - 1;  // the only vector that may be partial or hold t_new
  const int v0 = t_beg / VT;
  const int jn = (n_vec + NT - 1) / NT;  // rounds holding any vector (uniform)
  // The label loads go out after the small setup loads have landed: issued
  // together, the setup loads wait behind every workgroup's label stream.
  Vec vec[UNR];
  __syncthreads();
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const int v = u * NT + tid;
    if (v < n_vec) vec[u].load(p, v0 + v);
  }
  {
    float acc = 0.0f;
    if (tid < r) {
      const int col = f.chan[tid];
      const int qc = sa.keep ? f.keep[col] : col;
      for (int h = 0; h < sa.G; ++h) acc += h2f(f.qrows[h][qc]);
    }
    store_query(INT4, r, acc, f.q);
  }
  __syncthreads();
  if (has_new && tid < 64) append_label<R, INT4>(la, row, t_new, f, r, true);
  typename Vec::Q q;
  q.load(f.q);

  // --- score into registers --------------------------------------------------
  auto token = [&](int j, int e) { return t_beg + (j * NT + tid) * VT + e; };
  float sc[TPT];
  float mn = __builtin_huge_valf(), mx = kEmpty;
#pragma unroll
  for (int j0 = 0; j0 < JMAX; j0 += UNR) {
    if (j0 > 0) {
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int v = (j0 + u) * NT + tid;
        if (j0 + u < JMAX && v < n_vec) vec[u].load(p, v0 + v);
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int j = j0 + u;
      if (j >= JMAX) continue;
      const int v = j * NT + tid;
      float s[VT];
#pragma unroll
      for (int e = 0; e < VT; ++e) s[e] = kEmpty;
      if (v < v_last) {
        vec[u].score(q, r, s);
#pragma unroll
        for (int e = 0; e < VT; ++e) {
          mn = fminf(mn, s[e]);
          mx = fmaxf(mx, s[e]);
        }
      } else if (v == v_last) {
        vec[u].score(q, r, s);
#pragma unroll
        for (int e = 0; e < VT; ++e) {
          const int t = token(j, e);
          if (t >= t_end || (has_new && t == t_new)) {
            s[e] = kEmpty;
          } else {
            mn = fminf(mn, s[e]);
            mx = fmaxf(mx, s[e]);
          }
        }
      }
#pragma unroll
      for (int e = 0; e < VT; ++e) sc[j * VT + e] = s[e];
    }
  }
  if (has_new) {
    __syncthreads();
    const float sn = f.snew;
    if ((v_last & (NT - 1)) == tid) {
      const int jl = v_last / NT;
#pragma unroll
      for (int j = 0; j < JMAX; ++j)
#pragma unroll
        for (int e = 0; e < VT; ++e)
          if (j == jl && token(j, e) == t_new) sc[j * VT + e] = sn;
    }
    mn = fminf(mn, sn);
    mx = fmaxf(mx, sn);
  }

  // --- local threshold ---------------------------------------------------------
  const int n_ch = chunks_of(S, CH);
  const Quota qu(S, sa.k, CH, sa.cand_stride, n_ch);
  const int cap = qu.cap;
  const int M = qu.M;
  const int n_c = t_end - t_beg;
  const bool keep_all = n_c <= M;
  int kept = n_c;
  // bit (j * VT + e) of keptm: slot kept
  uint32_t keptm = 0u;
  uint32_t tmin = 0xFFFFFFFFu;
  if (!keep_all) {
    block_minmax<NT>(mn, mx, f.mm_tmp);
    const LinBins bin(mn, mx);
    SelScratch& ss = f.sel;
    for (int i = tid; i < kHistBins; i += NT) ss.hist[i] = 0u;
    if (tid == 0) f.theta = 0xFFFFFFFFu;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < JMAX; ++j)
      if (j < jn) {
#pragma unroll
        for (int e = 0; e < VT; ++e) {
          const uint32_t bi = bin(sc[j * VT + e]);
          if (bi != 0u) atomicAdd(&ss.hist[bi], 1u);  // bin 0: empty slots
        }
      }
    __syncthreads();
    // the bin of the M-th largest: every valid key lies in bins 1 .. 2047
    find_digit<NT>(ss.hist, (uint32_t)M, ss.misc + 4, f.scan_tmp);
    const uint32_t bM = ss.misc[4];
    kept = (int)(ss.misc[5] + ss.misc[6]);
    if (kept > cap) {  // the boundary bin is too full for this chunk's slots
      if (tid == 0) sa.cand_cnt[(int64_t)row * sa.n_chunks + c] = -1;
      return;
    }
#pragma unroll
    for (int j = 0; j < JMAX; ++j)
      if (j < jn) {
#pragma unroll
        for (int e = 0; e < VT; ++e) {
          const uint32_t bj = bin(sc[j * VT + e]);
          if (bj >= bM) {
            keptm |= 1u << (j * VT + e);
            if (bj == bM) tmin = min(tmin, score_key(sc[j * VT + e]));
          }
        }
      }
  } else {
#pragma unroll
    for (int j = 0; j < JMAX; ++j)
#pragma unroll
      for (int e = 0; e < VT; ++e)
        if (j < jn && sc[j * VT + e] != kEmpty) keptm |= 1u << (j * VT + e);
  }

  // --- ordered emission of the kept tokens ---------------------------------------
  uint32_t* ck = sa.cand_key + (int64_t)row * sa.cand_stride + (int64_t)c * cap;
  int32_t* ci = sa.cand_idx + (int64_t)row * sa.cand_stride + (int64_t)c * cap;
  uint32_t ex[JMAX];
#pragma unroll
  for (int j = 0; j < JMAX; ++j) {
    ex[j] = 0u;
    if (j >= jn) continue;
    const uint32_t cnt = __builtin_popcount((keptm >> (j * VT)) & ((1u << VT) - 1u));
    const uint32_t incl = wave_incl_scan(cnt);
    ex[j] = incl - cnt;
    if (lane == 63) f.tot[j][w] = incl;
  }
  if (!keep_all) {
    tmin = wave_min_u32(tmin);
    if (lane == 0) atomicMin(&f.theta, tmin);
  }
  __syncthreads();
  uint32_t run = 0u;
#pragma unroll
  for (int j = 0; j < JMAX; ++j) {
    if (j >= jn) continue;
    uint32_t pre = 0u, rowt = 0u;
#pragma unroll
    for (int ww = 0; ww < kWavesL; ++ww) {
      const uint32_t t = f.tot[j][ww];
      pre += ww < w ? t : 0u;
      rowt += t;
    }
    uint32_t pos = run + pre + ex[j];
#pragma unroll
    for (int e = 0; e < VT; ++e) {
      if (keptm & (1u << (j * VT + e))) {
        ck[pos] = score_key(sc[j * VT + e]);
        ci[pos] = token(j, e);
        ++pos;
      }
    }
    run += rowt;
  }
  if (tid == 0) {
    sa.cand_cnt[(int64_t)row * sa.n_chunks + c] = kept;
    sa.cand_theta[(int64_t)row * sa.n_chunks + c] = keep_all ? 0u : f.theta;
  }
}

constexpr int kMergeVT = 4;                             // consecutive slots per thread and round
constexpr int kMergeJ = kMergeCap / (kNTM * kMergeVT);  // rounds

struct MergeScratch {
  SelScratch sel;
  int32_t ch_cnt[kMaxLocalChunks];
  uint32_t ch_theta[kMaxLocalChunks];
  uint32_t scan_tmp[kNTM / 64];
  float mm_tmp[2 * kNTM / 64];
  uint32_t tot[kMergeJ * (kNTM / 64)];
  uint32_t flag;  // 1: fall back to the full select
  uint32_t total; // candidates of the row
};

// Token lists up to this long are built in LDS and copied out in one
// coalesced pass (placing them straight into global memory scatters 4-byte
// stores over the list).
constexpr int kMergeLdsList = 8192;

template <int R, bool INT4>
__global__ __launch_bounds__(kNTM) void k_select_merge(ScoreArgs sa) {
  __shared__ MergeScratch f;
  __shared__ int32_t lds_list[kMergeLdsList];
  const int row = blockIdx.x;
  const int b = row / sa.Hkv;
  const int g = row - b * sa.Hkv;
  const int S = row_len(sa, b);
  const int tid = threadIdx.x;
  int32_t* out = sa.idx + (int64_t)row * sa.idx_stride;

  if (S <= sa.k) {  // every token
    for (int t = tid; t < S; t += kNTM) out[t] = t;
    if (sa.pad_idx)
      for (int t = S + tid; t < sa.idx_stride; t += kNTM) out[t] = -1;
    if (tid == 0) sa.count[row] = S;
    return;
  }
  const int n_ch = chunks_of(S, sa.chunk);
  const int cap = Quota(S, sa.k, sa.chunk, sa.cand_stride, n_ch).cap;
  const int slots = n_ch * cap;  // <= cand_stride <= kMergeCap

  // Candidate slots (j * kNTM + tid) * 4 + e of this thread; chunk c owns
  // slots [c * cap, c * cap + cnt_c), in ascending token order, so slot order
  // is token order.  Every load is issued before the counts are known (a
  // group of four that starts below `slots` lies inside the row's area).
  constexpr int VTM = kMergeVT;
  const uint32_t* ck = sa.cand_key + (int64_t)row * sa.cand_stride;
  const int32_t* ci = sa.cand_idx + (int64_t)row * sa.cand_stride;
  float sc[kMergeJ * VTM];
  int32_t tok[kMergeJ * VTM];
#pragma unroll
  for (int j = 0; j < kMergeJ; ++j) {
    const int i = (j * kNTM + tid) * VTM;
    uint4 kk = make_uint4(0u, 0u, 0u, 0u), tt = make_uint4(0u, 0u, 0u, 0u);
    if (i < slots) {
      kk = *reinterpret_cast<const uint4*>(ck + i);
      tt = *reinterpret_cast<const uint4*>(ci + i);
    }
    const uint32_t kv[4] = {kk.x, kk.y, kk.z, kk.w};
    const uint32_t tv[4] = {tt.x, tt.y, tt.z, tt.w};
#pragma unroll
    for (int e = 0; e < VTM; ++e) {
      sc[j * VTM + e] = key_float(kv[e]);
      tok[j * VTM + e] = (int32_t)tv[e];
    }
  }
  if (tid == 0) {
    f.flag = n_ch > kMaxLocalChunks ? 1u : 0u;
    f.total = 0u;
  }
  __syncthreads();
  if (tid < min(n_ch, kMaxLocalChunks)) {
    const int cnt = sa.cand_cnt[(int64_t)row * sa.n_chunks + tid];
    f.ch_cnt[tid] = cnt;
    f.ch_theta[tid] = sa.cand_theta[(int64_t)row * sa.n_chunks + tid];
    if (cnt < 0 || cnt > cap) atomicOr(&f.flag, 1u);
    atomicAdd(&f.total, (uint32_t)max(cnt, 0));
  }
  __syncthreads();
  bool full = f.flag != 0u || f.total < (uint32_t)sa.k;

  if (!full) {
    // Slots past their chunk's count become empty (-inf); the chunk of slot
    // i is floor(i / cap).
    float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
    const float inv_cap = 1.0f / (float)cap;
#pragma unroll
    for (int j = 0; j < kMergeJ; ++j)
#pragma unroll
      for (int e = 0; e < VTM; ++e) {
        const int i = (j * kNTM + tid) * VTM + e;
        bool ok = false;
        if (i < slots) {
          int c = (int)((float)i * inv_cap);
          c += (i >= (c + 1) * cap) ? 1 : 0;
          c -= (i < c * cap) ? 1 : 0;
          ok = i - c * cap < f.ch_cnt[c];
        }
        if (ok) {
          mn = fminf(mn, sc[j * VTM + e]);
          mx = fmaxf(mx, sc[j * VTM + e]);
        } else {
          sc[j * VTM + e] = -__builtin_huge_valf();
        }
      }
    sel_clear<kNTM>(f.sel);  // published by block_minmax's barriers
    block_minmax<kNTM>(mn, mx, f.mm_tmp);
    auto valid = [&](int j, int) { return j * kNTM * VTM < slots; };  // empty slots hold -inf
    // slot order is token order, so ties go to the lower token either way
    auto order = [&](int j, int e) { return tok[j * VTM + e]; };
    // The selected tokens go straight to the output list, unordered (the
    // attention pass does not depend on their order), unless the caller
    // asked for the selected set, which is then written in ascending order.
    const LinBins bin(mn, mx);
    const bool in_lds = sa.k <= kMergeLdsList;
    int32_t* list = in_lds ? lds_list : out;
    const ListSel ls = list_select_a<kNTM, VTM, kMergeJ>(sc, valid, order, (uint32_t)sa.k, bin,
                                                         f.sel, f.scan_tmp, list);
    const RegSel rs =
        ls.cnt <= (uint32_t)kRankMax
            ? list_rank<kNTM>(ls, f.sel, list)
            : list_select_b<kNTM, VTM, kMergeJ>(sc, valid, order, bin, ls, f.sel, f.scan_tmp,
                                                f.tot, list);
    // Complete iff every chunk that dropped tokens (theta != 0) has theta at
    // or below the smallest selected key; e_lo is at or below that key.
    if (tid < min(n_ch, kMaxLocalChunks) && f.ch_theta[tid] > rs.e_lo) atomicOr(&f.flag, 1u);
    __syncthreads();
    full = f.flag != 0u;
    if (!full && sa.pad_idx) {
      reg_emit<kNTM, VTM, kMergeJ>(sc, valid, rs, f.tot, [&](uint32_t pos, int j, int e) {
        out[pos] = tok[j * VTM + e];
      });
    } else if (!full && in_lds) {
      for (int i = tid; i < sa.k; i += kNTM) out[i] = lds_list[i];
    }
  }

  if (full) {
    // Re-score the whole row into the workspace, then a radix select over it.
    __shared__ QueryLds qg;
    const RowPtrs p = row_ptrs(sa, row);
    uint32_t* kr = sa.keys + (int64_t)row * sa.keys_stride;
    score_range<kNTM, R, INT4>(
        sa, p, qg, 0, S, [&](int t, float, uint32_t key) { kr[t] = key; },
        [&]() {
          gather_query(sa, b, g, qg);
          __syncthreads();
        });
    __threadfence_block();
    __syncthreads();
    const Threshold th =
        radix_select_global<kNTM>(kr, S, (uint32_t)sa.k, f.sel.hist, f.scan_tmp, f.sel.misc);
    emit_global<kNTM>(kr, S, th, out, f.scan_tmp);
  }
  if (sa.pad_idx)
    for (int t = sa.k + tid; t < sa.idx_stride; t += kNTM) out[t] = -1;
  if (tid == 0) sa.count[row] = sa.k;
}

template <int R, bool INT4>
hipError_t launch_local_rt(const ScoreArgs& sa, const LabelArgs& la, int append, int rows,
                           hipStream_t s) {
  const dim3 grid(rows * sa.n_chunks);
  if (sa.chunk > 512 * 16)
    hipLaunchKernelGGL((k_score_local<512, 20, R, INT4>), grid, dim3(512), 0, s, sa, la, append);
  else if (sa.chunk > 256 * 16)
    hipLaunchKernelGGL((k_score_local<512, 16, R, INT4>), grid, dim3(512), 0, s, sa, la, append);
  else
    hipLaunchKernelGGL((k_score_local<256, 16, R, INT4>), grid, dim3(256), 0, s, sa, la, append);
  return hipGetLastError();
}

template <int R, bool INT4>
hipError_t launch_merge_rt(const ScoreArgs& sa, int rows, hipStream_t s) {
  hipLaunchKernelGGL((k_select_merge<R, INT4>), dim3(rows), dim3(kNTM), 0, s, sa);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score_local(const ScoreArgs& sa, const LabelArgs& la, int append, int rows,
                              hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (sa.is_int4) {
    if (sa.r == 8) return launch_local_rt<8, true>(sa, la, append, rows, s);
    if (sa.r == 16) return launch_local_rt<16, true>(sa, la, append, rows, s);
    return launch_local_rt<0, true>(sa, la, append, rows, s);
  }
  if (sa.r == 8) return launch_local_rt<8, false>(sa, la, append, rows, s);
  if (sa.r == 16) return launch_local_rt<16, false>(sa, la, append, rows, s);
  return launch_local_rt<0, false>(sa, la, append, rows, s);
}

hipError_t launch_select_merge(const ScoreArgs& sa, int rows, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (sa.is_int4) {
    if (sa.r == 8) return launch_merge_rt<8, true>(sa, rows, s);
    if (sa.r == 16) return launch_merge_rt<16, true>(sa, rows, s);
    return launch_merge_rt<0, true>(sa, rows, s);
  }
  if (sa.r == 8) return launch_merge_rt<8, false>(sa, rows, s);
  if (sa.r == 16) return launch_merge_rt<16, false>(sa, rows, s);
  return launch_merge_rt<0, false>(sa, rows, s);
}

}  // namespace ds
