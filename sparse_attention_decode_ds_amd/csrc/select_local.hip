// select_local.hip -- exact top-k for long rows in two kernels ([DS] "online
// forward computation", steps 1-3a), without writing every score to memory.
//
// k_score_local: one workgroup per (row, chunk of CH tokens).  It appends the
//   current token's label when the chunk holds it ([DS] "offline
//   calibration"), scores the chunk into registers and keeps a superset of
//   the chunk's share of the row's top k: with quota M, every token whose
//   score reaches the lower edge T of the linear bin (between the chunk's min
//   and max score) that holds the chunk's M-th largest score.  Any threshold
//   keeps the merge exact (every dropped score is below T, every kept one at
//   or above it); the bin edge makes the kept count about M.  Kept tokens
//   (score, index) go to the row's candidate area in ascending index order,
//   together with theta, the key of T (0 when the chunk is kept whole): every
//   dropped score lies strictly below it.  A chunk whose kept count exceeds
//   its slots reports an overflow.
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
};

// NT threads score a chunk of at most NT * TPT tokens.  Empty slots (past
// the chunk, and the appended token until its score is known) hold -inf.
// HALF: the chunk threshold from the histogram of every other item (large
// quotas only, chosen on the host).
template <int NT, int TPT, int R, bool INT4, bool HALF = false>
__global__ __launch_bounds__(NT) void k_score_local(ScoreArgs sa, LabelArgs la_in, int append) {
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
  if (sa.heads && sa.heads[g].k_cols == 0) return;  // a fully pruned head: no labels
  const LabelArgs la = with_head(la_in, g);
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
      for (int i = tid; i < sa.keep_ld; i += NT) f.keep[i] = sa.keep[(int64_t)g * sa.keep_ld + i];
  }
  for (int j = tid; j < r; j += NT) f.chan[j] = sa.chan[(int64_t)g * r + j];
  if (has_new && tid < (la.d_k >> 3)) {
    const __half* kr = la.K + kv_off(la.ptab, la.pshift, la.max_pages, b, t_new, la.ks0, la.ks2) +
                       (int64_t)g * la.ks1;
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
  // a slot is kept iff its score is at least thr (a whole chunk: every
  // non-empty slot)
  float thr = -3.402823466e38f;
  uint32_t theta = 0u;
  block_minmax<NT>(mn, mx, f.mm_tmp);  // the chunk's range goes to the merge
  if (!keep_all) {
    const LinBins bin(mn, mx);
    SelScratch& ss = f.sel;
    for (int i = tid; i < kHistBins; i += NT) ss.hist[i] = 0u;
    __syncthreads();
    // With HALF (quotas of at least 512), the histogram holds every other
    // item (even item index: every other token, or every other block of NT
    // tokens with one token per vector) and the search is for its
    // ceil(Ms / 2)-th largest, Ms = M less five standard deviations of the
    // sample's count: the chunk's items at or above that bin then number
    // about Ms, below M with the sample's noise and the boundary bin's items
    // on top.  A smaller quota reports an overflow (the merge's full select).
    if (HALF && M < 512) {
      if (tid == 0) sa.cand_cnt[(int64_t)row * sa.n_chunks + c] = -1;
      return;
    }
    const int need = HALF ? (M - (int)(5.0f * __builtin_sqrtf((float)M)) + 1) / 2 : M;
#pragma unroll
    for (int j = 0; j < JMAX; ++j)
      if (j < jn) {
#pragma unroll
        for (int e = 0; e < VT; ++e)
          if (!HALF || ((j * VT + e) & 1) == 0)  // empty slots count in bin 0,
            atomicAdd(&ss.hist[bin(sc[j * VT + e])], 1u);  // which the search never reaches
      }
    __syncthreads();
    // the bin of the need-th largest: every valid key lies in bins 1 .. 2047,
    // and a sample of every other item holds at least half the chunk (n_c > M)
    find_digit<NT>(ss.hist, (uint32_t)need, ss.misc + 4, f.scan_tmp);
    const uint32_t bM = ss.misc[4];
    if (!HALF && ss.misc[5] + ss.misc[6] > (uint32_t)cap) {  // the boundary bin overflows the slots
      if (tid == 0) sa.cand_cnt[(int64_t)row * sa.n_chunks + c] = -1;
      return;
    }
    // T: the lower edge of bin bM in score units (empty slots, -inf, stay
    // below it)
    thr = mn + ((float)bM - 1.5f) / bin.scale;
    theta = score_key(thr);
  }

  // --- ordered emission of the kept tokens ---------------------------------------
  // The chunk's slot arrays are addressed as a workgroup-uniform base plus a
  // 32-bit byte offset per store (no 64-bit address arithmetic per item).
  char* const ck = reinterpret_cast<char*>(sa.cand_score + (int64_t)row * sa.cand_stride +
                                           (int64_t)c * cap);
  char* const ci = reinterpret_cast<char*>(sa.cand_idx + (int64_t)row * sa.cand_stride +
                                           (int64_t)c * cap);
  uint32_t ex[JMAX];
#pragma unroll
  for (int j = 0; j < JMAX; ++j) {
    ex[j] = 0u;
    if (j >= jn) continue;
    uint32_t cnt = 0u;
#pragma unroll
    for (int e = 0; e < VT; ++e) cnt += sc[j * VT + e] >= thr ? 1u : 0u;
    const uint32_t incl = wave_incl_scan(cnt);
    ex[j] = incl - cnt;
    if (lane == 63) f.tot[j][w] = incl;
  }
  __syncthreads();
  // Item order is round j first, then wave, then lane.  With at most 64
  // (round, wave) groups one scan over their totals gives every group's base
  // (lane j * kWavesL + w holds group (j, w)); otherwise each wave sums the
  // totals before it.
  constexpr bool kOneScan = JMAX * kWavesL <= 64;
  uint32_t gbase = 0u, run = 0u;
  if (kOneScan) {
    const int gj = lane / kWavesL;
    const uint32_t t = (lane < JMAX * kWavesL && gj < jn) ? f.tot[gj][lane % kWavesL] : 0u;
    const uint32_t incl = wave_incl_scan(t);
    gbase = incl - t;
    run = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  }
  // Stores stop at the chunk's slots; a kept count beyond them is reported
  // as an overflow below (with one scan the count is known before the
  // stores, which then only run when it fits).
  const uint32_t lim = (uint32_t)cap * 4u;
  const int jlim = (kOneScan && run > (uint32_t)cap) ? 0 : jn;
#pragma unroll
  for (int j = 0; j < JMAX; ++j) {
    if (j >= jlim) continue;
    uint32_t base;
    if (kOneScan) {
      base = (uint32_t)__builtin_amdgcn_readlane((int)gbase, j * kWavesL + w);
    } else {
      uint32_t pre = 0u, rowt = 0u;
#pragma unroll
      for (int ww = 0; ww < kWavesL; ++ww) {
        const uint32_t t = f.tot[j][ww];
        pre += ww < w ? t : 0u;
        rowt += t;
      }
      base = run + pre;
      run += rowt;
    }
    uint32_t off = (base + ex[j]) * 4u;  // < 4 * kMergeCap
#pragma unroll
    for (int e = 0; e < VT; ++e) {
      if (sc[j * VT + e] >= thr && (kOneScan || off < lim)) {
        *reinterpret_cast<float*>(ck + off) = sc[j * VT + e];
        *reinterpret_cast<int32_t*>(ci + off) = token(j, e);
        off += 4u;
      }
    }
  }
  kept = (int)run;  // every thread holds the total
  // the chunk's unused slots hold -inf, which the merge's select treats as
  // empty (so the merge reads no per-chunk counts to mask them)
  if (kept <= cap)
    for (int i = kept + tid; i < cap; i += NT)
      *reinterpret_cast<float*>(ck + (uint32_t)i * 4u) = -__builtin_huge_valf();
  if (tid == 0) {
    // more scores at or above T than the chunk's slots: overflow
    sa.cand_cnt[(int64_t)row * sa.n_chunks + c] = kept > cap ? -1 : kept;
    sa.cand_theta[(int64_t)row * sa.n_chunks + c] = keep_all ? 0u : theta;
    sa.cand_range[(int64_t)row * sa.n_chunks + c] = make_float2(keep_all ? mn : thr, mx);
  }
}

constexpr int kMergeVT = 4;                             // consecutive slots per thread and round
constexpr int kMergeJ = kMergeCap / (kNTM * kMergeVT);  // rounds

// Per-wave summary of the chunk records (wave w: chunks 64w .. 64w + 63).
struct MergeRec {
  uint32_t bad;    // a chunk overflowed its slots
  uint32_t total;  // kept candidates
  uint32_t theta;  // largest threshold key of a chunk that dropped tokens
  float lo, hi;    // range of the kept scores
};

struct MergeScratch {
  SelScratch sel;
  MergeRec rec[kMaxLocalChunks / 64];
  uint32_t scan_tmp[kNTM / 64];
  uint32_t tot[kMergeJ * (kNTM / 64)];
  int32_t junk[64];  // spare words of the LDS list writes
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
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = wave_id();

  // Candidate slots (j * kNTM + tid) * 4 + e of this thread; chunk c owns
  // slots [c * cap, (c + 1) * cap): its kept scores in ascending token order
  // (so slot order is token order), then -inf.  The loads of the row's area
  // and of the chunk records depend on the kernel arguments only, so they go
  // out first, before the row's length and head arrive; slots past the
  // row's chunks (from an earlier call) are masked once they have.
  constexpr int VTM = kMergeVT;
  const float* ck = sa.cand_score + (int64_t)row * sa.cand_stride;
  const int32_t* ci = sa.cand_idx + (int64_t)row * sa.cand_stride;
  float sc[kMergeJ * VTM];
  int32_t tok[kMergeJ * VTM];
#pragma unroll
  for (int j = 0; j < kMergeJ; ++j) {
    const int i = (j * kNTM + tid) * VTM;
    uint4 kk = make_uint4(0u, 0u, 0u, 0u), tt = make_uint4(0u, 0u, 0u, 0u);
    if (i < sa.cand_stride) {
      kk = *reinterpret_cast<const uint4*>(ck + i);
      tt = *reinterpret_cast<const uint4*>(ci + i);
    }
    const uint32_t kv[4] = {kk.x, kk.y, kk.z, kk.w};
    const uint32_t tv[4] = {tt.x, tt.y, tt.z, tt.w};
#pragma unroll
    for (int e = 0; e < VTM; ++e) {
      sc[j * VTM + e] = __uint_as_float(kv[e]);
      tok[j * VTM + e] = (int32_t)tv[e];
    }
  }
  int rc_cnt = 0;
  uint32_t rc_theta = 0u;
  float2 rc_range = make_float2(0.0f, 0.0f);
  if (tid < min(sa.n_chunks, kMaxLocalChunks)) {
    const int64_t at = (int64_t)row * sa.n_chunks + tid;
    rc_cnt = sa.cand_cnt[at];
    rc_theta = sa.cand_theta[at];
    rc_range = sa.cand_range[at];
  }

  const int b = row / sa.Hkv;
  const int g = row - b * sa.Hkv;
  const int S = row_len(sa, b);
  int32_t* out = sa.idx + (int64_t)row * sa.idx_stride;
  if (pruned_row<kNTM>(sa, row, g)) return;

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

  // The chunk records, summarised per wave and then over the waves (one
  // barrier, which also publishes the cleared histogram).
  sel_clear<kNTM>(f.sel);
  if (w < kMaxLocalChunks / 64) {
    const bool in = tid < min(n_ch, kMaxLocalChunks);
    const uint32_t cnt = in ? (uint32_t)max(rc_cnt, 0) : 0u;
    const uint64_t bad = __ballot(in && (rc_cnt < 0 || rc_cnt > cap));
    const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(cnt), 63);
    const uint32_t th = wave_max_u32(in ? rc_theta : 0u);
    const float lo = wave_min(in ? rc_range.x : __builtin_huge_valf());
    const float hi = wave_max(in ? rc_range.y : -__builtin_huge_valf());
    if (lane == 0) f.rec[w] = MergeRec{bad != 0u ? 1u : 0u, tot, th, lo, hi};
  }
  __syncthreads();
  uint32_t bad = n_ch > kMaxLocalChunks ? 1u : 0u, total = 0u, theta_max = 0u;
  float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
#pragma unroll
  for (int i = 0; i < kMaxLocalChunks / 64; ++i) {
    const MergeRec r = f.rec[i];
    bad |= r.bad;
    total += r.total;
    theta_max = max(theta_max, r.theta);
    mn = fminf(mn, r.lo);
    mx = fmaxf(mx, r.hi);
  }
  bool full = bad != 0u || total < (uint32_t)sa.k;

  if (!full) {
    // Slots past the chunks become empty (-inf) too.  [mn, mx] holds every
    // kept score: the chunks report a bound at or below their kept scores
    // (the threshold, or the smallest score of a chunk kept whole) and their
    // largest score.
#pragma unroll
    for (int j = 0; j < kMergeJ; ++j)
#pragma unroll
      for (int e = 0; e < VTM; ++e) {
        const int i = (j * kNTM + tid) * VTM + e;
        if (i >= slots) sc[j * VTM + e] = -__builtin_huge_valf();
      }
    auto valid = [&](int j, int) { return j * kNTM * VTM < slots; };  // empty slots hold -inf
    // slot order is token order, so ties go to the lower token either way
    auto order = [&](int j, int e) { return tok[j * VTM + e]; };
    // The selected tokens go straight to the output list, unordered (the
    // attention pass does not depend on their order), unless the caller
    // asked for the selected set, which is then written in ascending order.
    const LinBins bin(mn, mx);
    const bool in_lds = sa.k <= kMergeLdsList;
    int32_t* list = in_lds ? lds_list : out;
    const ListSel ls =
        in_lds ? list_select_a<kNTM, VTM, kMergeJ, true>(sc, valid, order, (uint32_t)sa.k, bin,
                                                         f.sel, f.scan_tmp, list, f.junk)
               : list_select_a<kNTM, VTM, kMergeJ>(sc, valid, order, (uint32_t)sa.k, bin, f.sel,
                                                   f.scan_tmp, list);
    const RegSel rs =
        ls.cnt <= (uint32_t)kRankMax
            ? list_rank<kNTM>(ls, f.sel, list)
            : list_select_b<kNTM, VTM, kMergeJ>(sc, valid, order, bin, ls, f.sel, f.scan_tmp,
                                                f.tot, list);
    // Complete iff every chunk that dropped tokens (theta != 0) has theta,
    // which lies above each of its dropped keys, at or below the smallest
    // selected key; e_lo is at or below that key (the same on every thread).
    full = theta_max > rs.e_lo;
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
                           hipStream_t s, const KEvents& ev) {
  const dim3 grid(rows * sa.n_chunks);
  if (sa.chunk > 512 * 16 && sa.half_quota)
    return launch_k(k_score_local<512, 20, R, INT4, true>, grid, dim3(512), s, ev, sa, la, append);
  if (sa.chunk > 512 * 16)
    return launch_k(k_score_local<512, 20, R, INT4>, grid, dim3(512), s, ev, sa, la, append);
  if (sa.chunk > 256 * 16)
    return launch_k(k_score_local<512, 16, R, INT4>, grid, dim3(512), s, ev, sa, la, append);
  return launch_k(k_score_local<256, 16, R, INT4>, grid, dim3(256), s, ev, sa, la, append);
}

template <int R, bool INT4>
hipError_t launch_merge_rt(const ScoreArgs& sa, int rows, hipStream_t s, const KEvents& ev) {
  return launch_k(k_select_merge<R, INT4>, dim3(rows), dim3(kNTM), s, ev, sa);
}

}  // namespace

hipError_t launch_score_local(const ScoreArgs& sa, const LabelArgs& la, int append, int rows,
                              hipStream_t s, const KEvents& ev) {
  if (rows <= 0) return hipSuccess;
  if (sa.is_int4) {
    if (sa.r == 8) return launch_local_rt<8, true>(sa, la, append, rows, s, ev);
    if (sa.r == 16) return launch_local_rt<16, true>(sa, la, append, rows, s, ev);
    return launch_local_rt<0, true>(sa, la, append, rows, s, ev);
  }
  if (sa.r == 8) return launch_local_rt<8, false>(sa, la, append, rows, s, ev);
  if (sa.r == 16) return launch_local_rt<16, false>(sa, la, append, rows, s, ev);
  return launch_local_rt<0, false>(sa, la, append, rows, s, ev);
}

hipError_t launch_select_merge(const ScoreArgs& sa, int rows, hipStream_t s, const KEvents& ev) {
  if (rows <= 0) return hipSuccess;
  if (sa.is_int4) {
    if (sa.r == 8) return launch_merge_rt<8, true>(sa, rows, s, ev);
    if (sa.r == 16) return launch_merge_rt<16, true>(sa, rows, s, ev);
    return launch_merge_rt<0, true>(sa, rows, s, ev);
  }
  if (sa.r == 8) return launch_merge_rt<8, false>(sa, rows, s, ev);
  if (sa.r == 16) return launch_merge_rt<16, false>(sa, rows, s, ev);
  return launch_merge_rt<0, false>(sa, rows, s, ev);
}

}  // namespace ds
