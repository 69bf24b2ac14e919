// decode_fused.hip -- one workgroup per (batch, KV head) row runs the whole
// Double Sparsity decode step for that row ([DS] "offline calibration": label
// append; "online forward computation": steps 1-3):
//
//   setup    the row's query, heavy-channel table, kept-column table and the
//            current token's K row are fetched first (small loads ahead of the
//            label stream); the gathered query goes to LDS;
//   append   the current token's heavy-channel K values become its label (the
//            same bytes ds_label_append writes) and its score is taken from
//            them directly;
//   score    the label stream is scored into registers: thread tid holds the
//            vectors v = j * 256 + tid, so token order is (round j, wave,
//            lane, element);
//   select   exact top-k on the register-resident scores: linear-bin
//            histogram, then exact resolution of the boundary bin (rank count
//            or radix passes), see score_common.h;
//   emit     ordered compaction into an ascending token list in LDS (wave
//            scans per round plus one exchange of wave totals);
//   attend   exact attention over the list (attn_common.h), fp16 output.
//
// Used when the row fits the register budget (S <= 256 * TPT tokens, TPT
// scores per thread), k is small enough for the LDS list and the query group
// is a single head.
#include "attn_common.h"
#include "score_common.h"

namespace ds {
namespace {

constexpr int kNT = 256;
constexpr int kWaves = kNT / 64;

template <int TPT>
struct FusedScratch {
  __half qrow[256];
  int32_t chan[128];
  int32_t keep[128];
  __half knew[128];  // K row of the appended token
  float lnew[128];   // its label values (int4: codes)
  float qg[128];
  float snew;        // its score
  float mm_tmp[2 * kWaves];
  uint32_t scan_tmp[kWaves];
  SelScratch sel;
  uint32_t tot[TPT][kWaves];  // per round and wave: taken | equal << 16
  int32_t lidx[kDecodeFusedMaxK];
  AttnRed<1> red;
};

template <int R, bool INT4, int TPT>
__global__ __launch_bounds__(kNT, 4) void k_decode_fused(ScoreArgs sa, AttnArgs aa, LabelArgs la,
                                                      int append) {
  using Vec = typename VecSel<R, INT4>::type;
  constexpr int VT = Vec::VT;
  constexpr int JMAX = TPT / VT;  // rounds of vectors per thread
  constexpr int UNR = 4;
  constexpr int QR = R > 0 ? R : 1;
  __shared__ FusedScratch<TPT> f;

  const int row = blockIdx.x;
  const int b = row / sa.Hkv;
  const int g = row - b * sa.Hkv;
  const int S = row_len(sa, b);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int c = lane & 15;
  const int slot = w * 4 + (lane >> 4);
  const bool kl = c < (aa.d_k >> 3);
  const int r = sa.r;
  const int t_new = S - 1;
  const bool do_append = append && S >= 1;
  const bool sparse = sa.k > 0 && S > sa.k;

  // --- setup: small loads first --------------------------------------------
  {
    const __half* qh = sa.q + ((int64_t)b * sa.Hq + (int64_t)g) * sa.d_q;
    for (int i = tid; i < sa.d_q; i += kNT) f.qrow[i] = qh[i];
    for (int j = tid; j < r; j += kNT) f.chan[j] = sa.chan[(int64_t)g * r + j];
    if (sa.keep)
      for (int i = tid; i < sa.d_k; i += kNT) f.keep[i] = sa.keep[(int64_t)g * sa.d_k + i];
    if (do_append && tid < (la.d_k >> 3)) {
      const __half* kr = la.K + (int64_t)b * la.ks0 + (int64_t)g * la.ks1 + (int64_t)t_new * la.ks2;
      *reinterpret_cast<uint4*>(&f.knew[tid * 8]) = *reinterpret_cast<const uint4*>(kr + tid * 8);
    }
  }

  const RowPtrs p = row_ptrs(sa, row);
  const int n_vec = sparse ? (S + VT - 1) / VT : 0;
  const int J = (n_vec + kNT - 1) / kNT;
  Vec vec[UNR];
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const int v = u * kNT + tid;
    if (v < n_vec) vec[u].load(p, v);
  }
  __syncthreads();
  if (tid < r) {
    const int col = f.chan[tid];
    f.qg[tid] = h2f(f.qrow[sa.keep ? f.keep[col] : col]);
  }
  __syncthreads();

  if (!sparse) {
    if (do_append && tid < 64) append_label<INT4>(la, row, t_new, f, r, false);
  } else {
    if (do_append && tid < 64) append_label<INT4>(la, row, t_new, f, r, true);
    float qreg[QR];
    const float* qg = f.qg;
    if (R > 0) {
#pragma unroll
      for (int j = 0; j < QR; ++j) qreg[j] = f.qg[j];
      qg = qreg;
    }
    // --- score into registers ----------------------------------------------
    float sc[TPT];
    float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
#pragma unroll
    for (int j0 = 0; j0 < JMAX; j0 += UNR) {
      if (j0 > 0) {
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int v = (j0 + u) * kNT + tid;
          if (j0 + u < JMAX && v < n_vec) vec[u].load(p, v);
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int j = j0 + u;
        if (j >= JMAX) continue;
        const int v = j * kNT + tid;
        float s[VT];
#pragma unroll
        for (int e = 0; e < VT; ++e) s[e] = 0.0f;
        if (v < n_vec) vec[u].score(qg, r, s);
#pragma unroll
        for (int e = 0; e < VT; ++e) {
          const int t = v * VT + e;
          sc[j * VT + e] = s[e];
          if (v < n_vec && t < S && t != (do_append ? t_new : -1)) {
            mn = fminf(mn, s[e]);
            mx = fmaxf(mx, s[e]);
          }
        }
      }
    }
    if (do_append) {
      __syncthreads();
      const float sn = f.snew;
      const int vn = t_new / VT;
      if ((vn & (kNT - 1)) == tid) {
        const int jn = vn / kNT;
#pragma unroll
        for (int j = 0; j < JMAX; ++j)
#pragma unroll
          for (int e = 0; e < VT; ++e)
            if (j == jn && e == t_new - vn * VT) sc[j * VT + e] = sn;
      }
      mn = fminf(mn, sn);
      mx = fmaxf(mx, sn);
    }
    block_minmax<kNT>(mn, mx, f.mm_tmp);

    auto valid = [&](int j, int e) { return (j * kNT + tid) * VT + e < S; };
    auto token = [&](int j, int e) { return (j * kNT + tid) * VT + e; };

    // --- select ------------------------------------------------------------
    // Histogram of linear bins, then the boundary bin b* (holding the k-th
    // largest score) is resolved exactly.  The outcome is two keys E_lo <=
    // E_hi and a quota: keys above E_hi are taken, keys in [E_lo, E_hi] are
    // taken lowest index first up to the quota.  Keys in b* span [kmin, kmax]
    // and bins are monotone, so a key inside that span lies in b*.
    SelScratch& ss = f.sel;
    const float bmn = mn;
    const float bscale = 2048.0f / (mx - mn);  // +inf when all scores are equal: every key in bin 0
    for (int i = tid; i < kHistBins; i += kNT) ss.hist[i] = 0u;
    if (tid < 8) ss.misc[tid] = tid == 3 ? 0xFFFFFFFFu : 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < JMAX; ++j)
#pragma unroll
      for (int e = 0; e < VT; ++e)
        if (j < J && valid(j, e)) atomicAdd(&ss.hist[bin_of(sc[j * VT + e], bmn, bscale)], 1u);
    __syncthreads();
    find_digit<kNT>(ss.hist, (uint32_t)sa.k, ss.misc + 4, f.scan_tmp);
    const uint32_t bstar = ss.misc[4];
    const uint32_t cnt = ss.misc[6];
    uint32_t need = (uint32_t)sa.k - ss.misc[5];
    const bool few = cnt <= (uint32_t)kRankMax;
#pragma unroll
    for (int j = 0; j < JMAX; ++j)
#pragma unroll
      for (int e = 0; e < VT; ++e)
        if (j < J && valid(j, e) && bin_of(sc[j * VT + e], bmn, bscale) == bstar) {
          const uint32_t key = score_key(sc[j * VT + e]);
          atomicMin(&ss.misc[3], key);
          atomicMax(&ss.misc[7], key);
          if (few) {
            const uint32_t pos = atomicAdd(&ss.misc[0], 1u);
            ss.cand_key[pos] = key;
            ss.cand_idx[pos] = token(j, e);
          }
        }
    __syncthreads();
    uint32_t e_lo = ss.misc[3], e_hi = ss.misc[7];
    if (cnt != need) {
      if (few) {
        for (int i = tid; i < (int)cnt; i += kNT) {
          const uint32_t ki = ss.cand_key[i];
          const int ti = ss.cand_idx[i];
          uint32_t rank = 0;
          for (int m = 0; m < (int)cnt; ++m) {
            const uint32_t km = ss.cand_key[m];
            rank += (km > ki) || (km == ki && ss.cand_idx[m] < ti);
          }
          if (rank == need - 1) ss.misc[1] = ki;  // the last key taken
        }
        __syncthreads();
        const uint32_t T = ss.misc[1];
        for (int i = tid; i < (int)cnt; i += kNT)
          if (ss.cand_key[i] > T) atomicAdd(&ss.misc[2], 1u);
        __syncthreads();
        e_lo = e_hi = T;
        need -= ss.misc[2];
      } else {
        // many keys in b* (clustered or equal scores): radix passes over the
        // key bits inside b*
        uint32_t prefix = 0u, pmask = 0u;
#pragma unroll 1
        for (int pass = 0; pass < 3; ++pass) {
          const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
          const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
          __syncthreads();
          for (int i = tid; i < kHistBins; i += kNT) ss.hist[i] = 0u;
          __syncthreads();
#pragma unroll
          for (int j = 0; j < JMAX; ++j)
#pragma unroll
            for (int e = 0; e < VT; ++e) {
              if (j >= J || !valid(j, e)) continue;
              const float sv = sc[j * VT + e];
              const uint32_t key = score_key(sv);
              if ((key & pmask) == prefix && bin_of(sv, bmn, bscale) == bstar)
                atomicAdd(&ss.hist[(key >> shift) & dmask], 1u);
            }
          __syncthreads();
          find_digit<kNT>(ss.hist, need, ss.misc + 4, f.scan_tmp);
          const uint32_t d = ss.misc[4], ab = ss.misc[5], c2 = ss.misc[6];
          prefix |= d << shift;
          pmask |= dmask << shift;
          need -= ab;
          if (c2 == need) break;
        }
        e_lo = max(e_lo, prefix);
        e_hi = min(e_hi, prefix | ~pmask);
      }
    }

    // --- ordered emission ----------------------------------------------------
    auto cls = [&](float sv) {
      const uint32_t key = score_key(sv);
      return key > e_hi ? 2 : (key >= e_lo ? 1 : 0);
    };
    uint32_t ex[JMAX];
#pragma unroll
    for (int j = 0; j < JMAX; ++j) {
      ex[j] = 0u;
      if (j >= J) continue;
      uint32_t packed = 0u;
#pragma unroll
      for (int e = 0; e < VT; ++e) {
        if (!valid(j, e)) continue;
        const int cl = cls(sc[j * VT + e]);
        packed += cl == 2 ? 1u : (cl == 1 ? 0x10000u : 0u);
      }
      const uint32_t incl = wave_incl_scan(packed);
      ex[j] = incl - packed;
      if (lane == 63) f.tot[j][w] = incl;
    }
    __syncthreads();
    uint32_t run = 0u;
#pragma unroll
    for (int j = 0; j < JMAX; ++j) {
      if (j >= J) continue;
      uint32_t pre = 0u, rowt = 0u;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const uint32_t t = f.tot[j][ww];
        pre += ww < w ? t : 0u;
        rowt += t;
      }
      const uint32_t base = run + pre + ex[j];
      uint32_t ab = base & 0xFFFFu, eb = base >> 16;
#pragma unroll
      for (int e = 0; e < VT; ++e) {
        if (!valid(j, e)) continue;
        const int cl = cls(sc[j * VT + e]);
        if (cl == 2 || (cl == 1 && eb < need)) f.lidx[ab + min(eb, need)] = token(j, e);
        ab += cl == 2;
        eb += cl == 1;
      }
      run += rowt;
    }
    __syncthreads();
  }
  const int n_sel = sparse ? sa.k : S;

  if (sa.pad_idx) {  // caller asked for the selected set
    int32_t* out = sa.idx + (int64_t)row * sa.idx_stride;
    for (int i = tid; i < sa.idx_stride; i += kNT)
      out[i] = i < n_sel ? (sparse ? f.lidx[i] : i) : -1;
  }

  // --- attention ---------------------------------------------------------------
  float qf[1][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ch = c * 8 + i;
    qf[0][i] = kl ? h2f(f.qrow[sa.keep ? f.keep[ch] : ch]) * aa.scale_log2 : 0.0f;
  }
  AttnAcc<1> acc;
  acc_init<1>(acc);
  const __half* Kr = aa.K + (int64_t)b * aa.ks0 + (int64_t)g * aa.ks1 + c * 8;
  const __half* Vr = aa.V + (int64_t)b * aa.vs0 + (int64_t)g * aa.vs1 + c * 8;
  if (sparse)
    attend<1>(aa, Kr, Vr, kl, slot, n_sel, [&](int i) { return (int64_t)f.lidx[i]; }, qf, acc);
  else
    attend<1>(aa, Kr, Vr, kl, slot, n_sel, [&](int i) { return (int64_t)i; }, qf, acc);
  attn_finish<1, true>(aa, acc, f.red, b, g, 0);
}

template <int R, bool INT4, int TPT>
hipError_t launch_rt(const ScoreArgs& sa, const AttnArgs& aa, const LabelArgs& la, int append,
                     int rows, hipStream_t s) {
  hipLaunchKernelGGL((k_decode_fused<R, INT4, TPT>), dim3(rows), dim3(kNT), 0, s, sa, aa, la,
                     append);
  return hipGetLastError();
}

template <int TPT>
hipError_t launch_tpt(const ScoreArgs& sa, const AttnArgs& aa, const LabelArgs& la, int append,
                      int rows, hipStream_t s) {
  if (sa.is_int4) {
    if (sa.r == 8) return launch_rt<8, true, TPT>(sa, aa, la, append, rows, s);
    if (sa.r == 16) return launch_rt<16, true, TPT>(sa, aa, la, append, rows, s);
    return launch_rt<0, true, TPT>(sa, aa, la, append, rows, s);
  }
  if (sa.r == 8) return launch_rt<8, false, TPT>(sa, aa, la, append, rows, s);
  if (sa.r == 16) return launch_rt<16, false, TPT>(sa, aa, la, append, rows, s);
  return launch_rt<0, false, TPT>(sa, aa, la, append, rows, s);
}

}  // namespace

bool decode_fused_fits(int max_seq, int k, int r, int is_int4) {
  (void)r;
  (void)is_int4;
  return max_seq <= kNT * kDecodeFusedTPT && (k >= max_seq || k <= kDecodeFusedMaxK);
}

hipError_t launch_decode_fused(const ScoreArgs& sa, const AttnArgs& aa, const LabelArgs& la,
                               int append, int rows, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  return launch_tpt<kDecodeFusedTPT>(sa, aa, la, append, rows, s);
}

}  // namespace ds
