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
//   select   exact top-k on the register-resident scores into an LDS token
//            list (list_select_a/b: linear-bin histogram, the tokens of the
//            bins above the boundary bin listed first, then the boundary bin
//            resolved by rank count or radix passes);
//   attend   exact attention over the list (attn_common.h), fp16 output.
//            The first K/V loads of every slot go out as soon as the first
//            part of the list is written, while the boundary is resolved.
//            When the caller asks for the selected set, it is written in
//            ascending order by an ordered compaction (reg_emit).
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
// page-table entries of the longest row (pages of at least 16 tokens)
constexpr int kFusedPages = kNT * kDecodeFusedTPT / 16;

template <int TPT, bool PAGED>
struct FusedScratch {
  __half qrow[256];
  int32_t chan[128];
  int32_t keep[128];
  __half knew[128];  // K row of the appended token
  float lnew[128];   // its label values (int4: codes)
  QueryLds q;        // the gathered query
  float snew;        // its score
  float mm_tmp[2 * kWaves];
  uint32_t scan_tmp[kWaves];
  SelScratch sel;
  uint32_t tot[TPT * kWaves];  // per round and wave: taken | equal << 16
  int32_t lidx[kDecodeFusedMaxK];
  int32_t junk[64];  // spare words of the list writes
  AttnRed<1> red;
  int32_t ptab[PAGED ? kFusedPages : 1];  // the row's page-table entries (paged pool)
};



// PAGED: K/V in a paged pool; the row's page-table entries are staged in
// LDS with the other small loads, and list tokens become physical ids at
// the K/V loads.
template <int R, bool INT4, int TPT, bool PAGED, bool HEADS>
__global__ __launch_bounds__(kNT, 4) void k_decode_fused(ScoreArgs sa_in, AttnArgs aa_in,
                                                      LabelArgs la_in, int append) {
  using Vec = typename VecSel<R, INT4>::type;
  constexpr int VT = Vec::VT;
  constexpr int JMAX = TPT / VT;  // rounds of vectors per thread
  // label vectors in flight per thread: all of them when they fit in about
  // 40 registers, else 4 at a time
  constexpr int UNR = JMAX * (int)sizeof(Vec) <= 160 ? JMAX : 4;
  __shared__ FusedScratch<TPT, PAGED> f;

  const int row = blockIdx.x;
  const int b = row / sa_in.Hkv;
  const int g = row - b * sa_in.Hkv;
  // HEADS: a per-head layout; the plain instantiation reads none of its
  // fields (each argument read or rewritten here lengthens the chain of
  // scalar loads before the first label load)
  ScoreArgs sa = sa_in;
  if (!HEADS) sa.keep_ld = sa.d_k;
  const AttnArgs aa = HEADS ? with_head(aa_in, g) : aa_in;
  const LabelArgs la = HEADS ? with_head(la_in, g) : la_in;
  const int S = row_len(sa, b);
  const int tid = threadIdx.x;
  if (HEADS && aa.d_k == 0) {  // a fully pruned head: no token, zero output
    if (sa.pad_idx)
      for (int i = tid; i < sa.idx_stride; i += kNT) sa.idx[(int64_t)row * sa.idx_stride + i] = -1;
    if (tid < kDv / 8)
      *reinterpret_cast<uint4*>(aa.out + ((int64_t)b * aa.Hq + g) * kDv + tid * 8) =
          make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  const int lane = tid & 63;
  const int w = wave_id();
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
      for (int i = tid; i < sa.keep_ld; i += kNT) f.keep[i] = sa.keep[(int64_t)g * sa.keep_ld + i];
    if (do_append && tid < (la.d_k >> 3)) {
      const __half* kr = la.K + kv_off(la.ptab, la.pshift, la.max_pages, b, t_new, la.ks0, la.ks2) +
                         (int64_t)g * la.ks1;
      *reinterpret_cast<uint4*>(&f.knew[tid * 8]) = *reinterpret_cast<const uint4*>(kr + tid * 8);
    }
    if (PAGED) {
      const int npg = (sa.max_seq + (1 << aa.pshift) - 1) >> aa.pshift;
      for (int i = tid; i < npg; i += kNT) f.ptab[i] = aa.ptab[(int64_t)b * aa.max_pages + i];
    }
  }

  const RowPtrs p = row_ptrs(sa, row);
  const int n_vec = sparse ? (S + VT - 1) / VT : 0;
  const int v_last = n_vec - 1;  // the only vector that may be partial; it holds t_new
  const int jn = (n_vec + kNT - 1) / kNT;  // rounds holding any vector (uniform)
  // The first label loads go out before the row's length arrives (one
  // dependent load less ahead of the label stream): every slot below the
  // batch bound max_seq (<= slots, a multiple of 16) is fetched.
  const int n_vec_ld =
      sa.k > 0 && sa.max_seq > sa.k ? (min(sa.max_seq, sa.slots) + VT - 1) / VT : 0;
  Vec vec[UNR];
#pragma unroll
  for (int u = 0; u < UNR; ++u) {
    const int v = u * kNT + tid;
    if (v < n_vec_ld) vec[u].load(p, v);
  }
  __syncthreads();
  {
    float qgv = 0.0f;
    if (tid < r) {
      const int col = f.chan[tid];
      qgv = h2f(f.qrow[sa.keep ? f.keep[col] : col]);
    }
    store_query(INT4, r, qgv, f.q);
  }
  __syncthreads();

  // The append runs on the last wave: the first one holds the row's tail
  // vectors (round JMAX - 1 when S is just above a multiple of 256 VT).
  constexpr int kAppendWave = kWaves - 1;
  // Attention: lane c of slot `slot` holds K/V channels [8c, 8c + 8).  List
  // position i is token f.lidx[i] on the sparse path and token i on the
  // dense one; both paths share the attention code below.
  const __half* Kr = aa.K + (PAGED ? 0 : (int64_t)b * aa.ks0) + (int64_t)g * aa.ks1 +
                     min(c, (aa.d_k >> 3) - 1) * 8;
  const __half* Vr = aa.V + (PAGED ? 0 : (int64_t)b * aa.vs0) + (int64_t)g * aa.vs1 + c * 8;
  auto tok = [&](int i) -> int64_t {
    const int t = sparse ? f.lidx[i] : i;
    return PAGED ? (int64_t)phys_tok(f.ptab, aa.pshift, t) : (int64_t)t;
  };
  auto token = [&](int j, int e) { return (j * kNT + tid) * VT + e; };
  auto valid = [&](int j, int) { return j < jn; };  // empty slots hold -inf
  const int n_att = sparse ? sa.k : S;  // tokens attended
  AttnLoads L;
  if (!sparse) {
    if (do_append && w == kAppendWave) append_label<R, INT4>(la, row, t_new, f, r, false);
    if (sa.pad_idx) {
      int32_t* out = sa.idx + (int64_t)row * sa.idx_stride;
      for (int i = tid; i < sa.idx_stride; i += kNT) out[i] = i < S ? i : -1;
    }
    // label loads issued ahead of the row length are not used here; let them
    // land before the attention loads take their place
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    if (n_att > 0) attend_prime<PAGED>(aa, Kr, Vr, slot, n_att, tok, L);
  } else {
    sel_clear<kNT>(f.sel);  // published by the barrier after the scores
    if (do_append && w == kAppendWave) append_label<R, INT4>(la, row, t_new, f, r, true);
    typename Vec::Q q;
    q.load(f.q);
    // --- score into registers ----------------------------------------------
    // Slots without a token (and the appended token until its score is
    // known) hold -inf, which the select treats as empty.
    constexpr float kEmpty = -__builtin_huge_valf();
    float sc[TPT];
    float mn = __builtin_huge_valf(), mx = kEmpty;
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
        for (int e = 0; e < VT; ++e) s[e] = kEmpty;
        if (v < v_last) {  // a full vector of real tokens
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
            const int t = v * VT + e;
            if (t >= S || (do_append && t == t_new)) {
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
    // Row min and max: wave partials, one barrier (which also publishes the
    // appended token's score and the cleared select scratch).
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) {
      f.mm_tmp[w] = mn;
      f.mm_tmp[kWaves + w] = mx;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      mn = fminf(mn, f.mm_tmp[i]);
      mx = fmaxf(mx, f.mm_tmp[kWaves + i]);
    }
    if (do_append) {
      const float sn = f.snew;
      if ((v_last & (kNT - 1)) == tid) {
        const int jl = v_last / kNT;
#pragma unroll
        for (int j = 0; j < JMAX; ++j)
#pragma unroll
          for (int e = 0; e < VT; ++e)
            if (j == jl && e == t_new - v_last * VT) sc[j * VT + e] = sn;
      }
      mn = fminf(mn, sn);
      mx = fmaxf(mx, sn);
    }

    // --- exact select into the LDS token list --------------------------------
    const LinBins bin(mn, mx);
    const ListSel ls = list_select_a<kNT, VT, JMAX, true>(sc, valid, token, (uint32_t)sa.k, bin,
                                                          f.sel, f.scan_tmp, f.lidx, f.junk);
    const int n_a = (int)ls.n_a;
    if (!sa.pad_idx && ls.cnt <= (uint32_t)kRankMax) {
      // Common case: the tokens of the bins above the boundary bin are
      // listed; when they cover the first two groups of every slot, those
      // loads go out while the few boundary candidates are ranked (the
      // scores are no longer needed).
      const bool early = n_a >= 2 * kSlots * kUnroll;
      if (early) attend_prime<PAGED>(aa, Kr, Vr, slot, n_a, tok, L);
      list_rank<kNT>(ls, f.sel, f.lidx);
      if (!early) attend_prime<PAGED>(aa, Kr, Vr, slot, n_att, tok, L);
    } else {
      const RegSel rs = list_select_b<kNT, VT, JMAX>(sc, valid, token, bin, ls, f.sel,
                                                     f.scan_tmp, f.tot, f.lidx);
      if (sa.pad_idx) {  // caller asked for the selected set, ascending
        int32_t* out = sa.idx + (int64_t)row * sa.idx_stride;
        reg_emit<kNT, VT, JMAX>(sc, valid, rs, f.tot,
                                [&](uint32_t pos, int j, int e) { out[pos] = token(j, e); });
        for (int i = sa.k + tid; i < sa.idx_stride; i += kNT) out[i] = -1;
      }
      attend_prime<PAGED>(aa, Kr, Vr, slot, n_att, tok, L);
    }
  }

  // --- attention ---------------------------------------------------------------
  // the query row at the stored K columns' channels, scaled for exp2
  float qf[1][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ch = c * 8 + i;
    qf[0][i] = kl ? h2f(f.qrow[sa.keep ? f.keep[ch] : ch]) * aa.scale_log2 : 0.0f;
  }
  AttnAcc<1> acc;
  acc_init<1>(acc);
  attend_run<1, PAGED>(aa, Kr, Vr, slot, n_att, tok, qf, acc, L);
  attn_finish<1, true>(aa, acc, f.red, b, g, 0);
}

template <int R, bool INT4, int TPT, bool HEADS>
hipError_t launch_rt(const ScoreArgs& sa, const AttnArgs& aa, const LabelArgs& la, int append,
                     int rows, hipStream_t s, const KEvents& ev) {
  if (aa.ptab)
    return launch_k(k_decode_fused<R, INT4, TPT, true, HEADS>, dim3(rows), dim3(kNT), s, ev, sa,
                    aa, la, append);
  return launch_k(k_decode_fused<R, INT4, TPT, false, HEADS>, dim3(rows), dim3(kNT), s, ev, sa, aa,
                  la, append);
}

template <int TPT, bool HEADS>
hipError_t launch_tpt(const ScoreArgs& sa, const AttnArgs& aa, const LabelArgs& la, int append,
                      int rows, hipStream_t s, const KEvents& ev) {
  if (sa.is_int4) {
    if (sa.r == 8) return launch_rt<8, true, TPT, HEADS>(sa, aa, la, append, rows, s, ev);
    if (sa.r == 16) return launch_rt<16, true, TPT, HEADS>(sa, aa, la, append, rows, s, ev);
    return launch_rt<0, true, TPT, HEADS>(sa, aa, la, append, rows, s, ev);
  }
  if (sa.r == 8) return launch_rt<8, false, TPT, HEADS>(sa, aa, la, append, rows, s, ev);
  if (sa.r == 16) return launch_rt<16, false, TPT, HEADS>(sa, aa, la, append, rows, s, ev);
  return launch_rt<0, false, TPT, HEADS>(sa, aa, la, append, rows, s, ev);
}

}  // namespace

bool decode_fused_fits(int max_seq, int k, int r, int is_int4) {
  (void)r;
  (void)is_int4;
  return max_seq <= kNT * kDecodeFusedTPT && (k >= max_seq || k <= kDecodeFusedMaxK);
}

// Scores per thread: the smallest of 8, 20 and 24 that holds the longest row,
// so that no round of register slots is entirely empty for long rows of the
// common lengths.  Per-head layouts take the widest class only (it holds
// every length the fused path accepts), which keeps their instantiations few.
hipError_t launch_decode_fused(const ScoreArgs& sa, const AttnArgs& aa, const LabelArgs& la,
                               int append, int rows, hipStream_t s, const KEvents& ev) {
  if (rows <= 0) return hipSuccess;
  if (aa.heads) return launch_tpt<kDecodeFusedTPT, true>(sa, aa, la, append, rows, s, ev);
  if (sa.max_seq <= kNT * 8) return launch_tpt<8, false>(sa, aa, la, append, rows, s, ev);
  if (sa.max_seq <= kNT * 20) return launch_tpt<20, false>(sa, aa, la, append, rows, s, ev);
  return launch_tpt<kDecodeFusedTPT, false>(sa, aa, la, append, rows, s, ev);
}

}  // namespace ds
