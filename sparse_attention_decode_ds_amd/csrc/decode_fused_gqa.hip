// decode_fused_gqa.hip -- one workgroup of 1024 threads per (batch, KV head)
// row runs the whole Double Sparsity decode step for a query group of
// G = 2..8 heads ([DS] "offline calibration": label append; "online forward
// computation": steps 1-3; [GQA] section 4: the group's heads share the K/V
// rows, and the label score uses the query summed over the group):
//
//   setup    the group's query rows, the heavy-channel table, the kept-column
//            table and the appended token's K row are fetched ahead of the
//            label stream; the summed, gathered query and the query rows at
//            the stored K columns' channels go to LDS;
//   append   the appended token's label is written and scored from the K row;
//   score    the label stream is scored into registers (thread tid holds the
//            vectors v = j * 1024 + tid);
//   select   exact top-k into an LDS token list (list_select_a, then rank
//            count or radix passes for the boundary bin);
//   attend   each of the 16 waves takes every 16th 16-token tile of the list
//            on the matrix cores (gqa_tile.h; with k <= 256 one tile per
//            wave, so all K/V loads of the row are in flight at once); the 16
//            wave states are merged per head through LDS and the fp16 output
//            written.
//
// The rows of a decode batch with few KV heads are long (thousands of
// tokens), so the workgroup is as wide as a compute unit holds, and one pass
// replaces the chunked score, the merge and the attention launch.
#include "gqa_tile.h"
#include "score_common.h"

namespace ds {
namespace {

constexpr int kNTG = 1024;
constexpr int kWG = kNTG / 64;  // waves
constexpr int kFusedGPages = 16384 / 16;  // page-table entries of the longest row

template <int JMAX, bool PAGED>
struct FusedGScratch {
  __half qrows[kMaxGroup][256];  // the group's query rows
  int32_t chan[128];
  int32_t keep[128];
  __half knew[128];  // K row of the appended token
  float lnew[128];   // its label values (int4: codes)
  QueryLds q;        // the summed, gathered query
  float snew;        // the appended token's score
  float mm_tmp[2 * kWG];
  uint32_t scan_tmp[kWG];
  SelScratch sel;
  uint32_t tot[JMAX * kWG];  // per round and wave: taken | equal << 16
  alignas(16) __half qk[kMaxGroup][kDv];  // query rows at the stored K columns' channels
  int32_t lidx[kDecodeFusedMaxK];
  int32_t junk[64];  // spare words of the list writes
  AttnRed<kMaxGroup, kWG> red;
  int32_t ptab[PAGED ? kFusedGPages : 1];  // the row's page-table entries (paged pool)
};

// TPTC: tokens per thread before rounding up to whole label vectors.
// PAGED: K/V in a paged pool (the row's page-table entries staged in LDS).
template <int R, bool INT4, int TPTC, bool PAGED, bool HEADS>
__global__ __launch_bounds__(kNTG) void k_decode_fused_g(ScoreArgs sa_in, AttnArgs aa_in,
                                                       LabelArgs la_in, int append) {
  using Vec = typename VecSel<R, INT4>::type;
  constexpr int VT = Vec::VT;
  constexpr int JMAX = (TPTC + VT - 1) / VT;  // rounds of vectors per thread
  constexpr int TPT = JMAX * VT;
  // label vectors in flight per thread: all of them when they fit in about
  // 72 registers, else 4 at a time
  constexpr int UNR = JMAX * (int)sizeof(Vec) <= 288 ? JMAX : 4;
  __shared__ FusedGScratch<JMAX, PAGED> f;

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
  const int G = sa.G;
  const int tid = threadIdx.x;
  if (HEADS && aa.d_k == 0) {  // a fully pruned head: no token, zero output
    if (sa.pad_idx)
      for (int i = tid; i < sa.idx_stride; i += kNTG) sa.idx[(int64_t)row * sa.idx_stride + i] = -1;
    if (tid < G * (kDv / 8))
      *reinterpret_cast<uint4*>(aa.out + ((int64_t)b * aa.Hq + (int64_t)g * G) * kDv + tid * 8) =
          make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  const int lane = tid & 63;
  const int w = wave_id();
  const int r = sa.r;
  const int t_new = S - 1;
  const bool do_append = append && S >= 1;
  const bool sparse = sa.k > 0 && S > sa.k;

  // --- setup ----------------------------------------------------------------
  // The small loads (query rows, heavy channels, kept columns) go out first,
  // then the whole label stream, and only then are the small values written
  // to LDS, so their wait does not hold the label loads back.  Every label
  // load is unconditional (lanes past the batch bound max_seq re-read its
  // last vector): a path that issued fewer loads after the small ones would
  // make their wait cover the whole stream.
  const __half* qh = sa.q + ((int64_t)b * sa.Hq + (int64_t)g * G) * sa.d_q;
  const int nq = G * sa.d_q;  // <= 2 * kNTG
  __half qv0 = __float2half(0.0f), qv1 = __float2half(0.0f);
  int chv = 0, kpv = 0;
  if (tid < nq) qv0 = qh[tid];
  if (tid + kNTG < nq) qv1 = qh[tid + kNTG];
  if (tid < r) chv = sa.chan[(int64_t)g * r + tid];
  if (sa.keep && tid < sa.keep_ld) kpv = sa.keep[(int64_t)g * sa.keep_ld + tid];

  const RowPtrs p = row_ptrs(sa, row);
  const int n_vec = sparse ? (S + VT - 1) / VT : 0;
  const int v_last = n_vec - 1;  // the only vector that may be partial; it holds t_new
  const int jn = (n_vec + kNTG - 1) / kNTG;  // rounds holding any vector (uniform)
  // The label loads go out before the row's length arrives: every slot below
  // the batch bound max_seq (<= slots, a multiple of 16) is fetched.
  const int n_vec_ld =
      sa.k > 0 && sa.max_seq > sa.k ? (min(sa.max_seq, sa.slots) + VT - 1) / VT : 0;
  const int v_ld = max(n_vec_ld, 1) - 1;
  Vec vec[UNR];
#pragma unroll
  for (int u = 0; u < UNR; ++u) vec[u].load(p, min(u * kNTG + tid, v_ld));
  if (PAGED) {
    const int npg = (sa.max_seq + (1 << aa.pshift) - 1) >> aa.pshift;
    for (int i = tid; i < npg; i += kNTG) f.ptab[i] = aa.ptab[(int64_t)b * aa.max_pages + i];
  }
  if (tid < nq) f.qrows[tid / sa.d_q][tid % sa.d_q] = qv0;
  if (tid + kNTG < nq) f.qrows[(tid + kNTG) / sa.d_q][(tid + kNTG) % sa.d_q] = qv1;
  if (tid < r) f.chan[tid] = chv;
  if (sa.keep && tid < sa.keep_ld) f.keep[tid] = kpv;
  __syncthreads();
  {
    // qg[j] = sum over the group's heads of q[h][keep[chan[j]]], in head order
    float qgv = 0.0f;
    if (tid < r) {
      const int col = f.chan[tid];
      const int qc = sa.keep ? f.keep[col] : col;
      for (int h = 0; h < G; ++h) qgv += h2f(f.qrows[h][qc]);
    }
    store_query(INT4, r, qgv, f.q);
    for (int i = tid; i < G * kDv; i += kNTG) {
      const int h = i / kDv, c = i - h * kDv;
      f.qk[h][c] = c < aa.d_k ? f.qrows[h][sa.keep ? f.keep[c] : c] : __float2half(0.0f);
    }
  }
  __syncthreads();

  // The append runs on the last wave: the first one holds the row's tail
  // vectors (round JMAX - 1 when S is just above a multiple of 1024 VT).  It
  // fetches the appended token's K row itself, behind its own label loads.
  constexpr int kAppendWave = kWG - 1;
  auto append_new = [&](bool with_score) {
    if (lane < (la.d_k >> 3)) {
      const __half* kr = la.K + kv_off(la.ptab, la.pshift, la.max_pages, b, t_new, la.ks0, la.ks2) +
                         (int64_t)g * la.ks1;
      *reinterpret_cast<uint4*>(&f.knew[lane * 8]) = *reinterpret_cast<const uint4*>(kr + lane * 8);
    }
    __builtin_amdgcn_wave_barrier();
    append_label<R, INT4>(la, row, t_new, f, r, with_score);
  };
  // List position i is token f.lidx[i] on the sparse path and token i on the
  // dense one.
  auto tok = [&](int i) -> int64_t {
    const int t = sparse ? f.lidx[i] : i;
    return PAGED ? (int64_t)phys_tok(f.ptab, aa.pshift, t) : (int64_t)t;
  };
  auto token = [&](int j, int e) { return (j * kNTG + tid) * VT + e; };
  auto valid = [&](int j, int) { return j < jn; };  // empty slots hold -inf
  const int n_att = sparse ? sa.k : S;  // tokens attended
  const GqaLane ln(aa, b, g, PAGED);
  GqaTile cur;         // the wave's tile in registers
  bool early = false;  // its first tile was loaded during the select
  if (!sparse) {
    if (do_append && w == kAppendWave) append_new(false);
    if (sa.pad_idx) {
      int32_t* out = sa.idx + (int64_t)row * sa.idx_stride;
      for (int i = tid; i < sa.idx_stride; i += kNTG) out[i] = i < S ? i : -1;
    }
    // label loads issued ahead of the row length are not used here
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  } else {
    sel_clear<kNTG>(f.sel);  // published by the barrier after the scores
    if (do_append && w == kAppendWave) append_new(true);
    typename Vec::Q q;
    q.load(f.q);
    // --- score into registers ----------------------------------------------
    constexpr float kEmpty = -__builtin_huge_valf();
    float sc[TPT];
    float mn = __builtin_huge_valf(), mx = kEmpty;
#pragma unroll
    for (int j0 = 0; j0 < JMAX; j0 += UNR) {
      if (j0 > 0) {
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int v = (j0 + u) * kNTG + tid;
          if (j0 + u < JMAX && v < n_vec) vec[u].load(p, v);
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int j = j0 + u;
        if (j >= JMAX) continue;
        const int v = j * kNTG + tid;
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
      f.mm_tmp[kWG + w] = mx;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kWG; ++i) {
      mn = fminf(mn, f.mm_tmp[i]);
      mx = fmaxf(mx, f.mm_tmp[kWG + i]);
    }
    if (do_append) {
      const float sn = f.snew;
      if ((v_last & (kNTG - 1)) == tid) {
        const int jl = v_last / kNTG;
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
    const ListSel ls = list_select_a<kNTG, VT, JMAX, true>(sc, valid, token, (uint32_t)sa.k, bin,
                                                           f.sel, f.scan_tmp, f.lidx, f.junk);
    if (!sa.pad_idx && ls.cnt <= (uint32_t)kRankMax) {
      // The wave's first tile, when it lies in the part of the list already
      // complete (tokens above the boundary bin), is loaded while the few
      // boundary candidates are ranked.
      const int i0 = w * kGqaTile;
      if (i0 + kGqaTile <= (int)ls.n_a) {
        gqa_load<PAGED>(aa, ln, i0, n_att, tok, cur);
        early = true;
      }
      list_rank<kNTG>(ls, f.sel, f.lidx);
    } else {
      const RegSel rs = list_select_b<kNTG, VT, JMAX>(sc, valid, token, bin, ls, f.sel,
                                                      f.scan_tmp, f.tot, f.lidx);
      if (sa.pad_idx) {  // caller asked for the selected set, ascending
        int32_t* out = sa.idx + (int64_t)row * sa.idx_stride;
        reg_emit<kNTG, VT, JMAX>(sc, valid, rs, f.tot,
                                 [&](uint32_t pos, int j, int e) { out[pos] = token(j, e); });
        for (int i = sa.k + tid; i < sa.idx_stride; i += kNTG) out[i] = -1;
      }
    }
  }

  // --- attention -----------------------------------------------------------------
  // Each wave takes every 16th tile of the list, one tile in registers.
  half4_t qb[8];
  gqa_query(&f.qk[0][0], G, ln, qb);
  GqaState st;
  gqa_init(st);
  constexpr int D = kWG * kGqaTile;  // the wave's tiles are D positions apart
  for (int i0 = w * kGqaTile; i0 < n_att; i0 += D) {
    if (!early) gqa_load<PAGED>(aa, ln, i0, n_att, tok, cur);
    early = false;
    gqa_tile(cur, qb, i0, n_att, aa.scale_log2, ln.kg, st);
  }
  gqa_to_red(st, ln, G, w, f.red);
  __syncthreads();
  gqa_merge_out(aa, f.red, b, g, G);
}

template <int R, bool INT4, int TPTC, bool HEADS>
hipError_t launch_rt(const ScoreArgs& sa, const AttnArgs& aa, const LabelArgs& la, int append,
                     int rows, hipStream_t s, const KEvents& ev) {
  if (aa.ptab)
    return launch_k(k_decode_fused_g<R, INT4, TPTC, true, HEADS>, dim3(rows), dim3(kNTG), s, ev,
                    sa, aa, la, append);
  return launch_k(k_decode_fused_g<R, INT4, TPTC, false, HEADS>, dim3(rows), dim3(kNTG), s, ev,
                  sa, aa, la, append);
}

template <int TPTC, bool HEADS>
hipError_t launch_tpt(const ScoreArgs& sa, const AttnArgs& aa, const LabelArgs& la, int append,
                      int rows, hipStream_t s, const KEvents& ev) {
  if (sa.is_int4) {
    if (sa.r == 8) return launch_rt<8, true, TPTC, HEADS>(sa, aa, la, append, rows, s, ev);
    if (sa.r == 16) return launch_rt<16, true, TPTC, HEADS>(sa, aa, la, append, rows, s, ev);
    return launch_rt<0, true, TPTC, HEADS>(sa, aa, la, append, rows, s, ev);
  }
  if (sa.r == 8) return launch_rt<8, false, TPTC, HEADS>(sa, aa, la, append, rows, s, ev);
  if (sa.r == 16) return launch_rt<16, false, TPTC, HEADS>(sa, aa, la, append, rows, s, ev);
  return launch_rt<0, false, TPTC, HEADS>(sa, aa, la, append, rows, s, ev);
}

// Tokens per thread before rounding up to whole label vectors (1, 2 or 4
// tokens): the smallest class that holds the longest row.
constexpr int kTptClass[3] = {4, 9, 16};

int vec_tokens(int r, int is_int4) {
  if (!is_int4 || (r != 8 && r != 16)) return 1;
  return r == 8 ? 4 : 2;
}

int rows_capacity(int tptc, int r, int is_int4) {
  const int vt = vec_tokens(r, is_int4);
  return kNTG * ((tptc + vt - 1) / vt) * vt;
}

}  // namespace

bool decode_fused_g_fits(int max_seq, int k, int r, int is_int4, int G) {
  return G >= 2 && G <= kMaxGroup && max_seq <= rows_capacity(kTptClass[2], r, is_int4) &&
         (k >= max_seq || k <= kDecodeFusedMaxK);
}

hipError_t launch_decode_fused_g(const ScoreArgs& sa, const AttnArgs& aa, const LabelArgs& la,
                                 int append, int rows, hipStream_t s, const KEvents& ev) {
  if (rows <= 0) return hipSuccess;
  // per-head layouts: the widest class only (it holds every accepted length)
  if (aa.heads) return launch_tpt<kTptClass[2], true>(sa, aa, la, append, rows, s, ev);
  if (sa.max_seq <= rows_capacity(kTptClass[0], sa.r, sa.is_int4))
    return launch_tpt<kTptClass[0], false>(sa, aa, la, append, rows, s, ev);
  if (sa.max_seq <= rows_capacity(kTptClass[1], sa.r, sa.is_int4))
    return launch_tpt<kTptClass[1], false>(sa, aa, la, append, rows, s, ev);
  return launch_tpt<kTptClass[2], false>(sa, aa, la, append, rows, s, ev);
}

}  // namespace ds
