// api.hip -- the extern "C" entry points declared in ds.h: host-side
// validation, workspace planning and kernel launches on the caller's stream.
//
// Pages cited by title and section:
//   [DS]    "Double Sparsity" article, joto.ai blog archive 2025060420469,
//           sections "offline calibration", "online forward computation"
//           and "use in SGLang" (heavy-token count k; dense below threshold).
//   [LeanK] LeanK article, aitangshan.cn news 1293675, section 2.2.
//   [GQA]   grouped-query attention article, trdm.cn news 80600, section 4.
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "ds_internal.h"

namespace ds {
namespace {

constexpr int64_t kMaxCapacity = int64_t(1) << 24;
constexpr int kScoreChunk = 4096;      // tokens per chunked-score workgroup
constexpr int64_t kLocalSlotsPerCu = 256;  // compute units: chunk workgroups of 2048 threads per CU
constexpr int kTargetAttnBlocks = 1024;
constexpr int kMinTokensPerSplit = 64;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Paged pool: page size a power of two in [16, 65536], table given, the
// capacity exactly max_pages pages, physical token ids (page << log2(page
// size) | slot) below 2^31.  Contiguous rows: no paging fields.
ds_status check_pages(const ds_kv_desc* kv) {
  const int P = kv->page_size;
  if (P == 0) return (kv->page_table || kv->max_pages || kv->n_pages) ? DS_ERR_ARG : DS_OK;
  if (P < 16 || P > 65536 || (P & (P - 1))) return DS_ERR_SHAPE;
  if (!kv->page_table) return DS_ERR_ARG;
  if (kv->max_pages < 1 || kv->n_pages < 1) return DS_ERR_SHAPE;
  if ((int64_t)kv->max_pages * P != kv->capacity) return DS_ERR_SHAPE;
  if ((int64_t)kv->n_pages * P > INT32_MAX) return DS_ERR_SHAPE;
  return DS_OK;
}

int log2i(int v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

// K-side fields (all calls) and, for decode, the query and V fields.
ds_status check_kv(const ds_kv_desc* kv, bool decode) {
  if (!kv) return DS_ERR_ARG;
  if (kv->batch < 1 || kv->n_kv_heads < 1) return DS_ERR_SHAPE;
  if (kv->d_k < 8 || kv->d_k > 128 || kv->d_k % 8) return DS_ERR_SHAPE;
  if (kv->capacity < 1 || kv->capacity > kMaxCapacity) return DS_ERR_SHAPE;
  for (int i = 0; i < 3; ++i) {
    if (kv->k_stride[i] < 0) return DS_ERR_SHAPE;
    if (kv->k_stride[i] % 8) return DS_ERR_ALIGN;
  }
  if (ds_status st = check_pages(kv)) return st;
  if (!decode) return DS_OK;
  if (kv->n_q_heads < 1 || kv->n_q_heads % kv->n_kv_heads) return DS_ERR_SHAPE;
  if (kv->n_q_heads / kv->n_kv_heads > kMaxGroup) return DS_ERR_SHAPE;
  if (kv->d_q < 1 || kv->d_q > 256) return DS_ERR_SHAPE;
  if (kv->d_v != kDv) return DS_ERR_SHAPE;
  for (int i = 0; i < 3; ++i) {
    if (kv->v_stride[i] < 0) return DS_ERR_SHAPE;
    if (kv->v_stride[i] % 8) return DS_ERR_ALIGN;
  }
  return DS_OK;
}

ds_status check_lab(const ds_kv_desc* kv, const ds_label_desc* lab) {
  if (!lab || lab->reserved0 != 0) return DS_ERR_ARG;
  if (lab->dtype != DS_LABEL_F16 && lab->dtype != DS_LABEL_INT4) return DS_ERR_DTYPE;
  if (lab->r < 1 || lab->r > std::min(kv->d_k, 128)) return DS_ERR_SHAPE;
  if (lab->dtype == DS_LABEL_INT4 && (lab->r & 1)) return DS_ERR_DTYPE;
  if (lab->slots < kv->capacity || lab->slots % 16) return DS_ERR_SHAPE;
  if (!lab->codes) return DS_ERR_ARG;
  if (!aligned16(lab->codes)) return DS_ERR_ALIGN;
  if (lab->dtype == DS_LABEL_INT4) {
    if (!lab->scales) return DS_ERR_ARG;
    if (!aligned16(lab->scales)) return DS_ERR_ALIGN;
  }
  return DS_OK;
}

LabelArgs label_args(const ds_kv_desc* kv, const void* K, const int32_t* chan,
                     const ds_label_desc* lab) {
  LabelArgs a;
  memset(&a, 0, sizeof(a));
  a.K = static_cast<const __half*>(K);
  a.ks0 = kv->k_stride[0];
  a.ks1 = kv->k_stride[1];
  a.ks2 = kv->k_stride[2];
  a.Hkv = kv->n_kv_heads;
  a.d_k = kv->d_k;
  a.cap = kv->capacity;
  a.chan = chan;
  if (kv->page_size) {
    a.ptab = kv->page_table;
    a.pshift = log2i(kv->page_size);
    a.max_pages = kv->max_pages;
  }
  a.heads = kv->heads;
  a.r = lab->r;
  a.is_int4 = lab->dtype == DS_LABEL_INT4;
  a.slots = lab->slots;
  if (a.is_int4) {
    a.codes = static_cast<uint8_t*>(lab->codes);
    a.scales = static_cast<__half*>(lab->scales);
  } else {
    a.lab16 = static_cast<__half*>(lab->codes);
  }
  return a;
}

// Everything ds_decode_attn derives from the shapes alone.
struct Plan {
  bool sparse;
  int kk;           // tokens attended per row at most
  int idx_cap;      // workspace index slots per row
  int keys_stride;  // workspace key words per row
  int n_chunks;     // streaming select: score chunks per row
  int local_chunk;  // local top-M select: tokens per chunk workgroup
  int local_nch;    // and chunks per row
  int cand_stride;  // candidate slots per row
  bool local_half;  // the local quota of every row is at least 512
  int split_cap;
  size_t off_count, off_idx, off_keys, off_cand_key, off_cand_idx, off_cand_cnt, off_cand_theta,
      off_cand_range;
  size_t off_part, total;
};

Plan make_plan(const ds_kv_desc* kv, int k, int max_seq) {
  Plan p;
  memset(&p, 0, sizeof(p));
  const int64_t rows = (int64_t)kv->batch * kv->n_kv_heads;
  p.sparse = k > 0;
  p.kk = p.sparse ? std::min(k, max_seq) : max_seq;
  p.idx_cap = p.sparse ? std::max(p.kk, 1) : 0;
  p.keys_stride = p.sparse ? (int)round_up(std::max(max_seq, 1), 64) : 0;
  p.n_chunks = (int)std::max<int64_t>(1, ceil_div(max_seq, kScoreChunk));
  // Local top-M chunks (at least 1024 tokens unless the row is shorter).  A
  // chunk workgroup costs a fixed latency plus its tokens per thread, and the
  // chunks run in rounds of as many workgroups as the chip holds at once
  // (1024 of 512 threads, 2048 of 256): a single round costs its latency
  // however full it is, while beyond one round workgroups start as others
  // finish, so the rounds count in proportion to the workgroups.  A
  // 512-thread workgroup's fixed latency is one unit above a 256-thread
  // one's (its barriers and block scans span eight waves).  The merge then
  // costs about its candidates (quota per chunk, twice the expected share of
  // k) per merge thread.  Pick the chunk count with the lowest total.
  {
    const int64_t S = std::max(max_seq, 1);
    double best = 1e300;
    p.local_chunk = kMaxLocalChunk;
    const int64_t n_hi = std::min<int64_t>(kMaxLocalChunks, std::max<int64_t>(1, ceil_div(S, 1024)));
    for (int64_t n = ceil_div(S, kMaxLocalChunk); n <= n_hi; ++n) {
      const int64_t chunk = round_up(ceil_div(S, n), 64);
      const int64_t nch = ceil_div(S, chunk);
      const int threads = chunk > 4096 ? 512 : 256;
      const int64_t slots = kLocalSlotsPerCu * (2048 / threads);
      const double rounds = std::max(1.0, (double)(rows * nch) / (double)slots);
      const double quota = std::min<double>((double)chunk,
                                            std::max(64.0, 2.0 * std::max(k, 0) * chunk / S + 1));
      const double fixed = threads == 512 ? 17.0 : 16.0;
      const double cost = rounds * (fixed + (double)ceil_div(chunk, threads)) + nch * quota / 1024.0;
      if (cost < best - 1e-9) {
        best = cost;
        p.local_chunk = (int)chunk;
      }
    }
  }
  p.local_nch = (int)std::max<int64_t>(1, ceil_div(max_seq, p.local_chunk));
  p.cand_stride = p.sparse ? (int)std::min<int64_t>(kMergeCap, round_up(std::max(max_seq, 1), 64)) : 0;
  {
    // The local score kernel's quota for a row of max_seq tokens (the
    // smallest of any row: shorter rows expect more of k per chunk and own
    // more slots); at least 520 lets the large-chunk kernel take its
    // threshold from a sample of half the chunk (the kernel checks 512).
    const int64_t S = std::max(max_seq, 1);
    const int64_t CH = p.local_chunk, nch = p.local_nch;
    const double expected = (double)std::max(k, 0) * (double)CH / (double)S;
    int64_t m0 = std::min<int64_t>(CH, std::max<int64_t>(64, (int64_t)(2.0 * expected) + 1));
    const int64_t cap = std::min<int64_t>(p.cand_stride / nch, m0 + m0 / 8 + 64);
    p.local_half = p.sparse && std::min<int64_t>(m0, cap - cap / 8) >= 520;
  }
  p.split_cap = (int)std::min<int64_t>(kMaxSplit, std::max<int64_t>(1, ceil_div(p.kk, 16)));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (size_t)round_up((int64_t)bytes, 256);
    return at;
  };
  p.off_count = take(rows * sizeof(int32_t));
  p.off_idx = take(rows * (size_t)p.idx_cap * sizeof(int32_t));
  p.off_keys = take(rows * (size_t)p.keys_stride * sizeof(uint32_t));
  const size_t nch = p.sparse ? (size_t)p.local_nch : 0;
  p.off_cand_key = take(rows * (size_t)p.cand_stride * sizeof(uint32_t));
  p.off_cand_idx = take(rows * (size_t)p.cand_stride * sizeof(int32_t));
  p.off_cand_cnt = take(rows * nch * sizeof(int32_t));
  p.off_cand_theta = take(rows * nch * sizeof(uint32_t));
  p.off_cand_range = take(rows * nch * 2 * sizeof(float));
  p.off_part = take((size_t)kv->batch * kv->n_q_heads * p.split_cap * kPartStride * sizeof(float));
  p.total = off;
  return p;
}

AttnArgs attn_args(const ds_kv_desc* kv, const void* q, const void* K, const void* V,
                   const int32_t* seq_lens, int max_seq_len, const int32_t* keep, float sm_scale,
                   void* out, char* ws, const Plan& p) {
  AttnArgs aa;
  memset(&aa, 0, sizeof(aa));
  aa.q = static_cast<const __half*>(q);
  aa.Hq = kv->n_q_heads;
  aa.d_q = kv->d_q;
  aa.K = static_cast<const __half*>(K);
  aa.V = static_cast<const __half*>(V);
  aa.ks0 = kv->k_stride[0];
  aa.ks1 = kv->k_stride[1];
  aa.ks2 = kv->k_stride[2];
  aa.vs0 = kv->v_stride[0];
  aa.vs1 = kv->v_stride[1];
  aa.vs2 = kv->v_stride[2];
  aa.Hkv = kv->n_kv_heads;
  aa.d_k = kv->d_k;
  aa.keep = keep;
  aa.seq_lens = seq_lens;
  aa.max_seq = max_seq_len;
  aa.scale_log2 = sm_scale * 1.4426950408889634f;
  aa.out = static_cast<__half*>(out);
  aa.part = reinterpret_cast<float*>(ws + p.off_part);
  if (kv->page_size) {
    aa.ptab = kv->page_table;
    aa.pshift = log2i(kv->page_size);
    aa.pmask = kv->page_size - 1;
    aa.max_pages = kv->max_pages;
  }
  aa.heads = kv->heads;
  aa.keep_ld = kv->d_k;
  return aa;
}

// Attention partitions per row: about kTargetAttnBlocks workgroups in all,
// each with at least 64 tokens.  Query groups: about half as many
// workgroups (the group kernel holds two per compute unit) of at least 256
// tokens (four 16-token tiles per wave); one split also saves the combine.
int auto_splits(const Plan& p, int64_t rows, int G, int requested) {
  int ns;
  if (requested > 0) {
    ns = requested;
  } else {
    const int min_tok = G > 1 ? 4 * kMinTokensPerSplit : kMinTokensPerSplit;
    const int target = G > 1 ? kTargetAttnBlocks / 2 : kTargetAttnBlocks;
    ns = (int)ceil_div(target, std::max<int64_t>(rows, 1));
    ns = (int)std::min<int64_t>(ns, std::max<int64_t>(1, ceil_div(p.kk, min_tok)));
  }
  return std::max(1, std::min(ns, p.split_cap));
}

// Which kernels a call runs, and the attention split.
struct Route {
  int path;  // DS_PATH_*
  int n_split, tps;
};

Route route(const ds_kv_desc* kv, const ds_label_desc* lab, int k, int max_seq, uint32_t flags,
            int n_split_req, const Plan& p) {
  Route r;
  const int G = kv->n_q_heads / kv->n_kv_heads;
  const int64_t rows = (int64_t)kv->batch * kv->n_kv_heads;
  if (!p.sparse)
    r.path = DS_PATH_DENSE;
  else if (G == 1 && !(flags & (DS_DECODE_UNFUSED | DS_DECODE_STREAM)) &&
           decode_fused_fits(max_seq, k, lab->r, lab->dtype == DS_LABEL_INT4))
    r.path = DS_PATH_FUSED;
  else if (G > 1 && !(flags & (DS_DECODE_UNFUSED | DS_DECODE_STREAM)) &&
           decode_fused_g_fits(max_seq, k, lab->r, lab->dtype == DS_LABEL_INT4, G))
    r.path = DS_PATH_FUSED;
  else if (!(flags & DS_DECODE_STREAM) && p.local_nch <= kMaxLocalChunks)
    r.path = DS_PATH_LOCAL;
  else
    r.path = DS_PATH_STREAM;
  if (r.path == DS_PATH_FUSED) {
    r.n_split = 1;
    r.tps = std::max(p.kk, 1);
    return r;
  }
  r.n_split = auto_splits(p, rows, G, n_split_req);
  r.tps = (int)std::max<int64_t>(1, round_up(ceil_div(std::max(p.kk, 1), r.n_split), 16));
  r.n_split = (int)std::max<int64_t>(1, ceil_div(std::max(p.kk, 1), r.tps));
  return r;
}

}  // namespace
}  // namespace ds

using namespace ds;

extern "C" {

// Takes the code as a plain integer: any value may arrive here, and a
// ds_status outside its enumerators would not be a valid enum value.
const char* ds_status_str(int32_t status) {
  switch (status) {
    case DS_OK: return "ok";
    case DS_ERR_ARG: return "invalid argument";
    case DS_ERR_SHAPE: return "unsupported or inconsistent shape";
    case DS_ERR_DTYPE: return "unsupported label dtype";
    case DS_ERR_ALIGN: return "misaligned pointer or stride";
    case DS_ERR_WORKSPACE: return "workspace too small";
    case DS_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int32_t ds_abi_version(void) { return DS_ABI_VERSION; }

ds_status ds_label_build(const ds_kv_desc* kv, const void* K, const int32_t* chan,
                         const ds_label_desc* lab, int32_t t_begin, int32_t t_end,
                         hipStream_t stream) {
  ds_status st = check_kv(kv, false);
  if (st) return st;
  if ((st = check_lab(kv, lab))) return st;
  if (!K || !chan) return DS_ERR_ARG;
  if (!aligned16(K)) return DS_ERR_ALIGN;
  if (t_begin < 0 || t_end < t_begin || t_end > kv->capacity) return DS_ERR_ARG;
  if (t_end == t_begin) return DS_OK;
  LabelArgs a = label_args(kv, K, chan, lab);
  a.t_begin = t_begin;
  a.t_end = t_end;
  a.tiles_per_row = (int)ceil_div(t_end - t_begin, 64);
  const int64_t blocks = (int64_t)kv->batch * kv->n_kv_heads * a.tiles_per_row;
  if (blocks > INT32_MAX / 256) return DS_ERR_SHAPE;
  return launch_label(a, (int)blocks, stream) == hipSuccess ? DS_OK : DS_ERR_HIP;
}

ds_status ds_label_append(const ds_kv_desc* kv, const void* K, const int32_t* chan,
                          const ds_label_desc* lab, const int32_t* pos, hipStream_t stream) {
  ds_status st = check_kv(kv, false);
  if (st) return st;
  if ((st = check_lab(kv, lab))) return st;
  if (!K || !chan || !pos) return DS_ERR_ARG;
  if (!aligned16(K)) return DS_ERR_ALIGN;
  LabelArgs a = label_args(kv, K, chan, lab);
  a.pos = pos;
  a.n_items = kv->batch * kv->n_kv_heads;
  return launch_label(a, (int)ceil_div(a.n_items, 64), stream) == hipSuccess ? DS_OK : DS_ERR_HIP;
}

size_t ds_decode_attn_workspace_size(const ds_kv_desc* kv, const ds_label_desc* lab, int32_t k,
                                     int32_t max_seq_len) {
  if (check_kv(kv, true)) return 0;
  if (k > 0 && check_lab(kv, lab)) return 0;
  if (max_seq_len < 0 || max_seq_len > kv->capacity) return 0;
  return make_plan(kv, k, max_seq_len).total;
}

ds_status ds_decode_attn_plan(const ds_kv_desc* kv, const ds_label_desc* lab, int32_t k,
                              int32_t max_seq_len, const ds_decode_opts* opts,
                              ds_decode_plan* plan) {
  if (!plan) return DS_ERR_ARG;
  ds_status st = check_kv(kv, true);
  if (st) return st;
  if (k > 0 && (st = check_lab(kv, lab))) return st;
  if (max_seq_len < 0 || max_seq_len > kv->capacity) return DS_ERR_ARG;
  if (opts && opts->n_split < 0) return DS_ERR_ARG;
  const uint32_t flags = opts ? opts->flags : 0u;
  const Plan p = make_plan(kv, k, max_seq_len);
  const Route r = route(kv, lab, k, max_seq_len, flags, opts ? opts->n_split : 0, p);
  plan->path = r.path;
  plan->n_split = r.n_split;
  plan->tokens_per_split = r.tps;
  int n = 1;  // the attention pass, or the fused kernel
  if (r.path == DS_PATH_LOCAL) n += 2;
  if (r.path == DS_PATH_STREAM) n += 2 + ((flags & DS_DECODE_APPEND) ? 1 : 0);
  if (r.path == DS_PATH_DENSE && (flags & DS_DECODE_APPEND)) ++n;
  if (r.path != DS_PATH_FUSED && r.n_split > 1) ++n;
  plan->kernels = n;
  plan->chunk = r.path == DS_PATH_LOCAL ? p.local_chunk : (r.path == DS_PATH_STREAM ? kScoreChunk : 0);
  plan->reserved0 = 0;
  plan->workspace_bytes = p.total;
  return DS_OK;
}

}  // extern "C"

namespace ds {
namespace {

// The decode step behind both decode entry points: validation, plan, launches.
ds_status decode_impl(const ds_kv_desc* kv, const void* q, const void* K, const void* V,
                      const int32_t* seq_lens, int32_t max_seq_len, const int32_t* keep,
                      const int32_t* chan, const ds_label_desc* lab, int32_t k, float sm_scale,
                      void* out, int32_t* topk_idx, void* workspace, size_t workspace_bytes,
                      const ds_decode_opts* opts, hipStream_t stream) {
  ds_status st = check_kv(kv, true);
  if (st) return st;
  const bool sparse = k > 0;
  const uint32_t flags = opts ? opts->flags : 0u;
  if (sparse || (flags & DS_DECODE_APPEND)) {  // a dense step may still append labels
    if ((st = check_lab(kv, lab))) return st;
    if (!chan) return DS_ERR_ARG;
  }
  if (!q || !K || !V || !seq_lens || !out) return DS_ERR_ARG;
  if (!aligned16(K) || !aligned16(V) || !aligned16(out)) return DS_ERR_ALIGN;
  if (!keep && kv->d_k != kv->d_q) return DS_ERR_SHAPE;
  if (max_seq_len < 0 || max_seq_len > kv->capacity) return DS_ERR_ARG;
  if (flags & ~(DS_DECODE_APPEND | DS_DECODE_VALIDATE_ONLY | DS_DECODE_UNFUSED | DS_DECODE_STREAM))
    return DS_ERR_ARG;
  if (opts && opts->n_split < 0) return DS_ERR_ARG;
  if (!std::isfinite(sm_scale)) return DS_ERR_ARG;

  const Plan p = make_plan(kv, k, max_seq_len);
  if (workspace_bytes < p.total) return DS_ERR_WORKSPACE;
  if (p.total > 0 && !workspace) return DS_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return DS_ERR_ALIGN;
  if (flags & DS_DECODE_VALIDATE_ONLY) return DS_OK;

  const int B = kv->batch, Hkv = kv->n_kv_heads, G = kv->n_q_heads / kv->n_kv_heads;
  const int64_t rows = (int64_t)B * Hkv;
  char* ws = static_cast<char*>(workspace);
  hipEvent_t* ev = opts ? opts->stage_events : nullptr;
  // Kernel timing: when exactly two adjacent slots i and i + 1 are given,
  // stage i's launch records them at the kernel's own start and end (a stage
  // that launches nothing records them back to back); otherwise every given
  // slot is recorded on the stream between the stages.
  int own = -1;
  if (ev) {
    int n = 0, first = -1;
    for (int i = 0; i <= DS_STAGE_COUNT; ++i)
      if (ev[i]) {
        ++n;
        if (first < 0) first = i;
      }
    if (n == 2 && first < DS_STAGE_COUNT && ev[first + 1]) own = first;
  }
  bool own_done = false;
  auto kev = [&](int i) {
    KEvents e;
    if (own == i) {
      e.start = ev[i];
      e.stop = ev[i + 1];
      own_done = true;
    }
    return e;
  };
  auto mark = [&](int i) {
    if (own < 0 && ev && ev[i]) (void)hipEventRecord(ev[i], stream);
  };
  auto mark_end = [&]() {
    if (own >= 0 && !own_done) {
      (void)hipEventRecord(ev[own], stream);
      (void)hipEventRecord(ev[own + 1], stream);
    }
    mark(DS_STAGE_COUNT);
  };

  mark(DS_STAGE_APPEND);
  // Paths for the score and select: one kernel for the whole step (rows
  // whose scores fit in one workgroup's registers), local top-M + exact
  // merge, or a full streaming select over every score.
  const Route rt = route(kv, lab, k, max_seq_len, flags, opts ? opts->n_split : 0, p);
  const bool fused_step = rt.path == DS_PATH_FUSED;
  const bool local_path = rt.path == DS_PATH_LOCAL;
  if ((flags & DS_DECODE_APPEND) && !fused_step && !local_path) {
    LabelArgs la = label_args(kv, K, chan, lab);
    la.pos = seq_lens;
    la.pos_minus_one = 1;
    la.n_items = (int)rows;
    if (launch_label(la, (int)ceil_div(rows, 64), stream, kev(DS_STAGE_APPEND)) != hipSuccess)
      return DS_ERR_HIP;
  }

  const int32_t* idx = nullptr;
  int idx_stride = 0;
  int32_t* count = reinterpret_cast<int32_t*>(ws + p.off_count);
  mark(DS_STAGE_SCORE);
  if (sparse) {
    ScoreArgs sa;
    memset(&sa, 0, sizeof(sa));
    sa.q = static_cast<const __half*>(q);
    sa.Hq = kv->n_q_heads;
    sa.d_q = kv->d_q;
    sa.Hkv = Hkv;
    sa.G = G;
    sa.d_k = kv->d_k;
    sa.keep_ld = kv->d_k;
    sa.heads = kv->heads;
    sa.keep = keep;
    sa.chan = chan;
    sa.r = lab->r;
    sa.is_int4 = lab->dtype == DS_LABEL_INT4;
    sa.slots = lab->slots;
    if (sa.is_int4) {
      sa.codes = static_cast<const uint8_t*>(lab->codes);
      sa.scales = static_cast<const __half*>(lab->scales);
    } else {
      sa.lab16 = static_cast<const __half*>(lab->codes);
    }
    sa.seq_lens = seq_lens;
    sa.max_seq = max_seq_len;
    sa.k = k;
    if (topk_idx) {
      sa.idx = topk_idx;
      sa.idx_stride = k;
      sa.pad_idx = 1;
    } else {
      sa.idx = reinterpret_cast<int32_t*>(ws + p.off_idx);
      sa.idx_stride = p.idx_cap;
    }
    sa.count = count;
    sa.keys = reinterpret_cast<uint32_t*>(ws + p.off_keys);
    sa.keys_stride = p.keys_stride;
    sa.chunk = kScoreChunk;
    sa.n_chunks = p.n_chunks;
    sa.cand_score = reinterpret_cast<float*>(ws + p.off_cand_key);
    sa.cand_idx = reinterpret_cast<int32_t*>(ws + p.off_cand_idx);
    sa.cand_cnt = reinterpret_cast<int32_t*>(ws + p.off_cand_cnt);
    sa.cand_theta = reinterpret_cast<uint32_t*>(ws + p.off_cand_theta);
    sa.cand_range = reinterpret_cast<float2*>(ws + p.off_cand_range);
    sa.cand_stride = p.cand_stride;
    sa.half_quota = p.local_half ? 1 : 0;
    idx = sa.idx;
    idx_stride = sa.idx_stride;
    // One kernel for the whole step when the row's scores fit in one
    // workgroup's registers and its token list in LDS (256 threads for a
    // single query head, 1024 for a query group).
    if (fused_step) {
      LabelArgs la = label_args(kv, K, chan, lab);
      AttnArgs aa = attn_args(kv, q, K, V, seq_lens, max_seq_len, keep, sm_scale, out, ws, p);
      aa.n_split = 1;
      mark(DS_STAGE_SELECT);
      mark(DS_STAGE_ATTN);
      const int app = (flags & DS_DECODE_APPEND) ? 1 : 0;
      const hipError_t e =
          G == 1 ? launch_decode_fused(sa, aa, la, app, (int)rows, stream, kev(DS_STAGE_ATTN))
                 : launch_decode_fused_g(sa, aa, la, app, (int)rows, stream, kev(DS_STAGE_ATTN));
      if (e != hipSuccess) return DS_ERR_HIP;
      mark(DS_STAGE_COMBINE);
      mark_end();
      return DS_OK;
    }
    if (local_path) {
      LabelArgs la = label_args(kv, K, chan, lab);
      sa.chunk = p.local_chunk;
      sa.n_chunks = p.local_nch;
      if (launch_score_local(sa, la, (flags & DS_DECODE_APPEND) ? 1 : 0, (int)rows, stream,
                             kev(DS_STAGE_SCORE)) != hipSuccess)
        return DS_ERR_HIP;
      mark(DS_STAGE_SELECT);
      if (launch_select_merge(sa, (int)rows, stream, kev(DS_STAGE_SELECT)) != hipSuccess)
        return DS_ERR_HIP;
    } else {
      if (launch_score_chunks(sa, (int)rows, stream, kev(DS_STAGE_SCORE)) != hipSuccess)
        return DS_ERR_HIP;
      mark(DS_STAGE_SELECT);
      if (launch_select_stream(sa, (int)rows, stream, kev(DS_STAGE_SELECT)) != hipSuccess)
        return DS_ERR_HIP;
    }
  } else {
    mark(DS_STAGE_SELECT);
  }

  AttnArgs aa = attn_args(kv, q, K, V, seq_lens, max_seq_len, keep, sm_scale, out, ws, p);
  aa.sparse = sparse;
  aa.idx = idx;
  aa.idx_stride = idx_stride;
  aa.count = count;
  aa.n_split = rt.n_split;
  aa.tps = rt.tps;

  mark(DS_STAGE_ATTN);
  const bool final_out = aa.n_split == 1;
  if (launch_attn(aa, (int)rows, G, final_out, stream, kev(DS_STAGE_ATTN)) != hipSuccess)
    return DS_ERR_HIP;
  mark(DS_STAGE_COMBINE);
  if (!final_out && launch_combine(aa, B, stream, kev(DS_STAGE_COMBINE)) != hipSuccess)
    return DS_ERR_HIP;
  mark_end();
  return DS_OK;
}

// Scratch of ds_decode_attn_noalloc: one array per device, held from the
// code object's load until the process ends.  In host code its name is only
// a stand-in; the device address comes from hipGetSymbolAddress, once per
// device, and only that address is handed to the kernels.
static __device__ __align__(256) char scratch[DS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

ds_status scratch_ptr(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DS_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DS_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return DS_OK;
}

}  // namespace
}  // namespace ds

extern "C" {

ds_status ds_decode_attn(const ds_kv_desc* kv, const void* q, const void* K, const void* V,
                         const int32_t* seq_lens, int32_t max_seq_len, const int32_t* keep,
                         const int32_t* chan, const ds_label_desc* lab, int32_t k, float sm_scale,
                         void* out, int32_t* topk_idx, void* workspace, size_t workspace_bytes,
                         const ds_decode_opts* opts, hipStream_t stream) {
  return decode_impl(kv, q, K, V, seq_lens, max_seq_len, keep, chan, lab, k, sm_scale, out,
                     topk_idx, workspace, workspace_bytes, opts, stream);
}

ds_status ds_decode_attn_noalloc(const ds_kv_desc* kv, const void* q, const void* K,
                                 const void* V, const int32_t* seq_lens, int32_t max_seq_len,
                                 const int32_t* keep, const int32_t* chan,
                                 const ds_label_desc* lab, int32_t k, float sm_scale, void* out,
                                 int32_t* topk_idx, const ds_decode_opts* opts,
                                 hipStream_t stream) {
  void* ws = nullptr;
  const ds_status st = scratch_ptr(&ws);
  if (st != DS_OK) return st;
  return decode_impl(kv, q, K, V, seq_lens, max_seq_len, keep, chan, lab, k, sm_scale, out,
                     topk_idx, ws, DS_NOALLOC_SCRATCH_BYTES, opts, stream);
}

int32_t ds_sparse_decode_enabled(int32_t max_seq_len, int32_t min_seq_len, int32_t k,
                                 int32_t threshold) {
  return (k > 0 && max_seq_len >= threshold && min_seq_len >= k) ? 1 : 0;
}

ds_status ds_channel_overlap(const int32_t* chan_a, const int32_t* chan_b, int32_t n_kv_heads,
                             int32_t r, float* overlap) {
  if (!chan_a || !chan_b || !overlap || n_kv_heads < 1 || r < 1) return DS_ERR_ARG;
  constexpr int kIds = 4096;  // channel ids are K columns: far below this
  for (int64_t i = 0; i < (int64_t)n_kv_heads * r; ++i)
    if (chan_a[i] < 0 || chan_a[i] >= kIds || chan_b[i] < 0 || chan_b[i] >= kIds) return DS_ERR_ARG;
  for (int32_t g = 0; g < n_kv_heads; ++g) {
    // b's channels as a bitmap; each of a's channels counts once, when its
    // bit is still set, and clears it
    uint64_t bits[kIds / 64] = {};
    const int32_t* a = chan_a + (int64_t)g * r;
    const int32_t* b = chan_b + (int64_t)g * r;
    for (int32_t j = 0; j < r; ++j) bits[b[j] >> 6] |= 1ull << (b[j] & 63);
    int32_t shared = 0;
    for (int32_t j = 0; j < r; ++j) {
      const uint64_t m = 1ull << (a[j] & 63);
      if (bits[a[j] >> 6] & m) {
        ++shared;
        bits[a[j] >> 6] &= ~m;
      }
    }
    overlap[g] = (float)shared / (float)r;
  }
  return DS_OK;
}

size_t ds_calibrate_workspace_size(const ds_kv_desc* kv, int32_t n_tok, int32_t n_win) {
  if (check_kv(kv, false) || kv->page_size || kv->heads || n_tok < 0 || n_tok > kv->capacity || n_win < 0) return 0;
  if (n_win > 0 && (kv->n_q_heads < 1 || kv->n_q_heads % kv->n_kv_heads)) return 0;
  const int G = n_win > 0 ? kv->n_q_heads / kv->n_kv_heads : 1;
  const CalibPlan pl = calib_plan(kv->batch, kv->n_kv_heads, n_tok, kv->d_k, n_win * G);
  return std::max<size_t>(256, pl.ws_bytes);
}

ds_status ds_calibrate_channels(const ds_kv_desc* kv, const void* K, int32_t n_tok,
                                const void* qwin, int32_t n_win, const int32_t* keep,
                                int32_t criterion, int32_t r, int32_t* chan, float* norms,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  ds_status st = check_kv(kv, false);
  if (st) return st;
  if (kv->page_size || kv->heads) return DS_ERR_ARG;  // calibration samples: plain contiguous rows
  if (n_tok < 0 || n_tok > kv->capacity || n_win < 0) return DS_ERR_ARG;
  if (criterion < DS_CALIB_K || criterion > DS_CALIB_QK) return DS_ERR_ARG;
  if (r < 1 || r > kv->d_k || !chan) return DS_ERR_ARG;
  if (n_tok > 0 && !K) return DS_ERR_ARG;
  if (n_win > 0) {
    if (!qwin) return DS_ERR_ARG;
    if (kv->n_q_heads < 1 || kv->n_q_heads % kv->n_kv_heads) return DS_ERR_SHAPE;
    if (kv->d_q < 1 || kv->d_q > 256) return DS_ERR_SHAPE;
    if (!keep && kv->d_k > kv->d_q) return DS_ERR_SHAPE;
  }
  if (K && !aligned16(K)) return DS_ERR_ALIGN;
  const int G = n_win > 0 ? kv->n_q_heads / kv->n_kv_heads : 1;
  if ((int64_t)n_win * G > INT32_MAX / 2) return DS_ERR_SHAPE;
  const CalibPlan pl = calib_plan(kv->batch, kv->n_kv_heads, n_tok, kv->d_k, n_win * G);
  if (pl.ws_bytes > 0 && (!workspace || workspace_bytes < pl.ws_bytes)) return DS_ERR_WORKSPACE;
  if (pl.blocks > INT32_MAX) return DS_ERR_SHAPE;
  CalibArgs a{};
  a.K = static_cast<const __half*>(K);
  a.ks0 = kv->k_stride[0];
  a.ks1 = kv->k_stride[1];
  a.ks2 = kv->k_stride[2];
  a.B = kv->batch;
  a.Hkv = kv->n_kv_heads;
  a.d_k = kv->d_k;
  a.n_tok = n_tok;
  a.n_cpr = pl.n_cpr;
  a.chunk = pl.chunk;
  a.part = static_cast<float*>(workspace);
  a.qpart = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.qpart_off);
  a.n_qch = pl.n_qch;
  a.q_blocks = (int)pl.q_blocks;
  a.q = static_cast<const __half*>(qwin);
  a.n_win = n_win;
  a.Hq = n_win > 0 ? kv->n_q_heads : kv->n_kv_heads;
  a.d_q = n_win > 0 ? kv->d_q : kv->d_k;
  a.keep = keep;
  a.criterion = criterion;
  a.r = r;
  a.chan = chan;
  a.norms = norms;
  return launch_calib(a, pl.blocks, stream) == hipSuccess ? DS_OK : DS_ERR_HIP;
}

}  // extern "C"
