// ds_internal.h -- shared declarations of the HIP implementation behind ds.h.
//
// Pages cited by title and section:
//   [DS]    "Double Sparsity" article, joto.ai blog archive 2025060420469,
//           sections "offline calibration" and "online forward computation".
//   [LeanK] LeanK article, aitangshan.cn news 1293675, section 2.2.
//   [GQA]   grouped-query attention article, trdm.cn news 80600, section 4.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ds.h"

namespace ds {

// The fully fused decode kernel (append + score + select + attention in one
// 256-thread workgroup per row) keeps up to TPT scores per thread in
// registers and the selected token list in LDS.
constexpr int kDecodeFusedTPT = 24;  // rows up to 6144 tokens
constexpr int kDecodeFusedMaxK = 2048;
// Local top-M select: chunk workgroups keep a superset of their share of the
// top k (at most kMergeCap candidates per row in all), then one workgroup per
// row selects exactly among the candidates.
constexpr int kMergeCap = 16384;
constexpr int kMaxLocalChunks = 256;
constexpr int kMaxLocalChunk = 10240;  // tokens per local-select chunk at most (512 threads x 20)
// Attention splits per row are capped; partial results cost 528 B each.
constexpr int kMaxSplit = 64;
// Selected-token indices staged in LDS per attention workgroup.
constexpr int kMaxTokensPerSplit = 2048;
// Partial-result record: o[128] fp32, then m (log2 domain), l; padded to 16 B.
constexpr int kDv = 128;
constexpr int kPartStride = kDv + 4;
// Query heads per KV head handled by the attention kernel.
constexpr int kMaxGroup = 8;

// ---------------------------------------------------------------------------
// Launch arguments (plain structs passed by value to the kernels).
// ---------------------------------------------------------------------------
struct LabelArgs {
  const __half* K;
  int64_t ks0, ks1, ks2;
  int32_t Hkv, d_k, cap;
  const int32_t* chan;
  int32_t r, is_int4, slots;
  __half* lab16;
  uint8_t* codes;
  __half* scales;
  // build: tile -> (row, 64 consecutive tokens of [t_begin, t_end))
  int32_t t_begin, t_end, tiles_per_row;
  // append (pos != nullptr): item -> (row, pos[b]); n_items = B * Hkv
  const int32_t* pos;
  int32_t n_items;
  // append driven by seq_lens (pos = seq_lens, token = seq_lens[b] - 1)
  int32_t pos_minus_one;
  // paged K pool (ptab != nullptr): ks0 is the page stride
  const int32_t* ptab;
  int32_t pshift, max_pages;
  const ds_head_layout* heads;  // per-head K layout, or null
};

struct ScoreArgs {
  const __half* q;
  int32_t Hq, d_q, Hkv, G, d_k;
  const int32_t* keep;  // [Hkv][d_k] or null
  const int32_t* chan;  // [Hkv][r]
  int32_t r, is_int4, slots;
  const __half* lab16;
  const uint8_t* codes;
  const __half* scales;
  const int32_t* seq_lens;
  int32_t max_seq;
  int32_t k;
  // outputs
  int32_t* idx;         // [rows][idx_stride]
  int32_t idx_stride;
  int32_t pad_idx;      // write -1 after the selection up to idx_stride
  int32_t* count;       // [rows]
  uint32_t* keys;       // [rows][keys_stride] (chunked path)
  int32_t keys_stride;
  int32_t chunk;        // tokens per score workgroup (chunked path)
  int32_t n_chunks;
  // local top-M path: per row kMergeCap candidate slots, chunk c owns
  // [c * cap_row, (c + 1) * cap_row) with cap_row = kMergeCap / chunks_of_row
  float* cand_score;    // [rows][kMergeCap]: kept scores
  int32_t* cand_idx;    // [rows][kMergeCap]
  int32_t* cand_cnt;    // [rows][n_chunks], -1: overflow
  uint32_t* cand_theta; // [rows][n_chunks], key of the chunk's threshold (0: kept whole)
  float2* cand_range;   // [rows][n_chunks], (lowest kept score bound, largest score)
  int32_t cand_stride;  // candidate slots per row (<= kMergeCap)
  int32_t half_quota;   // every chunk's quota is at least 512 (sampled threshold)
  const ds_head_layout* heads;  // per-head K layout (fully pruned heads), or null
  int32_t keep_ld;              // row stride of the keep table (the widest d_k)
};

struct AttnArgs {
  const __half* q;
  int32_t Hq, d_q;
  const __half* K;
  const __half* V;
  int64_t ks0, ks1, ks2, vs0, vs1, vs2;
  int32_t Hkv, d_k;
  const int32_t* keep;
  const int32_t* seq_lens;
  int32_t max_seq;
  int32_t sparse;
  const int32_t* idx;
  int32_t idx_stride;
  const int32_t* count;
  int32_t n_split, tps;
  float scale_log2;
  __half* out;
  float* part;
  // paged K/V pool (ptab != nullptr): ks0 / vs0 are page strides, and the
  // kernels address tokens by physical id (page << pshift | slot)
  const int32_t* ptab;
  int32_t pshift, pmask, max_pages;
  const ds_head_layout* heads;  // per-head K/V layout, or null
  int32_t keep_ld;              // row stride of the keep table (the widest d_k)
};

// The arguments as seen by one KV head g: with a per-head layout, K and V
// point at the head's blocks, the head stride is 0 and K's token stride and
// width are the head's kept count (0: a fully pruned head).
__device__ __forceinline__ AttnArgs with_head(AttnArgs a, int g) {
  if (a.heads) {
    const ds_head_layout h = a.heads[g];
    a.K += h.k_off;
    a.V += h.v_off;
    a.ks1 = 0;
    a.vs1 = 0;
    a.ks2 = h.k_cols;
    a.d_k = (int32_t)h.k_cols;
  }
  return a;
}
__device__ __forceinline__ LabelArgs with_head(LabelArgs a, int g) {
  if (a.heads) {
    const ds_head_layout h = a.heads[g];
    a.K += h.k_off;
    a.ks1 = 0;
    a.ks2 = h.k_cols;
    a.d_k = (int32_t)h.k_cols;
  }
  return a;
}
// Kept K columns of head g (d_k without a per-head layout).
__device__ __forceinline__ int head_cols(const ds_head_layout* heads, int g, int d_k) {
  return heads ? (int)heads[g].k_cols : d_k;
}

// Optional timing events recorded by a launch itself, at the kernel's start
// and end (both or neither).
struct KEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

template <typename F, typename... Args>
inline hipError_t launch_k(F kernel, dim3 grid, dim3 block, hipStream_t s, const KEvents& ev,
                           Args... args) {
  if (ev.start && ev.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev.start, ev.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  return hipGetLastError();
}

// Heavy-channel calibration ([DS] "offline calibration"; [LeanK] section 1.1).
constexpr int kMaxDk = 128;  // stored K columns at most
constexpr int kQRows = 32;   // window-query rows per calibration workgroup
struct CalibArgs {
  const __half* K;
  int64_t ks0, ks1, ks2;
  int B, Hkv, d_k, n_tok;
  int n_cpr, chunk;  // token chunks per (KV head, sample) and tokens per chunk
  float* part;       // [Hkv][B][n_cpr][d_k] column sums of squares per chunk
  float* qpart;      // [Hkv][B][n_qch][d_k] the same over window-query rows
  int n_qch, q_blocks;
  const __half* q;   // [B][n_win][Hq][d_q] window queries
  int n_win, Hq, d_q;
  const int32_t* keep;  // [Hkv][d_k] or null
  int criterion, r;
  int32_t* chan;  // [Hkv][r]
  float* norms;   // [Hkv][3][d_k] or null
};
struct CalibPlan {
  int n_cpr = 0, chunk = 0, n_qch = 0;
  int64_t blocks = 0, q_blocks = 0;  // all workgroups; the window-query ones first
  size_t part_bytes = 0, qpart_off = 0, ws_bytes = 0;
};
CalibPlan calib_plan(int B, int Hkv, int n_tok, int d_k, int n_qrows);

// Launchers (return the launch status of the last kernel they enqueue).
hipError_t launch_label(const LabelArgs& a, int n_blocks, hipStream_t s,
                        const KEvents& ev = KEvents());
hipError_t launch_calib(const CalibArgs& a, int64_t blocks, hipStream_t s);
hipError_t launch_score_chunks(const ScoreArgs& a, int rows, hipStream_t s,
                               const KEvents& ev = KEvents());
hipError_t launch_select_stream(const ScoreArgs& a, int rows, hipStream_t s,
                                const KEvents& ev = KEvents());
hipError_t launch_attn(const AttnArgs& a, int rows, int G, bool final_out, hipStream_t s,
                       const KEvents& ev = KEvents());
hipError_t launch_attn_gqa(const AttnArgs& a, int rows, int G, bool final_out, hipStream_t s,
                           const KEvents& ev = KEvents());
hipError_t launch_combine(const AttnArgs& a, int B, hipStream_t s, const KEvents& ev = KEvents());
hipError_t launch_decode_fused(const ScoreArgs& sa, const AttnArgs& aa, const LabelArgs& la,
                               int append, int rows, hipStream_t s, const KEvents& ev = KEvents());
bool decode_fused_fits(int max_seq, int k, int r, int is_int4);
hipError_t launch_decode_fused_g(const ScoreArgs& sa, const AttnArgs& aa, const LabelArgs& la,
                                 int append, int rows, hipStream_t s,
                                 const KEvents& ev = KEvents());
bool decode_fused_g_fits(int max_seq, int k, int r, int is_int4, int G);
hipError_t launch_score_local(const ScoreArgs& sa, const LabelArgs& la, int append, int rows,
                              hipStream_t s, const KEvents& ev = KEvents());
hipError_t launch_select_merge(const ScoreArgs& sa, int rows, hipStream_t s,
                               const KEvents& ev = KEvents());

// ---------------------------------------------------------------------------
// Device helpers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float h2f(__half h) { return __half2float(h); }

// 16-byte load with the nontemporal hint: data read once per step (K/V rows,
// labels) streams through the caches instead of displacing reused lines.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void unpack8(const uint4 v, float* f) {
  const __half2* h = reinterpret_cast<const __half2*>(&v);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float2 x = __half22float2(h[i]);
    f[2 * i] = x.x;
    f[2 * i + 1] = x.y;
  }
}

// K rows of the label kernels: token t of batch row b at b * s0 + t * s2
// (contiguous rows, ptab == nullptr) or, in a paged pool, at page * s0 +
// (t mod 2^pshift) * s2 with page = ptab[b][t >> pshift].
__device__ __forceinline__ int64_t kv_off(const int32_t* ptab, int pshift, int max_pages, int b,
                                          int64_t t, int64_t s0, int64_t s2) {
  if (!ptab) return (int64_t)b * s0 + t * s2;
  const int64_t pg = ptab[(int64_t)b * max_pages + (t >> pshift)];
  return pg * s0 + (t & ((int64_t(1) << pshift) - 1)) * s2;
}

// Physical id (page << pshift | slot) of token t of batch row b in a paged
// pool, from a page table (global memory or a row's slice staged in LDS
// with first = the batch row's entry 0).
__device__ __forceinline__ int32_t phys_tok(const int32_t* row_tab, int pshift, int t) {
  return (row_tab[t >> pshift] << pshift) | (t & ((1 << pshift) - 1));
}

// Order-preserving map from fp32 to uint32 (larger value -> larger key);
// -0 is folded onto +0 first.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

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

// Exclusive prefix sum of one uint32 per thread over a workgroup of NT
// threads; `tmp` holds NT/64 words of LDS.  Contains two barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    uint32_t t = tmp[i];
    before += (i < w) ? t : 0u;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

// Cross-row lane exchange without LDS (v_permlane16_swap / v_permlane32_swap):
// for lanes l and l ^ 16 (resp. l ^ 32) both get the pair (value of the
// lower lane, value of the upper lane), so a combination of the two is the
// same, bit for bit, in both lanes.
struct LanePair {
  float lo, hi;
};
__device__ __forceinline__ LanePair xchg16(float x) {
  const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return {__uint_as_float(t[0]), __uint_as_float(t[1])};
}
__device__ __forceinline__ LanePair xchg32(float x) {
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return {__uint_as_float(t[0]), __uint_as_float(t[1])};
}

// Butterfly within each row of 16 lanes (swap neighbours, swap pairs,
// mirror within 8, mirror within 16), then across rows: every lane gets
// op over the whole wave.  op must be commutative and associative.
template <typename Op>
__device__ __forceinline__ float wave_reduce(float x, Op op) {
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false)));
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false)));
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false)));
  x = op(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false)));
  LanePair p = xchg16(x);
  x = op(p.lo, p.hi);
  p = xchg32(x);
  return op(p.lo, p.hi);
}
__device__ __forceinline__ float wave_max(float x) {
  return wave_reduce(x, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_min(float x) {
  return wave_reduce(x, [](float a, float b) { return fminf(a, b); });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  return __float_as_uint(wave_reduce(__uint_as_float(x), [](float a, float b) {
    return __uint_as_float(min(__float_as_uint(a), __float_as_uint(b)));
  }));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  return __float_as_uint(wave_reduce(__uint_as_float(x), [](float a, float b) {
    return __uint_as_float(max(__float_as_uint(a), __float_as_uint(b)));
  }));
}

// Sum over the 16 lanes of a row (lanes 16i .. 16i+15) with DPP moves:
// swap neighbours, swap pairs, mirror within 8, mirror within 16.
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false));
  return x;
}

}  // namespace ds
