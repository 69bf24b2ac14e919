// calib.hip -- heavy-channel calibration ([DS] "offline calibration": the
// channels that move the attention scores most are chosen once, from a few
// sample tokens, by a K-, Q- or QK-outlier criterion; [LeanK] section 1.1:
// a channel's importance is the L2 norm of the product of the observation
// window's query column and the key column).
//
// k_calib_cols: one workgroup per (KV head, sample, chunk of tokens) adds up
//   the squares of every stored K column over its tokens (16-byte row
//   pieces, four in flight per thread) and writes one fp32 partial per
//   column; the grid's first workgroups do the same for rows of the window
//   queries, so those loads overlap the K stream.  Summation order is fixed,
//   so results repeat bit for bit.
// k_calib_select: one workgroup per KV head, eight lanes per column, adds
//   the partials and the window queries' squares at each column's query
//   channel (each lane a fixed share, then the lanes in order), forms the
//   criterion's score and ranks the columns (score descending, column
//   ascending); the r best go out in ascending column order.
#include <algorithm>

#include "ds_internal.h"

namespace ds {
namespace {

constexpr int kCalNT = 256;
static_assert(kCalNT == 2 * kMaxDk, "window-query workgroups: two threads per column");

// Window-query workgroups (the first q_blocks of the grid): one per (KV
// head, sample, kQRows rows of (window query, head)); thread (c, l) adds the
// squares of rows l, l + 2, ... at column c's query channel.
__device__ __forceinline__ void calib_qrows(const CalibArgs& a, int blk, float* red) {
  const int qch = blk % a.n_qch;
  const int gb = blk / a.n_qch;  // g * B + b
  const int g = gb / a.B;
  const int b = gb - g * a.B;
  const int G = a.Hq / a.Hkv;
  const int c = threadIdx.x % kMaxDk;
  const int l = threadIdx.x / kMaxDk;  // 0 or 1
  const int i0 = qch * kQRows;
  const int i1 = min(a.n_win * G, i0 + kQRows);
  float acc = 0.0f;
  if (c < a.d_k) {
    const int qc = a.keep ? a.keep[(int64_t)g * a.d_k + c] : c;
    const __half* qb = a.q + ((int64_t)b * a.n_win * a.Hq + (int64_t)g * G) * a.d_q + qc;
#pragma unroll
    for (int u = 0; u < kQRows / 2; ++u) {
      const int i = i0 + l + 2 * u;
      if (i < i1) {
        const int w = i / G, h = i - w * G;
        const float x = __half2float(qb[((int64_t)w * a.Hq + h) * a.d_q]);
        acc = fmaf(x, x, acc);
      }
    }
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  if (l == 0 && c < a.d_k) a.qpart[(int64_t)blk * a.d_k + c] = red[c] + red[kMaxDk + c];
}

__global__ __launch_bounds__(kCalNT) void k_calib_cols(CalibArgs a) {
  __shared__ float red[kCalNT * 8];
  if ((int)blockIdx.x < a.q_blocks) {
    calib_qrows(a, blockIdx.x, red);
    return;
  }
  const int blk = blockIdx.x - a.q_blocks;
  const int ch = blk % a.n_cpr;
  const int gb = blk / a.n_cpr;  // g * B + b
  const int g = gb / a.B;
  const int b = gb - g * a.B;
  const int cg_n = a.d_k >> 3;      // 8-column pieces per token row
  const int tl_n = kCalNT / cg_n;   // token rows per pass
  const int tid = threadIdx.x;
  const int cg = tid % cg_n;
  const int tl = tid / cg_n;
  const int t0 = ch * a.chunk;
  const int t1 = min(a.n_tok, t0 + a.chunk);
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  auto add = [&](const uint4& x) {
    const __half2* h = reinterpret_cast<const __half2*>(&x);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float2 f = __half22float2(h[i]);
      acc[2 * i] = fmaf(f.x, f.x, acc[2 * i]);
      acc[2 * i + 1] = fmaf(f.y, f.y, acc[2 * i + 1]);
    }
  };
  if (tl < tl_n) {
    const __half* base = a.K + (int64_t)b * a.ks0 + (int64_t)g * a.ks1 + 8 * cg;
    int t = t0 + tl;
    for (; t + 3 * tl_n < t1; t += 4 * tl_n) {
      uint4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = ld_stream(base + (int64_t)(t + u * tl_n) * a.ks2);
#pragma unroll
      for (int u = 0; u < 4; ++u) add(x[u]);
    }
    for (; t < t1; t += tl_n) add(ld_stream(base + (int64_t)t * a.ks2));
#pragma unroll
    for (int i = 0; i < 8; ++i) red[tl * a.d_k + 8 * cg + i] = acc[i];
  }
  __syncthreads();
  for (int c = tid; c < a.d_k; c += kCalNT) {
    float s = 0.0f;
    for (int l = 0; l < tl_n; ++l) s += red[l * a.d_k + c];
    a.part[(int64_t)blk * a.d_k + c] = s;
  }
}

constexpr int kSelNT = 1024;                // 8 lanes per column
constexpr int kSelLanes = kSelNT / kMaxDk;  // lanes j that share column c

constexpr int kSelB = 4;                    // samples per round (loads in flight together)

__global__ __launch_bounds__(kSelNT) void k_calib_select(CalibArgs a) {
  __shared__ float red_k[kSelB][kSelLanes][kMaxDk];
  __shared__ float red_q[kSelB][kSelLanes][kMaxDk];
  __shared__ float sc[kMaxDk];
  __shared__ int32_t red_r[kSelLanes][kMaxDk];
  __shared__ int32_t wave_cnt[2];
  const int g = blockIdx.x;
  const int c = threadIdx.x % kMaxDk;
  const int j = threadIdx.x / kMaxDk;
  const bool col = c < a.d_k;
  float kn = 0.0f, qn = 0.0f, qk = 0.0f;
  for (int b0 = 0; b0 < a.B; b0 += kSelB) {
    // lane j adds, for each of up to four samples, the K and query partials
    // whose index is j modulo 8, in order
    float kp[kSelB], qp[kSelB];
#pragma unroll
    for (int bb = 0; bb < kSelB; ++bb) {
      kp[bb] = 0.0f;
      qp[bb] = 0.0f;
      const int b = b0 + bb;
      if (!col || b >= a.B) continue;
      const float* pp = a.part + ((int64_t)(g * a.B + b) * a.n_cpr) * a.d_k + c;
#pragma unroll 4
      for (int ch = j; ch < a.n_cpr; ch += kSelLanes) kp[bb] += pp[(int64_t)ch * a.d_k];
      const float* qq = a.qpart + ((int64_t)(g * a.B + b) * a.n_qch) * a.d_k + c;
#pragma unroll 4
      for (int i = j; i < a.n_qch; i += kSelLanes) qp[bb] += qq[(int64_t)i * a.d_k];
    }
#pragma unroll
    for (int bb = 0; bb < kSelB; ++bb) {
      red_k[bb][j][c] = kp[bb];
      red_q[bb][j][c] = qp[bb];
    }
    __syncthreads();
    if (j == 0) {
      for (int bb = 0; bb < kSelB && b0 + bb < a.B; ++bb) {
        float knb = 0.0f, qnb = 0.0f;
#pragma unroll
        for (int l = 0; l < kSelLanes; ++l) {
          knb += red_k[bb][l][c];
          qnb += red_q[bb][l][c];
        }
        kn += knb;
        qn += qnb;
        qk = fmaf(qnb, knb, qk);
      }
    }
    __syncthreads();
  }
  float score = 0.0f;
  if (j == 0 && col) {
    score = a.criterion == 0 ? kn : a.criterion == 1 ? qn : sqrtf(qk);
    if (!(score >= 0.0f)) score = -1.0f;  // NaN ranks last, so the order stays total
    sc[c] = score;
  }
  __syncthreads();
  // rank under (score descending, column ascending), a permutation of
  // 0 .. d_k - 1, so exactly r columns have rank < r: lane j counts the
  // columns i = j modulo 8 that come first
  int part = 0;
  if (col) {
    const float me = sc[c];
    for (int i = j; i < a.d_k; i += kSelLanes) {
      const float s = sc[i];
      part += (s > me || (s == me && i < c)) ? 1 : 0;
    }
  }
  red_r[j][c] = part;
  __syncthreads();
  const bool mine = j == 0 && col;
  bool sel = false;
  if (mine) {
    int rank = 0;
#pragma unroll
    for (int l = 0; l < kSelLanes; ++l) rank += red_r[l][c];
    sel = rank < a.r;
  }
  // output position: selected columns before c (columns 0..63 are wave 0)
  const uint64_t m = __ballot(sel);
  const int lane = threadIdx.x & 63;
  if (j == 0 && lane == 0) wave_cnt[threadIdx.x >> 6] = __popcll(m);
  __syncthreads();
  if (sel) {
    const int pos = __popcll(m & ((1ull << lane) - 1ull)) + (threadIdx.x >= 64 ? wave_cnt[0] : 0);
    a.chan[(int64_t)g * a.r + pos] = c;
  }
  if (a.norms && mine) {
    float* nd = a.norms + (int64_t)g * 3 * a.d_k;
    nd[c] = kn;
    nd[a.d_k + c] = qn;
    nd[2 * a.d_k + c] = score;
  }
}

}  // namespace

CalibPlan calib_plan(int B, int Hkv, int n_tok, int d_k, int n_qrows) {
  CalibPlan p;
  const int64_t rows = (int64_t)B * Hkv;
  p.n_qch = (n_qrows + kQRows - 1) / kQRows;
  if (n_tok > 0) {
    // about 2048 workgroups over the chip, chunks of at least 256 tokens
    const int64_t want = std::max<int64_t>(1, (2048 + rows - 1) / rows);
    const int64_t most = (n_tok + 255) / 256;
    const int64_t n = std::min(want, most);
    p.chunk = (int)((n_tok + n - 1) / n);
    p.n_cpr = (n_tok + p.chunk - 1) / p.chunk;
  }
  p.part_bytes = (size_t)rows * p.n_cpr * d_k * sizeof(float);
  p.qpart_off = (p.part_bytes + 255) / 256 * 256;
  p.ws_bytes = p.qpart_off + (size_t)rows * p.n_qch * d_k * sizeof(float);
  p.q_blocks = rows * p.n_qch;
  p.blocks = p.q_blocks + rows * p.n_cpr;
  return p;
}

hipError_t launch_calib(const CalibArgs& a, int64_t blocks, hipStream_t s) {
  if (blocks > 0) {
    hipLaunchKernelGGL(k_calib_cols, dim3((unsigned)blocks), dim3(kCalNT), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_calib_select, dim3(a.Hkv), dim3(kSelNT), 0, s, a);
  return hipGetLastError();
}

}  // namespace ds
