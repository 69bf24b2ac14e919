// calib.hip -- heavy-channel calibration ([DS] "offline calibration": the
// channels that move the attention scores most are chosen once, from a few
// sample tokens, by a K-, Q- or QK-outlier criterion; [LeanK] section 1.1:
// a channel's importance is the L2 norm of the product of the observation
// window's query column and the key column).
//
// k_calib_cols: one workgroup per (KV head, sample, chunk of tokens) adds up
//   the squares of every stored K column over its tokens (16-byte row
//   pieces, four in flight per thread) and writes one fp32 partial per
//   column.  Summation order is fixed, so results repeat bit for bit.
// k_calib_select: one workgroup per KV head adds the partials in order, the
//   window queries' squares at each column's query channel, forms the
//   criterion's score and ranks the columns (score descending, column
//   ascending); the r best go out in ascending column order.
#include <algorithm>

#include "ds_internal.h"

namespace ds {
namespace {

constexpr int kCalNT = 256;

__global__ __launch_bounds__(kCalNT) void k_calib_cols(CalibArgs a) {
  __shared__ float red[kCalNT * 8];
  const int blk = blockIdx.x;
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

__global__ __launch_bounds__(kMaxDk) void k_calib_select(CalibArgs a) {
  __shared__ float sc[kMaxDk];
  __shared__ int32_t picked[kMaxDk];
  const int g = blockIdx.x;
  const int c = threadIdx.x;
  float kn = 0.0f, qn = 0.0f, qk = 0.0f, score = 0.0f;
  if (c < a.d_k) {
    const int G = a.n_win > 0 ? a.Hq / a.Hkv : 1;
    const int qc = a.keep ? a.keep[(int64_t)g * a.d_k + c] : c;
    for (int b = 0; b < a.B; ++b) {
      float knb = 0.0f, qnb = 0.0f;
      const float* pp = a.part + ((int64_t)(g * a.B + b) * a.n_cpr) * a.d_k + c;
      for (int ch = 0; ch < a.n_cpr; ++ch) knb += pp[(int64_t)ch * a.d_k];
      for (int w = 0; w < a.n_win; ++w)
        for (int h = 0; h < G; ++h) {
          const float x = __half2float(
              a.q[(((int64_t)b * a.n_win + w) * a.Hq + (int64_t)g * G + h) * a.d_q + qc]);
          qnb = fmaf(x, x, qnb);
        }
      kn += knb;
      qn += qnb;
      qk = fmaf(qnb, knb, qk);
    }
    score = a.criterion == 0 ? kn : a.criterion == 1 ? qn : sqrtf(qk);
    if (!(score >= 0.0f)) score = -1.0f;  // NaN ranks last, so the order stays total
    sc[c] = score;
  }
  __syncthreads();
  // rank under (score descending, column ascending): a permutation of
  // 0 .. d_k - 1, so exactly r columns have rank < r
  int rank = 0;
  if (c < a.d_k)
    for (int j = 0; j < a.d_k; ++j) {
      const float s = sc[j];
      rank += (s > score || (s == score && j < c)) ? 1 : 0;
    }
  const bool sel = c < a.d_k && rank < a.r;
  picked[c] = sel ? 1 : 0;
  __syncthreads();
  if (sel) {
    int pos = 0;
    for (int j = 0; j < c; ++j) pos += picked[j];
    a.chan[(int64_t)g * a.r + pos] = c;
  }
  if (a.norms && c < a.d_k) {
    float* nd = a.norms + (int64_t)g * 3 * a.d_k;
    nd[c] = kn;
    nd[a.d_k + c] = qn;
    nd[2 * a.d_k + c] = score;
  }
}

}  // namespace

CalibPlan calib_plan(int B, int Hkv, int n_tok, int d_k) {
  CalibPlan p;
  const int64_t rows = (int64_t)B * Hkv;
  if (n_tok > 0) {
    // about 2048 workgroups over the chip, chunks of at least 256 tokens
    const int64_t want = std::max<int64_t>(1, (2048 + rows - 1) / rows);
    const int64_t most = (n_tok + 255) / 256;
    const int64_t n = std::min(want, most);
    p.chunk = (int)((n_tok + n - 1) / n);
    p.n_cpr = (n_tok + p.chunk - 1) / p.chunk;
  }
  p.part_bytes = (size_t)rows * p.n_cpr * d_k * sizeof(float);
  p.blocks = rows * p.n_cpr;
  return p;
}

hipError_t launch_calib(const CalibArgs& a, int64_t blocks, hipStream_t s) {
  if (blocks > 0) {
    hipLaunchKernelGGL(k_calib_cols, dim3((unsigned)blocks), dim3(kCalNT), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_calib_select, dim3(a.Hkv), dim3(kMaxDk), 0, s, a);
  return hipGetLastError();
}

}  // namespace ds
