// attn.hip -- step 3b of a Double Sparsity decode step: exact softmax
// attention over the selected tokens' full K/V rows, and the merge of
// split partial results.
//
// [DS] "online forward computation", step 3: attention over the top-k tokens
// uses the full query, K and V (not the channel-sparse ones), which is why the
// whole K/V cache is kept.  [GQA] section 4: the G query heads of a group read
// the same K/V rows, so a workgroup loads each selected row once and applies
// it to all G heads.  [LeanK] section 2.2: K may be stored compacted to d_k
// kept columns; the query is read at those channels (keep table).
//
// Work layout: a workgroup (4 waves) takes one (batch, KV head) row and one
// contiguous range of its selected tokens (a "split").  A wave is four rows
// of 16 lanes; each 16-lane row walks its own tokens, lane c holding K and V
// channels [8c, 8c+8) as one 16-byte load each, and keeps its own online
// softmax state (running max m in the log2 domain, sum l, output o) per head.
// The 16 states are merged through shuffles and LDS at the end.  With one
// split the workgroup writes the fp16 output; otherwise it writes (o, m, l)
// partials that k_combine merges with log-sum-exp weights.
#include "ds_internal.h"

namespace ds {
namespace {

constexpr int kThreads = 256;
constexpr int kSlots = 16;   // 16-lane rows per workgroup
constexpr int kUnroll = 4;   // tokens in flight per 16-lane row
constexpr float kNegInf = -__builtin_huge_valf();

// Merge state (m2, l2, o2) into (m, l, o); either may be empty (m = -inf).
__device__ __forceinline__ void merge_weights(float m, float m2, float& w1, float& w2, float& mx) {
  mx = fmaxf(m, m2);
  w1 = (m == kNegInf) ? 0.0f : exp2f(m - mx);
  w2 = (m2 == kNegInf) ? 0.0f : exp2f(m2 - mx);
}

template <int G, bool FINAL>
__global__ __launch_bounds__(kThreads) void k_attn(AttnArgs a) {
  __shared__ int32_t lidx[kMaxTokensPerSplit];
  __shared__ float red[4][G][kDv + 2];

  const int row = blockIdx.x / a.n_split;
  const int split = blockIdx.x - row * a.n_split;
  const int b = row / a.Hkv;
  const int g = row - b * a.Hkv;
  const int S = min(max(a.seq_lens[b], 0), a.max_seq);
  const int n_tok = a.sparse ? min(a.count[row], S) : S;
  const int t0 = split * a.tps;
  const int n_here = max(0, min(n_tok - t0, a.tps));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int c = lane & 15;
  const int slot = w * 4 + (lane >> 4);
  const bool kl = c < (a.d_k >> 3);

  // Query of each head at channels [8c, 8c+8) of the stored K, scaled so that
  // exp2 of the dot product is exp of the logit.
  float qf[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const __half* qh = a.q + ((int64_t)b * a.Hq + (int64_t)g * G + h) * a.d_q;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v = 0.0f;
      if (kl) {
        const int ch = c * 8 + i;
        const int qc = a.keep ? a.keep[(int64_t)g * a.d_k + ch] : ch;
        v = h2f(qh[qc]) * a.scale_log2;
      }
      qf[h][i] = v;
    }
  }

  float o[G][8], m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[h][i] = 0.0f;
  }

  const __half* Kr = a.K + (int64_t)b * a.ks0 + (int64_t)g * a.ks1 + c * 8;
  const __half* Vr = a.V + (int64_t)b * a.vs0 + (int64_t)g * a.vs1 + c * 8;

  for (int bat = 0; bat < n_here; bat += kMaxTokensPerSplit) {
    const int nb = min(kMaxTokensPerSplit, n_here - bat);
    if (a.sparse) {
      __syncthreads();
      const int32_t* src = a.idx + (int64_t)row * a.idx_stride + t0 + bat;
      for (int i = tid; i < nb; i += kThreads) lidx[i] = src[i];
      __syncthreads();
    }
    for (int base = slot; base < nb; base += kSlots * kUnroll) {
      uint4 kr[kUnroll], vr[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
        const int i = base + u * kSlots;
        if (i < nb) {
          const int64_t t = a.sparse ? lidx[i] : (int64_t)(t0 + bat + i);
          if (kl) kr[u] = *reinterpret_cast<const uint4*>(Kr + t * a.ks2);
          vr[u] = *reinterpret_cast<const uint4*>(Vr + t * a.vs2);
        }
      }
      float s[kUnroll][G];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        float kf[8];
        unpack8(kr[u], kf);
        const bool valid = base + u * kSlots < nb;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float d = 0.0f;
#pragma unroll
          for (int i = 0; i < 8; ++i) d += qf[h][i] * kf[i];
          d = row16_sum(d);
          s[u][h] = valid ? d : kNegInf;
        }
      }
      float vf[kUnroll][8];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) unpack8(vr[u], vf[u]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float mx = m[h];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) mx = fmaxf(mx, s[u][h]);
        if (mx == kNegInf) continue;
        const float alpha = exp2f(m[h] - mx);
        float p[kUnroll];
        float ps = 0.0f;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          p[u] = exp2f(s[u][h] - mx);
          ps += p[u];
        }
        l[h] = l[h] * alpha + ps;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float acc = o[h][i] * alpha;
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) acc += p[u] * vf[u][i];
          o[h][i] = acc;
        }
        m[h] = mx;
      }
    }
  }

  // Merge the four 16-lane rows of each wave.
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float m2 = __shfl_xor(m[h], off, 64);
      const float l2 = __shfl_xor(l[h], off, 64);
      float w1, w2, mx;
      merge_weights(m[h], m2, w1, w2, mx);
      l[h] = l[h] * w1 + l2 * w2;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[h][i] = o[h][i] * w1 + __shfl_xor(o[h][i], off, 64) * w2;
      m[h] = mx;
    }
  }
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int i = 0; i < 8; ++i) red[w][h][c * 8 + i] = o[h][i];
      if (c == 0) {
        red[w][h][kDv] = m[h];
        red[w][h][kDv + 1] = l[h];
      }
    }
  }
  __syncthreads();

  // Merge the four waves: thread (h, c) for h < G.
  if (tid >= G * 16) return;
  const int h = tid >> 4;
  const int cc = tid & 15;
  float M = kNegInf;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, red[ww][h][kDv]);
  float L = 0.0f, O[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) O[i] = 0.0f;
  if (M != kNegInf) {
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float mw = red[ww][h][kDv];
      if (mw == kNegInf) continue;
      const float sc = exp2f(mw - M);
      L += sc * red[ww][h][kDv + 1];
#pragma unroll
      for (int i = 0; i < 8; ++i) O[i] += sc * red[ww][h][cc * 8 + i];
    }
  }
  const int64_t bh = (int64_t)b * a.Hq + (int64_t)g * G + h;
  if (FINAL) {
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    __half2 r2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) r2[i] = __floats2half2_rn(O[2 * i] * inv, O[2 * i + 1] * inv);
    *reinterpret_cast<uint4*>(a.out + bh * kDv + cc * 8) = *reinterpret_cast<const uint4*>(r2);
  } else {
    float* dst = a.part + (bh * a.n_split + split) * kPartStride;
    *reinterpret_cast<float4*>(dst + cc * 8) = make_float4(O[0], O[1], O[2], O[3]);
    *reinterpret_cast<float4*>(dst + cc * 8 + 4) = make_float4(O[4], O[5], O[6], O[7]);
    if (cc == 0) {
      dst[kDv] = M;
      dst[kDv + 1] = L;
    }
  }
}

// Log-sum-exp merge of the split partials: 16 lanes per (batch, query head).
__global__ __launch_bounds__(kThreads) void k_combine(AttnArgs a, int n_rows) {
  const int rq = blockIdx.x * (kThreads / 16) + (threadIdx.x >> 4);
  const int c = threadIdx.x & 15;
  if (rq >= n_rows) return;
  const float* p = a.part + (int64_t)rq * a.n_split * kPartStride;
  float M = kNegInf;
  for (int sp = 0; sp < a.n_split; ++sp) M = fmaxf(M, p[sp * kPartStride + kDv]);
  float L = 0.0f, O[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) O[i] = 0.0f;
  if (M != kNegInf) {
    for (int sp = 0; sp < a.n_split; ++sp) {
      const float* q = p + sp * kPartStride;
      const float ms = q[kDv];
      if (ms == kNegInf) continue;
      const float sc = exp2f(ms - M);
      L += sc * q[kDv + 1];
      const float4 x0 = *reinterpret_cast<const float4*>(q + c * 8);
      const float4 x1 = *reinterpret_cast<const float4*>(q + c * 8 + 4);
      O[0] += sc * x0.x;
      O[1] += sc * x0.y;
      O[2] += sc * x0.z;
      O[3] += sc * x0.w;
      O[4] += sc * x1.x;
      O[5] += sc * x1.y;
      O[6] += sc * x1.z;
      O[7] += sc * x1.w;
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  __half2 r2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) r2[i] = __floats2half2_rn(O[2 * i] * inv, O[2 * i + 1] * inv);
  *reinterpret_cast<uint4*>(a.out + (int64_t)rq * kDv + c * 8) = *reinterpret_cast<const uint4*>(r2);
}

template <int G>
hipError_t launch_g(const AttnArgs& a, int rows, bool final_out, hipStream_t s) {
  const dim3 grid(rows * a.n_split);
  if (final_out)
    hipLaunchKernelGGL((k_attn<G, true>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k_attn<G, false>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, int rows, int G, bool final_out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  switch (G) {
    case 1: return launch_g<1>(a, rows, final_out, s);
    case 2: return launch_g<2>(a, rows, final_out, s);
    case 3: return launch_g<3>(a, rows, final_out, s);
    case 4: return launch_g<4>(a, rows, final_out, s);
    case 5: return launch_g<5>(a, rows, final_out, s);
    case 6: return launch_g<6>(a, rows, final_out, s);
    case 7: return launch_g<7>(a, rows, final_out, s);
    case 8: return launch_g<8>(a, rows, final_out, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_combine(const AttnArgs& a, int B, hipStream_t s) {
  const int n_rows = B * a.Hq;
  if (n_rows <= 0) return hipSuccess;
  const int per = kThreads / 16;
  hipLaunchKernelGGL(k_combine, dim3((n_rows + per - 1) / per), dim3(kThreads), 0, s, a, n_rows);
  return hipGetLastError();
}

}  // namespace ds
