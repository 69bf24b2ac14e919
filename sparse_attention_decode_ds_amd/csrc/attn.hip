// attn.hip -- standalone attention pass (step 3b, [DS] "online forward
// computation") over a token list produced by the select kernels (or every
// token on the dense path), split over several workgroups per row, and the
// log-sum-exp merge of the split partial results.
#include "attn_common.h"

namespace ds {
namespace {

template <int G, bool FINAL>
__global__ __launch_bounds__(kAttnThreads) void k_attn(AttnArgs a) {
  __shared__ int32_t lidx[kMaxTokensPerSplit];
  __shared__ AttnRed<G> red;

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
  const int c = lane & 15;
  const int slot = (tid >> 6) * 4 + (lane >> 4);
  const bool kl = c < (a.d_k >> 3);

  float qf[G][8];
  load_query<G>(a, b, g, c, kl, qf);
  AttnAcc<G> acc;
  acc_init<G>(acc);
  const __half* Kr = a.K + (int64_t)b * a.ks0 + (int64_t)g * a.ks1 + min(c, (a.d_k >> 3) - 1) * 8;
  const __half* Vr = a.V + (int64_t)b * a.vs0 + (int64_t)g * a.vs1 + c * 8;

  if (a.sparse) {
    for (int bat = 0; bat < n_here; bat += kMaxTokensPerSplit) {
      const int nb = min(kMaxTokensPerSplit, n_here - bat);
      __syncthreads();
      const int32_t* src = a.idx + (int64_t)row * a.idx_stride + t0 + bat;
      for (int i = tid; i < nb; i += kAttnThreads) lidx[i] = src[i];
      __syncthreads();
      attend<G>(a, Kr, Vr, slot, nb, [&](int i) { return (int64_t)lidx[i]; }, qf, acc);
    }
  } else {
    attend<G>(a, Kr, Vr, slot, n_here, [&](int i) { return (int64_t)(t0 + i); }, qf, acc);
  }
  attn_finish<G, FINAL>(a, acc, red, b, g, split);
}

// Log-sum-exp merge of the split partials: 16 lanes per (batch, query head).
__global__ __launch_bounds__(kAttnThreads) void k_combine(AttnArgs a, int n_rows) {
  const int rq = blockIdx.x * (kAttnThreads / 16) + (threadIdx.x >> 4);
  if (rq >= n_rows) return;
  merge_partials(a, rq, threadIdx.x & 15);
}

template <int G>
hipError_t launch_g(const AttnArgs& a, int rows, bool final_out, hipStream_t s, const KEvents& ev) {
  const dim3 grid(rows * a.n_split);
  if (final_out) return launch_k(k_attn<G, true>, grid, dim3(kAttnThreads), s, ev, a);
  return launch_k(k_attn<G, false>, grid, dim3(kAttnThreads), s, ev, a);
}

}  // namespace

// Single-head groups stream rows through the vector units; groups of 2 to 8
// query heads take the matrix-core kernel (attn_gqa.hip).
hipError_t launch_attn(const AttnArgs& a, int rows, int G, bool final_out, hipStream_t s,
                       const KEvents& ev) {
  if (rows <= 0) return hipSuccess;
  if (G == 1) return launch_g<1>(a, rows, final_out, s, ev);
  return launch_attn_gqa(a, rows, G, final_out, s, ev);
}

hipError_t launch_combine(const AttnArgs& a, int B, hipStream_t s) {
  const int n_rows = B * a.Hq;
  if (n_rows <= 0) return hipSuccess;
  const int per = kAttnThreads / 16;
  hipLaunchKernelGGL(k_combine, dim3((n_rows + per - 1) / per), dim3(kAttnThreads), 0, s, a, n_rows);
  return hipGetLastError();
}

}  // namespace ds
