// attn.hip -- standalone attention pass (step 3b, [DS] "online forward
// computation") over a token list produced by the select kernels (or every
// token on the dense path), split over several workgroups per row, and the
// log-sum-exp merge of the split partial results.
#include "attn_common.h"

namespace ds {
namespace {

// PAGED: K/V in a paged pool; the staged list holds physical token ids (the
// dense path stages its positions too).
template <int G, bool FINAL, bool PAGED>
__global__ __launch_bounds__(kAttnThreads) void k_attn(AttnArgs a_in) {
  __shared__ int32_t lidx[kMaxTokensPerSplit];
  __shared__ AttnRed<G> red;

  const SplitItem it = split_item(a_in, blockIdx.x);
  if (it.n == 0) return;  // every head pruned: the combine writes zeros
  const int b = it.b, g = it.g;
  const int row = b * a_in.Hkv + g;
  const AttnArgs a = with_head(a_in, g);
  const int tid = threadIdx.x;
  // With plain splits the first batch of the split's token list depends on
  // the kernel arguments only: its loads go out before the row's length and
  // count arrive (entries past the count are read but never used).
  constexpr int kPre = kMaxTokensPerSplit / kAttnThreads;
  const bool early = a.sparse && !split_by_bytes(a);
  int32_t pre[kPre];
  if (early) {
    const int te = it.split * a.tps;
    const int32_t* src = a.idx + (int64_t)row * a.idx_stride + te;
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int i = u * kAttnThreads + tid;
      pre[u] = (i < a.tps && te + i < a.idx_stride) ? src[i] : 0;
    }
  }
  const int S = min(max(a.seq_lens[b], 0), a.max_seq);
  // a fully pruned head (no K columns) attends nothing: zero output
  const int n_tok = a.d_k == 0 ? 0 : (a.sparse ? min(a.count[row], S) : S);
  const int tps = split_tokens(a, it, n_tok);
  const int t0 = it.split * tps;
  const int n_here = max(0, min(n_tok - t0, tps));

  const int lane = tid & 63;
  const int c = lane & 15;
  const int slot = (tid >> 6) * 4 + (lane >> 4);
  const bool kl = c < (a.d_k >> 3);

  float qf[G][8];
  load_query<G>(a, b, g, c, kl, qf);
  AttnAcc<G> acc;
  acc_init<G>(acc);
  const __half* Kr = a.K + (PAGED ? 0 : (int64_t)b * a.ks0) + (int64_t)g * a.ks1 +
                     min(c, (a.d_k >> 3) - 1) * 8;
  const __half* Vr = a.V + (PAGED ? 0 : (int64_t)b * a.vs0) + (int64_t)g * a.vs1 + c * 8;
  const int32_t* ptab = PAGED ? a.ptab + (int64_t)b * a.max_pages : nullptr;

  if (a.sparse || PAGED) {
    auto stage = [&](int bat, int nb) {
      const int32_t* src = a.idx + (int64_t)row * a.idx_stride + t0 + bat;
      for (int i = tid; i < nb; i += kAttnThreads) {
        const int t = a.sparse ? src[i] : t0 + bat + i;
        lidx[i] = PAGED ? phys_tok(ptab, a.pshift, t) : t;
      }
    };
    auto run = [&](int nb) {
      attend<G, PAGED>(a, Kr, Vr, slot, nb, [&](int i) { return (int64_t)lidx[i]; }, qf, acc);
    };
    // The first batch on its own, so that the prefetched entries are dead
    // before the attention loop (no registers held across it).
    if (n_here > 0) {
      const int nb = min(kMaxTokensPerSplit, n_here);
      if (early) {
#pragma unroll
        for (int u = 0; u < kPre; ++u) {
          const int i = u * kAttnThreads + tid;
          if (i < nb) lidx[i] = PAGED ? phys_tok(ptab, a.pshift, pre[u]) : pre[u];
        }
      } else {
        stage(0, nb);
      }
      __syncthreads();
      run(nb);
    }
    for (int bat = kMaxTokensPerSplit; bat < n_here; bat += kMaxTokensPerSplit) {
      const int nb = min(kMaxTokensPerSplit, n_here - bat);
      __syncthreads();
      stage(bat, nb);
      __syncthreads();
      run(nb);
    }
  } else {
    attend<G, false>(a, Kr, Vr, slot, n_here, [&](int i) { return (int64_t)(t0 + i); }, qf, acc);
  }
  attn_finish<G, FINAL>(a, acc, red, b, g, it.split);
}

// Log-sum-exp merge of the split partials: 16 lanes per (batch, query head),
// one wave of four rows per workgroup, so that the few rows of a long-context
// batch spread over many compute units (one round of dependent loads each).
constexpr int kCombineThreads = 64;
__global__ __launch_bounds__(kCombineThreads) void k_combine(AttnArgs a, int n_rows) {
  const int rq0 = blockIdx.x * (kCombineThreads / 16) + (threadIdx.x >> 4);
  if (!split_by_bytes(a)) {
    if (rq0 >= n_rows) return;
    merge_partials(a.part + (int64_t)rq0 * a.n_split * kPartStride, a.n_split, kPartStride,
                   a.out + (int64_t)rq0 * kDv, threadIdx.x & 15);
    return;
  }
  const int rq = min(rq0, n_rows - 1);
  const int G = a.Hq / a.Hkv;
  const int b = rq / a.Hq;
  const int hq = rq - b * a.Hq;
  const int g = hq / G;
  const int h = hq - g * G;
  int base, n;
  head_items(a, g, base, n);  // every lane of the wave takes part
  if (rq0 >= n_rows) return;
  const int64_t slot0 = ((int64_t)b * a.Hkv * a.n_split + base) * G + h;
  merge_partials(a.part + slot0 * kPartStride, n, (int64_t)G * kPartStride,
                 a.out + (int64_t)rq * kDv, threadIdx.x & 15);
}

template <int G>
hipError_t launch_g(const AttnArgs& a, int rows, bool final_out, hipStream_t s, const KEvents& ev) {
  const dim3 grid(rows * a.n_split);
  if (a.ptab) {
    if (final_out) return launch_k(k_attn<G, true, true>, grid, dim3(kAttnThreads), s, ev, a);
    return launch_k(k_attn<G, false, true>, grid, dim3(kAttnThreads), s, ev, a);
  }
  if (final_out) return launch_k(k_attn<G, true, false>, grid, dim3(kAttnThreads), s, ev, a);
  return launch_k(k_attn<G, false, false>, grid, dim3(kAttnThreads), s, ev, a);
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

hipError_t launch_combine(const AttnArgs& a, int B, hipStream_t s, const KEvents& ev) {
  const int n_rows = B * a.Hq;
  if (n_rows <= 0) return hipSuccess;
  const int per = kCombineThreads / 16;
  return launch_k(k_combine, dim3((n_rows + per - 1) / per), dim3(kCombineThreads), s, ev, a,
                  n_rows);
}

}  // namespace ds
