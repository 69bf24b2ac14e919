// score_select.hip -- streaming score and select kernels (steps 1-2 and 3a
// of a Double Sparsity decode step, [DS] "online forward computation") for
// rows outside the other paths' limits: many workgroups per row write every
// score as a key to the workspace, then one workgroup per row runs a radix
// select over them (they are still cache resident).
#include "score_common.h"

namespace ds {
namespace {

// Rows with S <= k (or k <= 0): every token, in order.  Returns true if so.
template <int NT>
__device__ __forceinline__ bool emit_all_if_short(const ScoreArgs& a, int row, int S) {
  if (a.k > 0 && S > a.k) return false;
  int32_t* out = a.idx + (int64_t)row * a.idx_stride;
  for (int t = threadIdx.x; t < S; t += NT) out[t] = t;
  if (a.pad_idx)
    for (int t = S + threadIdx.x; t < a.idx_stride; t += NT) out[t] = -1;
  if (threadIdx.x == 0) a.count[row] = S;
  return true;
}

template <int NT>
__device__ __forceinline__ void finish_row(const ScoreArgs& a, int row) {
  int32_t* out = a.idx + (int64_t)row * a.idx_stride;
  if (a.pad_idx)
    for (int t = a.k + threadIdx.x; t < a.idx_stride; t += NT) out[t] = -1;
  if (threadIdx.x == 0) a.count[row] = a.k;
}

template <int NT, int R, bool INT4>
__global__ __launch_bounds__(NT) void k_score_chunk(ScoreArgs a) {
  __shared__ QueryLds qg;
  const int row = blockIdx.x / a.n_chunks;
  const int c = blockIdx.x - row * a.n_chunks;
  const int b = row / a.Hkv;
  const int g = row - b * a.Hkv;
  const int S = row_len(a, b);
  if (a.k <= 0 || S <= a.k) return;
  if (a.heads && a.heads[g].k_cols == 0) return;  // a fully pruned head: no labels
  const int t_beg = c * a.chunk;
  const int t_end = min(S, t_beg + a.chunk);
  if (t_beg >= t_end) return;
  const RowPtrs p = row_ptrs(a, row);
  uint32_t* kr = a.keys + (int64_t)row * a.keys_stride;
  score_range<NT, R, INT4>(
      a, p, qg, t_beg, t_end, [&](int t, float, uint32_t key) { kr[t] = key; },
      [&]() {
        gather_query(a, b, g, qg);
        __syncthreads();
      });
}

template <int NT>
__global__ __launch_bounds__(NT) void k_select_stream(ScoreArgs a) {
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t scan_tmp[NT / 64];
  __shared__ uint32_t sel[4];
  const int row = blockIdx.x;
  const int b = row / a.Hkv;
  const int S = row_len(a, b);
  if (pruned_row<NT>(a, row, row - b * a.Hkv)) return;
  if (emit_all_if_short<NT>(a, row, S)) return;
  const uint32_t* kr = a.keys + (int64_t)row * a.keys_stride;
  const Threshold th = radix_select_global<NT>(kr, S, (uint32_t)a.k, hist, scan_tmp, sel);
  emit_global<NT>(kr, S, th, a.idx + (int64_t)row * a.idx_stride, scan_tmp);
  finish_row<NT>(a, row);
}

constexpr int kChunkThreads = 256;
constexpr int kSelectThreads = 1024;

template <template <int, int, bool> class KT, int NT>
struct Pick {
  static void* get(int r, bool int4) {
    if (int4) {
      if (r == 8) return (void*)KT<NT, 8, true>::fn;
      if (r == 16) return (void*)KT<NT, 16, true>::fn;
      return (void*)KT<NT, 0, true>::fn;
    }
    if (r == 8) return (void*)KT<NT, 8, false>::fn;
    if (r == 16) return (void*)KT<NT, 16, false>::fn;
    return (void*)KT<NT, 0, false>::fn;
  }
};

template <int NT, int R, bool INT4>
struct ChunkK {
  static constexpr auto fn = k_score_chunk<NT, R, INT4>;
};

}  // namespace

hipError_t launch_score_chunks(const ScoreArgs& a, int rows, hipStream_t s, const KEvents& ev) {
  if (rows <= 0 || a.n_chunks <= 0) return hipSuccess;
  void* fn = Pick<ChunkK, kChunkThreads>::get(a.r, a.is_int4 != 0);
  void* args[] = {const_cast<ScoreArgs*>(&a)};
  if (ev.start && ev.stop)
    return hipExtLaunchKernel(fn, dim3(rows * a.n_chunks), dim3(kChunkThreads), args, 0, s,
                              ev.start, ev.stop, 0);
  return hipLaunchKernel(fn, dim3(rows * a.n_chunks), dim3(kChunkThreads), args, 0, s);
}

hipError_t launch_select_stream(const ScoreArgs& a, int rows, hipStream_t s, const KEvents& ev) {
  if (rows <= 0) return hipSuccess;
  return launch_k(k_select_stream<kSelectThreads>, dim3(rows), dim3(kSelectThreads), s, ev, a);
}

}  // namespace ds
