// label.hip -- label-cache build (prefill) and append (decode).
//
// [DS] "offline calibration": the heavy-channel values of K are copied into
// a contiguous label cache so that the approximate scores read contiguous
// memory; at prefill every token is copied, at decode only the new one.  The
// label may be stored in 4 bits; the format (symmetric codes in [-7, 7] with
// one fp16 absmax scale per token, low nibble first) is specified in ds.h.
//
// Layout of the work: a workgroup takes 64 items (an item is one (batch, KV
// head, token)).  Their K rows are first staged in LDS with coalesced 16-byte
// loads (a whole row per 16 lanes), then four lanes per item pick the r heavy
// channels out of LDS, quantise if needed and store the label.
#include "ds_internal.h"

namespace ds {
namespace {

constexpr int kItems = 64;
constexpr int kThreads = 256;
constexpr int kMaxDk = 128;
constexpr int kRowPad = 8;  // halves; keeps 16-byte alignment, spreads LDS banks

__global__ __launch_bounds__(kThreads) void k_label(LabelArgs a) {
  __shared__ __align__(16) __half rows[kItems][kMaxDk + kRowPad];
  __shared__ int64_t src_off[kItems];
  __shared__ int64_t dst_tok[kItems];  // label slot index (row * slots + t), -1 if idle
  __shared__ int32_t src_c8[kItems];   // 16-byte pieces of the item's K row

  const int tid = threadIdx.x;
  if (tid < kItems) {
    int64_t so = 0, dt = -1;
    int row, t;
    if (a.pos != nullptr) {
      const int item = blockIdx.x * kItems + tid;
      row = item;
      t = -1;
      if (item < a.n_items) {
        const int b = item / a.Hkv;
        t = a.pos[b] - a.pos_minus_one;
      }
    } else {
      row = blockIdx.x / a.tiles_per_row;
      const int tile = blockIdx.x - row * a.tiles_per_row;
      t = a.t_begin + tile * kItems + tid;
      if (t >= a.t_end) t = -1;
    }
    int c8 = a.d_k >> 3;
    if (t >= 0 && t < a.cap) {
      const int b = row / a.Hkv;
      const int g = row - b * a.Hkv;
      // per-head layout: the head's block, rows of its kept columns; a fully
      // pruned head (no K columns) has no label
      const LabelArgs h = with_head(a, g);
      c8 = h.d_k >> 3;
      if (c8 > 0) {
        so = kv_off(h.ptab, h.pshift, h.max_pages, b, t, h.ks0, h.ks2) + (int64_t)g * h.ks1 +
             (h.K - a.K);
        dt = (int64_t)row * a.slots + t;
      }
    }
    src_off[tid] = so;
    dst_tok[tid] = dt;
    src_c8[tid] = c8;
  }
  __syncthreads();

  // Stage the K rows: d_k / 8 lanes per row, one 16-byte load each.
  const int c8n = a.d_k >> 3;  // the widest row
  for (int i = tid; i < kItems * c8n; i += kThreads) {
    const int item = i / c8n;
    const int c8 = i - item * c8n;
    if (dst_tok[item] >= 0 && c8 < src_c8[item]) {
      const uint4 v = *reinterpret_cast<const uint4*>(a.K + src_off[item] + c8 * 8);
      *reinterpret_cast<uint4*>(&rows[item][c8 * 8]) = v;
    }
  }
  __syncthreads();

  // Four lanes per item; lane `part` takes channel pairs part, part+4, ...
  const int item = tid >> 2;
  const int part = tid & 3;
  const int64_t dt = dst_tok[item];
  const int row = dt >= 0 ? (int)(dt / a.slots) : 0;
  const int g = row % a.Hkv;
  const int32_t* chan = a.chan + (int64_t)g * a.r;
  const int npairs = (a.r + 1) >> 1;

  if (!a.is_int4) {
    if (dt < 0) return;
    __half* dst = a.lab16 + dt * a.r;
    for (int p = part; p < npairs; p += 4) {
      const int j = 2 * p;
      dst[j] = rows[item][chan[j]];
      if (j + 1 < a.r) dst[j + 1] = rows[item][chan[j + 1]];
    }
    return;
  }

  // int4: absmax over the token's r heavy values (all four lanes of the item
  // take part in the reduction, idle items included, so the shuffles see a
  // full quad).
  float amax = 0.0f;
  if (dt >= 0) {
    for (int p = part; p < npairs; p += 4) {
      amax = fmaxf(amax, fabsf(h2f(rows[item][chan[2 * p]])));
      amax = fmaxf(amax, fabsf(h2f(rows[item][chan[2 * p + 1]])));
    }
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  if (dt < 0) return;

  const __half s16 = __float2half_rn(amax / 7.0f);  // IEEE division, round to nearest even
  const float sf = h2f(s16);
  uint8_t* dst = a.codes + dt * (a.r >> 1);
  for (int p = part; p < npairs; p += 4) {
    int c[2] = {0, 0};
    if (sf != 0.0f) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float v = rintf(h2f(rows[item][chan[2 * p + u]]) / sf);
        v = fminf(fmaxf(v, -7.0f), 7.0f);
        c[u] = (int)v;
      }
    }
    dst[p] = (uint8_t)((c[0] & 0xF) | ((c[1] & 0xF) << 4));
  }
  if (part == 0) a.scales[dt] = s16;
}

}  // namespace

hipError_t launch_label(const LabelArgs& a, int n_blocks, hipStream_t s, const KEvents& ev) {
  if (n_blocks <= 0) return hipSuccess;
  return launch_k(k_label, dim3(n_blocks), dim3(kThreads), s, ev, a);
}

}  // namespace ds
