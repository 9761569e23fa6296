// Per-chunk statistics of one logits row, computed by one wavefront from
// its registers (see sv_device.h for the chunk layout).
//
// For a row x at temperature tau the step needs, per row: the maximum m,
// the sum S = sum_t 2^((x_t - m) * c) with c = log2(e) / tau (so that
// softmax(x / tau)_t = 2^((x_t - m) c) / S), the argmax (temperature 0), and
// for the draft rows with forks the top-f candidates with the drafted token
// masked out.  A chunk reports (m_c, S_c) with S_c taken at its own m_c;
// rows merge them as S = sum_c S_c 2^((m_c - m) c).
#pragma once

#include "sv_device.h"

namespace sv {

template <int F>
struct ChunkStats {
  float m;       // chunk maximum (masked element excluded)
  double s;      // sum of 2^((x - m) c) over the chunk, exact reference m
  int arg;       // lowest id holding m (only when asked for)
  TopList<F> top;  // chunk top-f by (logit desc, id asc), masked id excluded
};

// Statistics of one chunk held in `raw`.
//   c        log2(e)/tau in fp32; ignored when greedy
//   greedy   tau == 0: no sums, only maxima (and argmax / top-f)
//   mask_id  token id excluded from everything (-1: none)
//   want_arg compute the argmax (lowest id among maxima)
//   f        runtime fan-out (F >= f), used only when F > 0
template <typename In, int F>
__device__ __forceinline__ ChunkStats<F> chunk_stats(uint4 (&raw)[kU], int64_t cstart, int V,
                                                     float c, bool greedy, int64_t mask_id,
                                                     bool want_arg, int f) {
  constexpr int VEC = Elem<In>::VEC;
  constexpr int CH = chunk_elems<In>();
  const int lane = lane_id();
  ChunkStats<F> r;
  r.top.clear();
  r.arg = kEmptyId;
  r.s = 0.0;

  // Exclude the masked token (only the one wave whose chunk holds it).
  if (mask_id >= cstart && mask_id < cstart + CH) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const int64_t id = cstart + (int64_t)(u * kLanes + lane) * VEC + e;
        if (id == mask_id) set_neg_inf<In>(raw[u], e);
      }
    }
  }

  // Pass 1: lane maximum, then the wave's.
  float m = neg_inf();
#pragma unroll
  for (int u = 0; u < kU; ++u) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) m = fmaxf(m, elem<In>(raw[u], e));
  }
  const float M = wave_max(m);
  r.m = M;

  if (want_arg) {
    int best = kEmptyId;
    if (m == M) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const int64_t id = cstart + (int64_t)(u * kLanes + lane) * VEC + e;
          if (best == kEmptyId && elem<In>(raw[u], e) == M && id < V) best = (int)id;
        }
      }
    }
    r.arg = wave_min(best);
  }

  // Candidates for the top-f: any element of the chunk's top-f is at least
  // the f-th largest lane maximum.
  float theta = pos_inf();
  if constexpr (F > 0) theta = wave_fth_largest<F>(m, f);
  TopList<F> mine;
  mine.clear();

  if (!greedy && finitef(M)) {
    // Pass 2: S = sum 2^((x - M) c).  M*c is split exactly into hi + lo
    // (fma gives the rounding error of the product), the elements use hi,
    // and the common factor 2^-lo is applied once to the wave's sum.
    const float hi = M * c;
    const float lo = fmaf(M, c, -hi);
    float su[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float a[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float x = elem<In>(raw[u], e);
        a[e] = __builtin_amdgcn_exp2f(fmaf(x, c, -hi));
        if constexpr (F > 0) {
          if (x >= theta) {
            const int64_t id = cstart + (int64_t)(u * kLanes + lane) * VEC + e;
            if (id < V && id != mask_id) mine.insert(x, (int)id);
          }
        }
      }
      // pairwise sum of the vector's elements
#pragma unroll
      for (int w = VEC / 2; w > 0; w >>= 1) {
#pragma unroll
        for (int e = 0; e < w; ++e) a[e] = a[e] + a[e + w];
      }
      su[u] = a[0];
    }
#pragma unroll
    for (int w = kU / 2; w > 0; w >>= 1) {
#pragma unroll
      for (int u = 0; u < w; ++u) su[u] = su[u] + su[u + w];
    }
    const double s = wave_sum((double)su[0]);
    r.s = s * exp2(-(double)lo);
  } else if constexpr (F > 0) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float x = elem<In>(raw[u], e);
        if (x >= theta) {
          const int64_t id = cstart + (int64_t)(u * kLanes + lane) * VEC + e;
          if (id < V && id != mask_id) mine.insert(x, (int)id);
        }
      }
    }
  }
  if constexpr (F > 0) wave_merge_lists<F>(mine, f, r.top);
  return r;
}

}  // namespace sv
