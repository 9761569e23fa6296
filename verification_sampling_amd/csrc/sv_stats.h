// Statistics of a logits row, gathered by one wavefront over a segment of
// consecutive chunks (see sv_device.h for the chunk layout).
//
// For a row x at temperature tau the step needs, per row, a reference r and
// the sum S = sum_t 2^((x_t - r) c) with c = log2(e) / tau, so that
// softmax(x / tau)_t = 2^((x_t - r) c) / S for any reference r (the row
// maximum is the usual choice; any value near it keeps the terms in range);
// the maximum and argmax at temperature 0; and, for draft rows with forks,
// the top-f tokens with the drafted token masked out.
//
// Temperature > 0: each lane fixes its reference r to the maximum of its
// elements in the segment's first chunk and then only exponentiates (no
// maximum pass); a chunk whose terms overflow (an element far above r)
// raises r to that chunk's maximum and is recomputed.  Lanes, then
// segments, are combined with S = sum_i S_i 2^((r_i - r) c).
// Temperature 0: maxima only.
#pragma once

#include "sv_device.h"

namespace sv {

struct LaneStats {
  float r;   // reference (temperature > 0) or running maximum (temperature 0)
  float hi;  // r * c rounded; the terms are 2^(x c - hi)
  float s;   // sum of 2^(x c - hi) over the lane's elements so far
  int arg;   // temperature 0: lowest id holding the maximum (when asked for)
};

__device__ __forceinline__ void lane_init(LaneStats& a) {
  a.r = neg_inf();
  a.hi = neg_inf();
  a.s = 0.0f;
  a.arg = kEmptyId;
}

// Maximum of each 16-byte vector and of the lane's whole chunk.
template <typename In>
__device__ __forceinline__ float vec_maxima(const uint4 (&raw)[kU], float (&m8)[kU]) {
  constexpr int VEC = Elem<In>::VEC;
  float mc = neg_inf();
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    float m = elem<In>(raw[u], 0);
#pragma unroll
    for (int e = 1; e < VEC; ++e) m = fmaxf(m, elem<In>(raw[u], e));
    m8[u] = m;
    mc = fmaxf(mc, m);
  }
  return mc;
}

// Sums of 2^(x c - hi) per vector (pairwise inside the vector) and for the
// chunk (pairwise over the vectors).
template <typename In>
__device__ __forceinline__ float exp_sums(const uint4 (&raw)[kU], float c, float hi,
                                          float (&vs)[kU]) {
  constexpr int VEC = Elem<In>::VEC;
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    float t[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) t[e] = __builtin_amdgcn_exp2f(fmaf(elem<In>(raw[u], e), c, -hi));
#pragma unroll
    for (int w = VEC / 2; w > 0; w >>= 1) {
#pragma unroll
      for (int e = 0; e < w; ++e) t[e] = t[e] + t[e + w];
    }
    vs[u] = t[0];
  }
  float a[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) a[u] = vs[u];
#pragma unroll
  for (int w = kU / 2; w > 0; w >>= 1) {
#pragma unroll
    for (int u = 0; u < w; ++u) a[u] = a[u] + a[u + w];
  }
  return a[0];
}

// Temperature > 0, rare path: a chunk whose terms overflowed (an element
// far above the lane's reference, or no reference yet) raises the reference
// to the chunk's maximum; the old sum is rescaled and the chunk recomputed.
struct WarmFix {
  float r, hi, s, sc;
  float vs[kU];
};

template <typename In>
__device__ __noinline__ WarmFix warm_redo(uint4 v0, uint4 v1, uint4 v2, uint4 v3, float r,
                                          float hi, float s, float c) {
  const uint4 raw[kU] = {v0, v1, v2, v3};
  static_assert(kU == 4, "warm_redo takes four vectors");
  WarmFix w;
  float m8[kU];
  const float mc = vec_maxima<In>(raw, m8);
  const float rn = fmaxf(r, mc);
  w.r = r;
  w.hi = hi;
  w.s = s;
  w.sc = 0.0f;
#pragma unroll
  for (int u = 0; u < kU; ++u) w.vs[u] = 0.0f;
  if (rn > neg_inf()) {
    const float hn = rn * c;
    // old terms 2^(x c - hi) become 2^(x c - hn) = old * 2^(hi - hn)
    if (s > 0.0f) w.s = s * __builtin_amdgcn_exp2f(hi - hn);
    w.r = rn;
    w.hi = hn;
    w.sc = exp_sums<In>(raw, c, hn, w.vs);
  }
  return w;
}

// Temperature > 0: folds one chunk into the lane's sum; vs gets the
// per-vector sums (for the fork prefilter).  On the segment's first chunk
// the reference is set to the lane's maximum of that chunk (returned in
// lane_max; otherwise lane_max is the current reference).  Every lane must
// call it (it contains a wave-uniform branch).
template <typename In>
__device__ __forceinline__ void fold_warm(LaneStats& a, const uint4 (&raw)[kU], float c,
                                          bool first, float (&vs)[kU], float& lane_max) {
  if (first) {
    float m8[kU];
    const float mc = vec_maxima<In>(raw, m8);
    if (mc > neg_inf()) {
      a.r = fmaxf(a.r, mc);
      a.hi = a.r * c;
    }
    lane_max = mc;
  } else {
    lane_max = a.r;
  }
  float sc = exp_sums<In>(raw, c, a.hi, vs);
  const bool redo = !(sc < pos_inf());  // overflow, or no reference yet
  if (__ballot(redo)) {
    if (redo) {
      const WarmFix w = warm_redo<In>(raw[0], raw[1], raw[2], raw[3], a.r, a.hi, a.s, c);
      a.r = w.r;
      a.hi = w.hi;
      a.s = w.s;
      sc = w.sc;
#pragma unroll
      for (int u = 0; u < kU; ++u) vs[u] = w.vs[u];
    }
  }
  a.s += sc;
}

// Temperature 0: running maximum, and the lowest id holding it.
template <typename In>
__device__ __forceinline__ void fold_greedy(LaneStats& a, const uint4 (&raw)[kU], int64_t cstart,
                                            bool want_arg, float (&m8)[kU], float& mc) {
  constexpr int VEC = Elem<In>::VEC;
  const int lane = lane_id();
  mc = vec_maxima<In>(raw, m8);
  if (want_arg && mc > a.r) {
    // first element equal to the new maximum (ids increase with u then e;
    // padding reads -inf and never equals mc > -inf)
    int first = kEmptyId;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const int id = (int)(cstart + (int64_t)(u * kLanes + lane) * VEC + e);
        if (first == kEmptyId && elem<In>(raw[u], e) == mc) first = id;
      }
    }
    a.arg = first;
  }
  a.r = fmaxf(a.r, mc);
}

struct WaveStats {
  float m;   // reference (temperature > 0) or maximum (temperature 0)
  double s;  // sum of 2^((x - m) c)
  int arg;
};

// Combines the lanes' statistics; every lane gets the result.
__device__ __forceinline__ WaveStats wave_finish(const LaneStats& a, float c, bool greedy) {
  WaveStats r;
  r.m = wave_max(a.r);
  r.s = 0.0;
  r.arg = kEmptyId;
  if (greedy) {
    r.arg = wave_min(a.r == r.m ? a.arg : (int)kEmptyId);
  } else if (finitef(r.m)) {
    // lane terms are 2^(x c - hi_l); relative to M they are multiplied by
    // 2^(hi_l - M c): M*c is split exactly (hm + lm) and 2^-lm applied in fp64
    const float hm = r.m * c;
    const float lm = fmaf(r.m, c, -hm);
    const float part = (a.s > 0.0f) ? a.s * __builtin_amdgcn_exp2f(a.hi - hm) : 0.0f;
    r.s = wave_sum((double)part) * exp2(-(double)lm);
  }
  return r;
}

// Fork candidates of a row segment, per wave: elements that reach the
// threshold `kv` are appended to a buffer in LDS (kCandCap entries of
// (logit, id) per wave) by ballot compaction, one element position at a
// time; the buffer is reduced to its top-F (logit descending, id ascending)
// whenever another round could overflow it, which also raises kv to the
// F-th best candidate so far.  F is the fork fan-out rounded up to a power
// of two (the top-F contain the top-f); all list indices are compile-time.
constexpr int kCandCap = 128;

struct CandBuf {
  float* v;   // LDS, kCandCap entries
  int* id;    // LDS, kCandCap entries
  int n;      // entries in use (wave-uniform)
  float kv;   // threshold: F-th best so far once n >= F, else the first-chunk bound
};

// Top-F of the buffer, in every lane (entries past n empty).
template <int F>
__device__ __forceinline__ void cand_select(const CandBuf& cb, TopList<F>& out) {
  const int lane = lane_id();
  // each lane holds entries lane and lane + 64
  float v0 = neg_inf(), v1 = neg_inf();
  int i0 = kEmptyId, i1 = kEmptyId;
  if (lane < cb.n) { v0 = cb.v[lane]; i0 = cb.id[lane]; }
  if (lane + kLanes < cb.n) { v1 = cb.v[lane + kLanes]; i1 = cb.id[lane + kLanes]; }
  out.clear();
#pragma unroll
  for (int r = 0; r < F; ++r) {
    const bool first = better(v0, i0, v1, i1);
    float bv = first ? v0 : v1;
    int bi = first ? i0 : i1;
    wave_best(bv, bi);
    out.v[r] = bv;
    out.i[r] = bi;
    if (bi != kEmptyId) {
      if (i0 == bi) { v0 = neg_inf(); i0 = kEmptyId; }
      if (i1 == bi) { v1 = neg_inf(); i1 = kEmptyId; }
    }
  }
}

struct CandState {
  int n;
  float kv;
};

// Reduces the buffer to its top-F and raises the threshold.
template <int F>
__device__ __noinline__ CandState cand_compact(float* cv, int* ci, CandState st) {
  CandBuf cb;
  cb.v = cv;
  cb.id = ci;
  cb.n = st.n;
  cb.kv = st.kv;
  TopList<F> t;
  cand_select<F>(cb, t);
  const int lane = lane_id();
  int n = 0;
#pragma unroll
  for (int r = 0; r < F; ++r) n += (t.i[r] != kEmptyId) ? 1 : 0;
#pragma unroll
  for (int r = 0; r < F; ++r) {
    if (lane == r) { cv[r] = t.v[r]; ci[r] = t.i[r]; }
  }
  CandState out;
  out.n = n;
  out.kv = (n == F) ? fmaxf(st.kv, t.v[F - 1]) : st.kv;
  return out;
}

// Appends the elements of the flagged vectors (bit u of candbits) that reach
// the threshold: one ballot-compacted round per element position.
template <typename In, int F>
__device__ __noinline__ CandState cand_chunk(uint4 v0, uint4 v1, uint4 v2, uint4 v3,
                                             unsigned candbits, int64_t cstart, int V,
                                             int64_t mask_id, float* cv, int* ci, CandState st) {
  constexpr int VEC = Elem<In>::VEC;
  static_assert(kU == 4, "cand_chunk takes four vectors");
  const uint4 raw[kU] = {v0, v1, v2, v3};
  const int lane = lane_id();
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const bool cu = (candbits >> u) & 1u;
    if (__ballot(cu) == 0ull) continue;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const float x = elem<In>(raw[u], e);
      const int64_t id = cstart + (int64_t)(u * kLanes + lane) * VEC + e;
      const bool ok = cu && id < V && id != mask_id;
      unsigned long long m = __ballot(ok && x >= st.kv);
      if (m == 0ull) continue;
      if (st.n + kLanes > kCandCap) {
        st = cand_compact<F>(cv, ci, st);
        m = __ballot(ok && x >= st.kv);
        if (m == 0ull) continue;
      }
      const int pos = st.n + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32),
                                  __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
      if ((m >> lane) & 1ull) { cv[pos] = x; ci[pos] = (int)id; }
      st.n += __popcll(m);
    }
  }
  return st;
}

}  // namespace sv
