// Streaming statistics of logits rows, gathered by one wavefront over a
// segment of consecutive slabs of one row (see sv_device.h for the layout).
//
// For a row x at temperature tau the step needs a reference r and the sum
// S = sum_t 2^((x_t - r) c) with c = log2(e) / tau, so that
// softmax(x / tau)_t = 2^((x_t - r) c) / S for any reference r (the row
// maximum is the usual choice; any value near it keeps the terms in range);
// the maximum and its lowest id at temperature 0; and, for draft rows with
// forks, the top-F tokens with the drafted token masked out.
//
// Temperature > 0: each lane fixes its reference to the maximum of its
// elements in the segment's first chunk and afterwards only exponentiates
// (no maximum pass); a chunk whose terms overflow (an element far above the
// reference) raises the reference to that chunk's maximum and is
// recomputed.  A chunk's terms are summed in fp32 (pairwise), chunks in
// fp64.  Lanes, then segments, are combined with S = sum_i S_i 2^((r_i - r) c).
// Temperature 0: maxima only.
#pragma once

#include "sv_device.h"

namespace sv {

struct Warm {
  float r;   // reference (-inf until the lane has seen an element)
  float hi;  // r * c rounded to fp32: the lane's terms are 2^(x c - hi)
  double s;  // sum of the terms so far
};

struct Greedy {
  float m;   // running maximum
  int arg;   // lowest id holding it (when asked for)
};

__device__ __forceinline__ void warm_init(Warm& a) {
  a.r = neg_inf();
  a.hi = neg_inf();
  a.s = 0.0;
}
__device__ __forceinline__ void greedy_init(Greedy& a) {
  a.m = neg_inf();
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

// Sums of 2^(x c - hi) per vector (pairwise inside the vector) and over the
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
#ifdef SV_EXP_SCHED
    __builtin_amdgcn_sched_barrier(0);
#endif
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

// Rare path: the chunk's terms overflowed (an element far above the
// reference) or the lane had no reference yet.  The reference is raised to
// the chunk's maximum, the old sum rescaled and the chunk recomputed.
struct WarmFix {
  float r, hi, sc;
  double s;
  float vs[kU];
};

template <typename In>
__device__ __noinline__ WarmFix warm_redo(uint4 v0, uint4 v1, uint4 v2, uint4 v3, float r,
                                          float hi, double s, float c) {
  static_assert(kU == 4, "warm_redo takes four vectors");
  const uint4 raw[kU] = {v0, v1, v2, v3};
  WarmFix w;
  float m8[kU];
  const float rn = fmaxf(r, vec_maxima<In>(raw, m8));
  w.r = r;
  w.hi = hi;
  w.s = s;
  w.sc = 0.0f;
#pragma unroll
  for (int u = 0; u < kU; ++u) w.vs[u] = 0.0f;
  if (rn > neg_inf()) {
    // hn is the new reference exactly as the terms use it (rn c rounded to
    // fp32): the product is not contracted into the rescaling below
#pragma clang fp contract(off)
    const float hn = rn * c;
    // old terms 2^(x c - hi) become 2^(x c - hn) = old * 2^(hi - hn)
    if (s > 0.0) w.s = s * (double)__builtin_amdgcn_exp2f(hi - hn);
    w.r = rn;
    w.hi = hn;
    w.sc = exp_sums<In>(raw, c, hn, w.vs);
  }
  return w;
}

// The chunk's sums of terms (per vector in vs, and the total), before the
// overflow check.  On the segment's first chunk the reference is first set
// to the lane's maximum of that chunk (m8 then holds the vector maxima).
template <typename In, bool FIRST>
__device__ __forceinline__ float warm_terms(Warm& a, const uint4 (&raw)[kU], float c,
                                            float (&m8)[kU], float (&vs)[kU]) {
  if constexpr (FIRST) {
    const float mc = vec_maxima<In>(raw, m8);
    if (mc > neg_inf()) {
      a.r = mc;
      a.hi = mc * c;
    }
  }
  return exp_sums<In>(raw, c, a.hi, vs);
}

__device__ __forceinline__ bool warm_overflow(float sc) { return !(sc < pos_inf()); }

// A lane whose chunk overflowed (or that had no reference yet): the
// reference is raised and the chunk recomputed (sc, vs replaced).
template <typename In>
__device__ __forceinline__ void warm_fix(Warm& a, const uint4 (&raw)[kU], float c, float& sc,
                                         float (&vs)[kU]) {
  const WarmFix w = warm_redo<In>(raw[0], raw[1], raw[2], raw[3], a.r, a.hi, a.s, c);
  a.r = w.r;
  a.hi = w.hi;
  a.s = w.s;
  sc = w.sc;
#pragma unroll
  for (int u = 0; u < kU; ++u) vs[u] = w.vs[u];
}

// Folds one chunk into the lane's sum and returns the chunk's sum of terms;
// vs gets the per-vector sums and `fixed` whether some lane's reference was
// raised (wave-uniform).  Every lane must call it (it contains a
// wave-uniform branch).
template <typename In, bool FIRST>
__device__ __forceinline__ float warm_fold_vs(Warm& a, const uint4 (&raw)[kU], float c,
                                              float (&m8)[kU], float (&vs)[kU], bool& fixed) {
  float sc = warm_terms<In, FIRST>(a, raw, c, m8, vs);
  const bool redo = warm_overflow(sc);
  fixed = false;
  if (__ballot(redo)) {
    fixed = true;
    if (redo) warm_fix<In>(a, raw, c, sc, vs);
  }
  a.s += (double)sc;
  return sc;
}

template <typename In, bool FIRST>
__device__ __forceinline__ float warm_fold(Warm& a, const uint4 (&raw)[kU], float c,
                                           float (&m8)[kU]) {
  float vs[kU];
  bool fixed;
  return warm_fold_vs<In, FIRST>(a, raw, c, m8, vs, fixed);
}

// Temperature 0: running maximum, and the lowest id holding it.  e_base is
// the element index of the lane's vector 0; vector u starts u slabs later.
template <typename In>
__device__ __forceinline__ void greedy_fold(Greedy& a, const uint4 (&raw)[kU], int e_base,
                                            bool want_arg, float (&m8)[kU]) {
  constexpr int VEC = Elem<In>::VEC;
  const float mc = vec_maxima<In>(raw, m8);
  if (want_arg && mc > a.m) {
    // first element equal to the new maximum (ids increase with u, then e;
    // padding reads -inf and never equals mc > -inf)
    int first = kEmptyId;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const int id = e_base + u * slab_elems<In>() + e;
        if (first == kEmptyId && elem<In>(raw[u], e) == mc) first = id;
      }
    }
    a.arg = first;
  }
  a.m = fmaxf(a.m, mc);
}

struct WaveStats {
  float m;   // reference (temperature > 0) or maximum (temperature 0)
  double s;  // sum of 2^((x - m) c)
  int arg;
};

// Combines the lanes' sums relative to M = the largest lane reference; every
// lane gets the result.  Lane terms are 2^(x c - hi_l); relative to M they
// are multiplied by 2^(hi_l - hm) with hm = M c rounded to fp32.  The sum
// returned is relative to 2^hm: the exact M c = hm + lm (lm = fma(M, c,
// -hm)), and the factor 2^-lm that makes it relative to M is applied by
// whoever merges the partials (merge_scale), once per partial.
__device__ __forceinline__ WaveStats wave_finish_warm(const Warm& a, float c) {
  // hm must be M c rounded to fp32 (merge_scale corrects for that rounding),
  // so the product is not contracted into the subtraction
#pragma clang fp contract(off)
  WaveStats r;
  r.m = wave_max(a.r);
  r.s = 0.0;
  r.arg = kEmptyId;
  if (finitef(r.m)) {
    const float hm = r.m * c;
    const double part = (a.s > 0.0) ? a.s * (double)__builtin_amdgcn_exp2f(a.hi - hm) : 0.0;
    r.s = wave_sum(part);
  }
  return r;
}

// The factor that turns a partial sum relative to 2^(m c rounded to fp32)
// (wave_finish_warm) into one relative to the reference M >= m:
// 2^((m - M) c - lm) with lm = fma(m, c, -m c), the rounding of m c.
__device__ __forceinline__ double merge_scale(float m, float M, float c) {
  const float hm = m * c;
  const float lm = fmaf(m, c, -hm);
  return exp2(((double)m - (double)M) * (double)c - (double)lm);
}

__device__ __forceinline__ WaveStats wave_finish_greedy(const Greedy& a) {
  WaveStats r;
  r.m = wave_max(a.m);
  r.s = 0.0;
  r.arg = wave_min(a.m == r.m ? a.arg : (int)kEmptyId);
  return r;
}

// ---------------------------------------------------------------- forks
// Fork candidates of a wave's segment of a row.  A vector is a candidate
// when it may hold an element in the segment's top-f: in the segment's
// first chunk, when its maximum reaches the threshold kv (the f-th largest
// lane maximum of that chunk: at least f elements reach it, so no element
// of the top-f lies below it); in later chunks, at temperature 0 when its
// maximum exceeds kv (an element equal to kv there has a larger id than
// the f elements that reach kv in the first chunk, so it cannot enter the
// top-f), and at temperature > 0 when its sum of terms reaches
// 2^(kv c - hi) (less a margin for rounding), which any element at or
// above kv guarantees.  A candidate lane appends the vector's element index
// and its maximum to its own slots in LDS; where the maximum was not
// computed (later chunks at temperature > 0) the index is tagged in its low
// bit (indices are multiples of the vector width) and the maximum replaced
// by the key of inexact_key, which bounds it from both sides.  Nothing
// else happens while streaming, so the chunk's registers
// are free as soon as it is folded.  At the end of the segment the slots
// are written out, compacted, for the row's ranking; they are reduced in
// the wave instead (vectors re-read, elements ranked, the wave's top-F kept
// and kv raised) only if some lane could overflow with the next chunk, or
// if the segment has more candidates than its share of the output.
constexpr int kCandSlots = 16;
constexpr int kCandInexact = 1;  // tag bit of a candidate whose maximum is unknown

// Key of a vector whose maximum was not computed, from its sum of terms vs
// = sum_e 2^(x_e c - hi): with vs in [2^(e-1), 2^e) (e its binary exponent),
// key = e + hi.  Its largest element x_max has a term of at most vs and at
// least vs / VEC (the other terms are no larger), so
//   key - 1 - log2(VEC) <= x_max c <= key,
// up to the rounding of the terms and of the key (a relative 1e-6 or so;
// the reader adds a margin).  A sum that is zero, subnormal or not finite
// gives +inf: no bound.
__device__ __forceinline__ float inexact_key(float vs, float hi) {
  if (!(vs >= 1.17549435e-38f && vs < pos_inf())) return pos_inf();
  return (float)__builtin_amdgcn_frexp_expf(vs) + hi;
}

template <int F>
struct CandLds {
  int pos[kCandSlots][kLanes];    // element index of each candidate vector (| tag)
  float vm[kCandSlots][kLanes];   // its maximum, the drafted token masked (inexact: the key)
  float wv[F > 0 ? F : 1];        // the wave's top-F so far (best first)
  int wi[F > 0 ? F : 1];
};

// Appends vector u of this lane's chunk when bit u of `bits` is set.
template <int F>
__device__ __forceinline__ void cand_append(CandLds<F>* L, unsigned bits, int e_base, int slab,
                                            const float (&m8)[kU], bool exact, int& nc) {
  const int lane = lane_id();
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    if ((bits >> u) & 1u) {
      L->pos[nc][lane] = (e_base + u * slab) | (exact ? 0 : kCandInexact);
      L->vm[nc][lane] = m8[u];
      ++nc;
    }
  }
}

// Reduces the slots: re-reads the candidate vectors (NB per round), ranks
// their elements (id < V, id != mask_id, at or above the lane's running
// threshold) together with the wave's list, keeps the top-F and raises kv to
// the list's F-th entry once the list is full (F >= f, so every element of
// the top-f is at or above it).  Clears the slots.
template <typename In, int F, int NB>
__device__ __forceinline__ void cand_reduce(CandLds<F>* L, const In* __restrict__ row, int V,
                                            int mask_id, int& nc, float& kv) {
  if constexpr (F > 0) {
    constexpr int VEC = Elem<In>::VEC;
    const int lane = lane_id();
    TopList<F> mine;
    mine.clear();
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < F; ++r) mine.insert(L->wv[r], L->wi[r]);
    }
    const int nmax = wave_max_int(nc);
    for (int i0 = 0; i0 < nmax; i0 += NB) {
      uint4 v[NB];
      int e0[NB];
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        e0[q] = -1;
        v[q] = make_uint4(Elem<In>::kNegInfWord, Elem<In>::kNegInfWord, Elem<In>::kNegInfWord,
                          Elem<In>::kNegInfWord);
        if (i0 + q < nc) {
          e0[q] = L->pos[i0 + q][lane] & ~kCandInexact;
          load_vec<In>(row, e0[q], V, v[q]);
        }
      }
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        float thr = fmaxf(kv, mine.v[F - 1]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float x = elem<In>(v[q], e);
          const int id = e0[q] + e;
          if (x >= thr && e0[q] >= 0 && id < V && id != mask_id) {
            mine.insert(x, id);
            thr = fmaxf(kv, mine.v[F - 1]);
          }
        }
      }
    }
    TopList<F> top;
    wave_merge_lists<F>(mine, F, top);
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < F; ++r) { L->wv[r] = top.v[r]; L->wi[r] = top.i[r]; }
    }
    if (top.i[F - 1] != kEmptyId) kv = fmaxf(kv, top.v[F - 1]);
    nc = 0;
  }
}

}  // namespace sv
