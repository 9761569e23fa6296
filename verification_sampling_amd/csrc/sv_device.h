// Device-side building blocks of libspecverify (gfx950, wave64).
//
// Layout convention used by every kernel: a logits row is cut into slabs of
// kLanes 16-byte vectors (512 bf16 or 256 fp32 elements); lane l holds the
// l-th vector of a slab, so one vector load instruction of a wave reads 1 KiB
// of contiguous memory.  A wave walks a row kU slabs (a chunk) at a time;
// inside a chunk lane l's vector u is at element (u * 64 + l) * VEC, so token
// order inside a chunk is slab by slab (u outer, lanes inner).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kLanes = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kLanes * kWavesPerBlock;
constexpr int kU = 4;          // 16-byte vectors per lane per tensor per chunk
constexpr int kMaxF = 16;      // largest fork fan-out
constexpr int kMaxK = 63;      // drafted positions: one lane each in a ballot
constexpr int kEmptyId = 0x7fffffff;

__device__ __forceinline__ float neg_inf() { return __uint_as_float(0xff800000u); }
__device__ __forceinline__ float pos_inf() { return __uint_as_float(0x7f800000u); }
__device__ __forceinline__ bool finitef(float x) { return x > neg_inf() && x < pos_inf(); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kLanes - 1); }

// Wave index inside the grid, as a wave-uniform (scalar) value.
__device__ __forceinline__ int64_t wave_global_id() {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  return (int64_t)blockIdx.x * kWavesPerBlock + w;
}

// Wave-uniform copies (lane 0's value), so the compiler can keep them in
// scalar registers and branch on them with scalar branches.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ unsigned uniform(unsigned x) {
  return (unsigned)__builtin_amdgcn_readfirstlane((int)x);
}
__device__ __forceinline__ float uniform(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// ---------------------------------------------------------------- handoffs
// Hand-off of data between workgroups of one launch (the blocks that share
// one row's residual sums and the block that draws from them).  The data are
// written with device-scope stores (sc1: written through to the
// device-coherent level) and read with device-scope loads; each writer waits
// for its stores to complete (s_waitcnt vmcnt(0)) before the arrival is
// counted with a device-scope atomic, and the reader loads only after
// seeing the final count.  A device-scope fence would also write back the
// whole L2 of the writer's XCD; this avoids that.

template <typename T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until this wave's vector memory operations have completed.
__device__ __forceinline__ void vm_complete() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt not waited on
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Counts one arrival (lane 0 of the calling wave) on a device-scope counter;
// returns true, in every lane, on the arrival that completes `count`, which
// also resets the counter for the next launch.  The caller must have made
// its data visible first (vm_complete in every wave that wrote).
__device__ __forceinline__ bool arrive_last(unsigned* ctr, unsigned count) {
  unsigned old = 0;
  if ((threadIdx.x & 63) == 0)
    old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = (unsigned)__builtin_amdgcn_readfirstlane((int)__shfl((int)old, 0));
  if (old != count - 1) return false;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if ((threadIdx.x & 63) == 0) st_dev(ctr, 0u);
  return true;
}

// ---------------------------------------------------------------- dtypes

template <typename In> struct Elem;
template <> struct Elem<float> {
  static constexpr int VEC = 4;                      // elements per 16 bytes
  static constexpr uint32_t kNegInfWord = 0xff800000u;
};
template <> struct Elem<uint16_t> {                  // bf16 bit patterns
  static constexpr int VEC = 8;
  static constexpr uint32_t kNegInfWord = 0xff80ff80u;
};

template <typename In>
constexpr int slab_elems() { return kLanes * Elem<In>::VEC; }
template <typename In>
constexpr int chunk_elems() { return kU * slab_elems<In>(); }

__device__ __forceinline__ uint32_t word_of(const uint4& v, int q) {
  return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}
__device__ __forceinline__ void set_word(uint4& v, int q, uint32_t w) {
  if (q == 0) v.x = w; else if (q == 1) v.y = w; else if (q == 2) v.z = w; else v.w = w;
}

// Element e (compile-time after unrolling) of a 16-byte vector, as fp32.
// bf16 -> fp32 is exact: the bf16 bits are the upper half of the fp32.
template <typename In>
__device__ __forceinline__ float elem(const uint4& v, int e) {
  if constexpr (sizeof(In) == 4) {
    return __uint_as_float(word_of(v, e));
  } else {
    const uint32_t w = word_of(v, e >> 1);
    return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
}

template <typename In>
__device__ __forceinline__ void set_neg_inf(uint4& v, int e) {
  if constexpr (sizeof(In) == 4) {
    set_word(v, e, 0xff800000u);
  } else {
    const uint32_t w = word_of(v, e >> 1);
    set_word(v, e >> 1, (e & 1) ? ((w & 0x0000ffffu) | 0xff800000u)
                                : ((w & 0xffff0000u) | 0x0000ff80u));
  }
}

// Loads this lane's kU vectors of one chunk: vector u at element
// e_base + u * slab_elems (e_base = the chunk's first element + lane * VEC).
// Vectors u >= nvalid and elements at or beyond V read as -inf; that memory
// is never touched (a partial vector is loaded element by element).  full:
// nvalid == kU and the whole chunk lies inside the row.
template <typename In>
__device__ __forceinline__ void load_vec(const In* __restrict__ row, int e0, int V, uint4& v);

#ifndef SV_NT_LOADS
#define SV_NT_LOADS 1
#endif

// One 16-byte load of streamed logits.  Every byte of a row is read once per
// pass, so the loads are marked non-temporal: the lines are not kept in the
// caches for reuse.
__device__ __forceinline__ uint4 load_stream16(const void* p) {
#if SV_NT_LOADS
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *reinterpret_cast<const uint4*>(p);
#endif
}

template <typename In>
__device__ __forceinline__ void load_chunk(const In* __restrict__ row, int e_base, int nvalid,
                                           int V, bool full, uint4 (&raw)[kU]) {
  constexpr int SLAB = slab_elems<In>();
  if (full) {
#pragma unroll
    for (int u = 0; u < kU; ++u) raw[u] = load_stream16(row + e_base + u * SLAB);
  } else {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (u < nvalid) {
        load_vec<In>(row, e_base + u * SLAB, V, raw[u]);
      } else {
        raw[u] = make_uint4(Elem<In>::kNegInfWord, Elem<In>::kNegInfWord,
                            Elem<In>::kNegInfWord, Elem<In>::kNegInfWord);
      }
    }
  }
}

// Loads one 16-byte vector at element e0 of a row; elements at or beyond V
// read as -inf and are never touched.
template <typename In>
__device__ __forceinline__ void load_vec(const In* __restrict__ row, int e0, int V, uint4& v) {
  constexpr int VEC = Elem<In>::VEC;
  if (e0 + VEC <= V) {
    v = *reinterpret_cast<const uint4*>(row + e0);
    return;
  }
  v = make_uint4(Elem<In>::kNegInfWord, Elem<In>::kNegInfWord, Elem<In>::kNegInfWord,
                 Elem<In>::kNegInfWord);
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    if (e0 + e < V) {
      if constexpr (sizeof(In) == 4) {
        set_word(v, e, __float_as_uint(row[e0 + e]));
      } else {
        const uint32_t h = row[e0 + e];
        const uint32_t w = word_of(v, e >> 1);
        set_word(v, e >> 1, (e & 1) ? ((w & 0xffffu) | (h << 16)) : ((w & 0xffff0000u) | h));
      }
    }
  }
}

// ---------------------------------------------------------------- wave ops
// Cross-lane operations use DPP lane permutations inside each row of 16
// lanes (quad swaps, half-row and row mirrors, row shifts) and v_readlane to
// combine the four rows, so every lane ends with the same value.  They must
// be called with all 64 lanes active.

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(x)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
  return __hiloint2double(dpp_i<CTRL>(__double2hiint(x)), dpp_i<CTRL>(__double2loint(x)));
}
__device__ __forceinline__ int readlane_i(int x, int l) { return __builtin_amdgcn_readlane(x, l); }
__device__ __forceinline__ float readlane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ double readlane_d(double x, int l) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(x), l),
                          __builtin_amdgcn_readlane(__double2loint(x), l));
}

constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppRowMirror = 0x140;     // lane i <-> 15-i within 16
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;

// Reduce within each row of 16 lanes (commutative op), then across the rows.
#define SV_ROW_REDUCE(T, DPP, OP, x)                  \
  x = OP(x, DPP<kDppQuadXor1>(x));                    \
  x = OP(x, DPP<kDppQuadXor2>(x));                    \
  x = OP(x, DPP<kDppRowHalfMirror>(x));               \
  x = OP(x, DPP<kDppRowMirror>(x));

__device__ __forceinline__ float op_maxf(float a, float b) { return fmaxf(a, b); }
__device__ __forceinline__ int op_mini(int a, int b) { return min(a, b); }
__device__ __forceinline__ int op_maxi(int a, int b) { return max(a, b); }
__device__ __forceinline__ double op_addd(double a, double b) { return a + b; }

__device__ __forceinline__ float wave_max(float x) {
  SV_ROW_REDUCE(float, dpp_f, op_maxf, x)
  return fmaxf(fmaxf(readlane_f(x, 0), readlane_f(x, 16)),
               fmaxf(readlane_f(x, 32), readlane_f(x, 48)));
}
__device__ __forceinline__ int wave_min(int x) {
  SV_ROW_REDUCE(int, dpp_i, op_mini, x)
  return min(min(readlane_i(x, 0), readlane_i(x, 16)), min(readlane_i(x, 32), readlane_i(x, 48)));
}
__device__ __forceinline__ int wave_max_int(int x) {
  SV_ROW_REDUCE(int, dpp_i, op_maxi, x)
  return max(max(readlane_i(x, 0), readlane_i(x, 16)), max(readlane_i(x, 32), readlane_i(x, 48)));
}
// Sum in a fixed order (pairwise inside rows, then (r0 + r1) + (r2 + r3)).
__device__ __forceinline__ double wave_sum(double x) {
  SV_ROW_REDUCE(double, dpp_d, op_addd, x)
  return (readlane_d(x, 0) + readlane_d(x, 16)) + (readlane_d(x, 32) + readlane_d(x, 48));
}
// Inclusive prefix sum over lanes: Hillis-Steele inside each row of 16,
// then each row adds the totals of the rows before it.
__device__ __forceinline__ double wave_inclusive_scan(double x) {
  x += dpp_d<kDppRowShr1>(x);
  x += dpp_d<kDppRowShr2>(x);
  x += dpp_d<kDppRowShr4>(x);
  x += dpp_d<kDppRowShr8>(x);
  const double t0 = readlane_d(x, 15), t1 = readlane_d(x, 31), t2 = readlane_d(x, 47);
  const int row = lane_id() >> 4;
  const double off = row == 0 ? 0.0 : row == 1 ? t0 : row == 2 ? t0 + t1 : (t0 + t1) + t2;
  return x + off;
}

// The same for integers.
__device__ __forceinline__ int wave_inclusive_scan_i(int x) {
  x += dpp_i<kDppRowShr1>(x);
  x += dpp_i<kDppRowShr2>(x);
  x += dpp_i<kDppRowShr4>(x);
  x += dpp_i<kDppRowShr8>(x);
  const int t0 = readlane_i(x, 15), t1 = readlane_i(x, 31), t2 = readlane_i(x, 47);
  const int row = lane_id() >> 4;
  const int off = row == 0 ? 0 : row == 1 ? t0 : row == 2 ? t0 + t1 : (t0 + t1) + t2;
  return x + off;
}

// Ranking key of fork candidates: higher logit first, lower id on ties.
// An empty slot is (-inf, kEmptyId): any real element, even at -inf, beats it.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

template <int CTRL>
__device__ __forceinline__ void best_step(float& v, int& i) {
  const float ov = dpp_f<CTRL>(v);
  const int oi = dpp_i<CTRL>(i);
  if (better(ov, oi, v, i)) { v = ov; i = oi; }
}

// Wave-wide best (v, i) by `better`; all lanes get the result.
__device__ __forceinline__ void wave_best(float& v, int& i) {
  best_step<kDppQuadXor1>(v, i);
  best_step<kDppQuadXor2>(v, i);
  best_step<kDppRowHalfMirror>(v, i);
  best_step<kDppRowMirror>(v, i);
  float bv = readlane_f(v, 0);
  int bi = readlane_i(i, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16) {
    const float rv = readlane_f(v, r);
    const int ri = readlane_i(i, r);
    if (better(rv, ri, bv, bi)) { bv = rv; bi = ri; }
  }
  v = bv;
  i = bi;
}

// Sorted per-lane list of the F best candidates (best first).
template <int F>
struct TopList {
  float v[F > 0 ? F : 1];
  int i[F > 0 ? F : 1];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int p = 0; p < (F > 0 ? F : 1); ++p) { v[p] = neg_inf(); i[p] = kEmptyId; }
  }
  __device__ __forceinline__ void insert(float x, int id) {
    if constexpr (F > 0) {
      if (!better(x, id, v[F - 1], i[F - 1])) return;
#pragma unroll
      for (int p = F - 1; p > 0; --p) {
        const bool up = better(x, id, v[p - 1], i[p - 1]);
        const bool here = better(x, id, v[p], i[p]);
        const float nv = up ? v[p - 1] : (here ? x : v[p]);
        const int ni = up ? i[p - 1] : (here ? id : i[p]);
        v[p] = nv;
        i[p] = ni;
      }
      if (better(x, id, v[0], i[0])) { v[0] = x; i[0] = id; }
    }
  }
  __device__ __forceinline__ void pop_front() {
    if constexpr (F > 0) {
#pragma unroll
      for (int p = 0; p + 1 < F; ++p) { v[p] = v[p + 1]; i[p] = i[p + 1]; }
      v[F - 1] = neg_inf();
      i[F - 1] = kEmptyId;
    }
  }
};

// Merges the lanes' lists into the wave's top-f (f <= F); every lane gets
// the result in out (entries past f are left empty).
template <int F>
__device__ __forceinline__ void wave_merge_lists(TopList<F>& mine, int f, TopList<F>& out) {
  out.clear();
  if constexpr (F > 0) {
#pragma unroll
    for (int r = 0; r < F; ++r) {
      if (r < f) {
        float bv = mine.v[0];
        int bi = mine.i[0];
        wave_best(bv, bi);
        out.v[r] = bv;
        out.i[r] = bi;
        if (bi != kEmptyId && mine.i[0] == bi) mine.pop_front();
      }
    }
  }
}

// The f-th largest of the lanes' values (f <= F; -inf if fewer than f lanes
// hold a value above -inf).
template <int F>
__device__ __forceinline__ float wave_fth_largest(float x, int f) {
  float th = neg_inf();
#pragma unroll
  for (int r = 0; r < F; ++r) {
    if (r < f) {
      th = wave_max(x);
      const unsigned long long m = __ballot(x == th);
      const int first = __ffsll((long long)m) - 1;
      if (lane_id() == first) x = neg_inf();
    }
  }
  return th;
}

// The f-th largest of the values the lanes hold (NV each; empty entries
// hold -inf): -inf if fewer than f values exceed it.
template <int NV>
__device__ __forceinline__ float fth_largest_multi(const float (&x0)[NV], int f) {
  float x[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) x[i] = x0[i];
  float th = neg_inf();
  for (int r = 0; r < f; ++r) {
    float lm = x[0];
#pragma unroll
    for (int i = 1; i < NV; ++i) lm = fmaxf(lm, x[i]);
    th = wave_max(lm);
    const unsigned long long m = __ballot(lm == th);
    const int first = __ffsll((long long)m) - 1;
    if (lane_id() == first) {
      bool done = false;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        if (!done && x[i] == th) { x[i] = neg_inf(); done = true; }
      }
    }
  }
  return th;
}

}  // namespace sv
