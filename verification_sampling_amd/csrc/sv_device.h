// Device-side building blocks of libspecverify (gfx950, wave64).
//
// Layout convention used by every kernel: a logits row is cut into chunks of
// kLanes * kU 16-byte vectors; one wavefront owns one chunk of one row.  Lane
// l holds vectors u = 0..kU-1 at element offsets (u * 64 + l) * VEC inside
// the chunk, so each vector load instruction of the wave reads 1 KiB of
// contiguous memory, and a lane visits its own elements in increasing token
// id order (u outer, element inner).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kLanes = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kLanes * kWavesPerBlock;
constexpr int kU = 8;          // 16-byte vectors per lane per tensor per chunk
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
constexpr int chunk_elems() { return kLanes * kU * Elem<In>::VEC; }

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

// Loads this lane's kU vectors of one chunk.  Elements at or beyond V read
// as -inf; beyond-V memory is never touched (a partial vector is loaded
// element by element).
template <typename In>
__device__ __forceinline__ void load_chunk(const In* __restrict__ row, int64_t cstart,
                                           int V, bool full, uint4 (&raw)[kU]) {
  constexpr int VEC = Elem<In>::VEC;
  const int lane = lane_id();
  if (full) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const In* p = row + cstart + (int64_t)(u * kLanes + lane) * VEC;
      raw[u] = *reinterpret_cast<const uint4*>(p);
    }
  } else {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t e0 = cstart + (int64_t)(u * kLanes + lane) * VEC;
      if (e0 + VEC <= V) {
        raw[u] = *reinterpret_cast<const uint4*>(row + e0);
      } else {
        uint4 v = make_uint4(Elem<In>::kNegInfWord, Elem<In>::kNegInfWord,
                             Elem<In>::kNegInfWord, Elem<In>::kNegInfWord);
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
        raw[u] = v;
      }
    }
  }
}

// ---------------------------------------------------------------- wave ops
// Butterfly reductions: every lane ends with the same value (the operations
// are commutative, so each lane's pairwise tree gives identical bits).

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_max_int(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
// Inclusive prefix sum over lanes (Hillis-Steele), fixed order.
__device__ __forceinline__ double wave_inclusive_scan(double x) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < kLanes; o <<= 1) {
    const double y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Ranking key of fork candidates: higher logit first, lower id on ties.
// An empty slot is (-inf, kEmptyId): any real element, even at -inf, beats it.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// Wave-wide best (v, i) by `better`; all lanes get the result.
__device__ __forceinline__ void wave_best(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o);
    const int oi = __shfl_xor(i, o);
    if (better(ov, oi, v, i)) { v = ov; i = oi; }
  }
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

}  // namespace sv
