// libspecverify: the drafter's own draw from its logits rows (gfx950).
//
// Sampling is greedy or stochastic according to the temperature (the
// sampler file highlighted in the tanishqkumar/ssd repository summary,
// thehardwarestore.ai): at temperature 0 the token is the lowest id holding
// the row maximum; above it, the inverse-CDF draw from softmax(x / tau) with
// a caller-supplied uniform, in token-id order (the first t whose running
// sum exceeds u * Z; the last token of positive weight if rounding leaves
// none).
//
// One block of sixteen waves per row.  Each wave streams a contiguous range of
// slabs once, keeping a wave-uniform running maximum as its reference; every
// slab's sum of 2^(x c - hi) is kept in LDS with the reference it was taken
// against.  Wave 0 then rescales the slab sums to the row maximum, finds the
// slab that holds u * Z by a scan in slab order, re-reads that slab and
// finds the lane, then the element.  A row is read once from HBM plus one
// slab.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "specverify.h"
#include "sv_device.h"

namespace sv {
namespace samp {

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * kLanes;
constexpr int kMaxSlabs = 4096;  // 1,048,576 fp32 elements per row
constexpr int kAhead = 8;        // slabs a wave has in flight

struct Lds {
  double s[kMaxSlabs];   // slab sum of 2^(x c - hi[slab])
  float hi[kMaxSlabs];   // slab reference times c, rounded to fp32
  float wm[kWaves];      // each wave's maximum
  int wa[kWaves];        // each wave's lowest id holding it (temperature 0)
};

__device__ __forceinline__ bool tau_valid(float t) { return t >= 0.0f && t < pos_inf(); }

template <typename In>
__device__ __forceinline__ float vmax(const uint4& v) {
  constexpr int VEC = Elem<In>::VEC;
  float m = elem<In>(v, 0);
#pragma unroll
  for (int e = 1; e < VEC; ++e) m = fmaxf(m, elem<In>(v, e));
  return m;
}

// Pairwise fp32 sum of a vector's terms 2^(x c - hi), element order fixed.
template <typename In>
__device__ __forceinline__ float vterms(const uint4& v, float c, float hi, float (&t)[Elem<In>::VEC]) {
  constexpr int VEC = Elem<In>::VEC;
  float a[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    t[e] = __builtin_amdgcn_exp2f(fmaf(elem<In>(v, e), c, -hi));
    a[e] = t[e];
  }
#pragma unroll
  for (int h = VEC / 2; h > 0; h >>= 1) {
#pragma unroll
    for (int e = 0; e < h; ++e) a[e] = a[e] + a[e + h];
  }
  return a[0];
}

template <typename In>
__global__ __launch_bounds__(kThreads) void k_sample(const In* __restrict__ logits, int64_t rows,
                                                      int V, int64_t row_stride,
                                                      const float* __restrict__ tau_in,
                                                      int64_t rows_per_temp,
                                                      const float* __restrict__ uniforms,
                                                      int32_t* __restrict__ tokens) {
  constexpr int VEC = Elem<In>::VEC;
  constexpr int SLAB = slab_elems<In>();
  __shared__ Lds S;
  const int64_t r = blockIdx.x;
  if (r >= rows) return;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const float tau = tau_in[r / rows_per_temp];
  const bool valid_tau = tau_valid(tau);
  const bool greedy = tau == 0.0f;
  const float c = (valid_tau && !greedy) ? (float)(1.4426950408889634074 / (double)tau) : 0.0f;
  const In* row = logits + r * row_stride;
  const int nslab = (V + SLAB - 1) / SLAB;
  const int s0 = (int)((int64_t)w * nslab / kWaves);
  const int s1 = (int)((int64_t)(w + 1) * nslab / kWaves);

  // 1. one pass over this wave's slabs
  float run = neg_inf();  // wave-uniform running maximum
  float lm = neg_inf();   // this lane's maximum and lowest id (temperature 0)
  int la = kEmptyId;
  if (valid_tau) {
    for (int b0 = s0; b0 < s1; b0 += kAhead) {
      uint4 v[kAhead];
#pragma unroll
      for (int q = 0; q < kAhead; ++q) {
        v[q] = make_uint4(Elem<In>::kNegInfWord, Elem<In>::kNegInfWord, Elem<In>::kNegInfWord,
                          Elem<In>::kNegInfWord);
        if (b0 + q < s1) load_vec<In>(row, (b0 + q) * SLAB + lane * VEC, V, v[q]);
      }
#pragma unroll
      for (int q = 0; q < kAhead; ++q) {
        if (b0 + q >= s1) break;
        const int s = b0 + q;
        const float vm = vmax<In>(v[q]);
        if (greedy) {
          if (vm > lm) {
            int first = kEmptyId;
#pragma unroll
            for (int e = 0; e < VEC; ++e)
              if (first == kEmptyId && elem<In>(v[q], e) == vm) first = s * SLAB + lane * VEC + e;
            lm = vm;
            la = first;
          }
          continue;
        }
        run = fmaxf(run, wave_max(vm));
        double sum = 0.0;
        float hi = neg_inf();
        if (run > neg_inf()) {
          hi = run * c;
          float t[VEC];
          sum = wave_sum((double)vterms<In>(v[q], c, hi, t));
        }
        if (lane == 0) {
          S.s[s] = sum;
          S.hi[s] = hi;
        }
      }
    }
  }
  if (greedy) {
    const float m = wave_max(lm);
    const int a = wave_min(lm == m ? la : (int)kEmptyId);
    if (lane == 0) { S.wm[w] = m; S.wa[w] = a; }
  } else if (lane == 0) {
    S.wm[w] = run;
  }
  __syncthreads();
  if (w != 0) return;

  float M = neg_inf();
#pragma unroll
  for (int i = 0; i < kWaves; ++i) M = fmaxf(M, S.wm[i]);
  if (!valid_tau || !finitef(M)) {
    if (lane == 0) tokens[r] = -1;
    return;
  }
  if (greedy) {
    int a = kEmptyId;
#pragma unroll
    for (int i = 0; i < kWaves; ++i)
      if (S.wm[i] == M) a = min(a, S.wa[i]);
    if (lane == 0) tokens[r] = a;
    return;
  }

  // 2. slab weights relative to the row maximum, scanned in slab order (hm
  // is M c rounded to fp32, as the slabs' references are)
  const float hm = __fmul_rn(M, c);
  const double target_u = (double)uniforms[r];
  double Z = 0.0;
  for (int g = 0; g < nslab; g += kLanes) {
    const int s = g + lane;
    double ws = 0.0;
    if (s < nslab && S.hi[s] > neg_inf()) ws = S.s[s] * exp2((double)S.hi[s] - (double)hm);
    Z += wave_sum(ws);
  }
  const double target = target_u * Z;
  int sstar = -1, slast = -1;
  double before = 0.0, before_last = 0.0, carry = 0.0;
  for (int g = 0; g < nslab; g += kLanes) {
    const int s = g + lane;
    double ws = 0.0;
    if (s < nslab && S.hi[s] > neg_inf()) ws = S.s[s] * exp2((double)S.hi[s] - (double)hm);
    const double incl = carry + wave_inclusive_scan(ws);
    double excl = __shfl_up(incl, 1);
    if (lane == 0) excl = carry;
    const unsigned long long hit = __ballot(s < nslab && ws > 0.0 && incl > target);
    if (sstar < 0 && hit) {
      const int l = __ffsll((long long)hit) - 1;
      sstar = g + l;
      before = readlane_d(excl, l);
    }
    const unsigned long long posm = __ballot(s < nslab && ws > 0.0);
    if (posm) {
      const int l = 63 - __clzll((long long)posm);
      slast = g + l;
      before_last = readlane_d(excl, l);
    }
    carry = readlane_d(incl, kLanes - 1);
  }
  if (sstar < 0) { sstar = slast; before = before_last; }
  if (sstar < 0) {  // no positive weight (cannot happen with a finite maximum)
    if (lane == 0) tokens[r] = -1;
    return;
  }

  // 3. the slab again: the lane, then the element
  const float hs = S.hi[sstar];
  const double fac = exp2((double)hs - (double)hm);
  const int e0 = sstar * SLAB + lane * VEC;
  uint4 v = make_uint4(Elem<In>::kNegInfWord, Elem<In>::kNegInfWord, Elem<In>::kNegInfWord,
                       Elem<In>::kNegInfWord);
  load_vec<In>(row, e0, V, v);
  float t[VEC];
  const float lsum = vterms<In>(v, c, hs, t);
  const double lw = (double)lsum * fac;
  const double incl = before + wave_inclusive_scan(lw);
  double excl = __shfl_up(incl, 1);
  if (lane == 0) excl = before;
  int lstar;
  const unsigned long long hit = __ballot(lw > 0.0 && incl > target);
  if (hit) {
    lstar = __ffsll((long long)hit) - 1;
  } else {
    const unsigned long long posm = __ballot(lw > 0.0);
    lstar = posm ? 63 - __clzll((long long)posm) : 0;
  }
  int tk = -1, tlast = -1;
  float acc = 0.0f;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    acc += t[e];
    if (t[e] > 0.0f && e0 + e < V) {
      tlast = e0 + e;
      if (tk < 0 && excl + (double)acc * fac > target) tk = e0 + e;
    }
  }
  const int tok = readlane_i(tk < 0 ? tlast : tk, lstar);
  if (lane == 0) tokens[r] = tok;
}

}  // namespace samp
}  // namespace sv

extern "C" sv_status sv_sample_temp(const void* logits, int32_t dtype, int64_t rows, int32_t V,
                                    int64_t row_stride, const float* temperature,
                                    int64_t rows_per_temp, const float* uniforms,
                                    int32_t* tokens, void* stream) {
  using namespace sv;
  if (rows < 0 || V < 2 || rows_per_temp < 1 || row_stride < V) return SV_ERR_INVALID_ARG;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_INVALID_ARG;
  const int64_t slab = dtype == SV_BF16 ? slab_elems<uint16_t>() : slab_elems<float>();
  if ((V + slab - 1) / slab > samp::kMaxSlabs) return SV_ERR_INVALID_ARG;
  if (rows > 0x7fffffff) return SV_ERR_INVALID_ARG;
  if (rows == 0) return SV_OK;
  if (!logits || !temperature || !uniforms || !tokens) return SV_ERR_INVALID_ARG;
  const int64_t eb = dtype == SV_BF16 ? 2 : 4;
  if (((uintptr_t)logits & 15u) != 0 || (row_stride * eb) % 16 != 0) return SV_ERR_MISALIGNED;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == SV_BF16) {
    hipLaunchKernelGGL(samp::k_sample<uint16_t>, dim3((unsigned)rows), dim3(samp::kThreads), 0, s,
                       (const uint16_t*)logits, rows, V, row_stride, temperature, rows_per_temp,
                       uniforms, tokens);
  } else {
    hipLaunchKernelGGL(samp::k_sample<float>, dim3((unsigned)rows), dim3(samp::kThreads), 0, s,
                       (const float*)logits, rows, V, row_stride, temperature, rows_per_temp,
                       uniforms, tokens);
  }
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}
