// libspecverify: kernels and the C ABI entry points (gfx950).
//
// Kernel chain of sv_verify (one stream, no host synchronisation):
//   k_stats   one round of resident waves; each streams one segment of
//             consecutive slabs of one row (target and draft together,
//             non-temporal 16-byte loads, the next chunk in flight while the
//             current one is folded) and writes the segment's partial
//             statistics: row reference, fp64 sum of exponentials, argmax at
//             temperature 0, and the draft's fork candidates with the
//             drafted token masked out.  No atomics.
//   k_decide  1024-thread blocks, several per sequence: each merges the
//             rows' partials in LDS (row reference and sum, argmax, p(d),
//             q(d)); wave 0 runs the acceptance tests and finds the first
//             rejection by ballot; the owner block writes the outputs; for
//             temperature > 0 the blocks split row n, sum max(0, p - q) (or
//             p) per chunk, hand the chunk totals to the last to arrive
//             (device-scope stores and one arrival counter per sequence;
//             through LDS when one block sums the whole row), and that block
//             draws the token by inverse CDF.  Fork blocks (one per
//             sequence, or one per few rows at small batches) rank the fork
//             candidates beside them.  With forks->hits, whichever of the
//             draw and the fork ranking finishes second writes the
//             speculation-cache lookup (no further launch).
// sv_residual_sample runs k_stats and k_decide at given positions (plus
// k_write for the full residual distributions); sv_softmax_temp runs
// k_stats then k_write; sv_forked_topf runs k_stats then k_decide without
// draws; sv_cache_hit runs k_hits, the lookup alone, on forks from another
// call.
//
// The speculative-sampling rule (accept iff u < min(1, p/q), first
// rejection, draw from max(0, p - q), bonus draw from p_k) follows the
// speculative-sampling project page ("How It Works", "Highlighted
// Details", sourcepulse.org project 1842340) and the exactness requirement
// of "What changes in SSD" (hysenlabs.com editorial); the forked top-f with
// the drafted token masked follows the async-SD utilities file described in
// the tanishqkumar/ssd repository summary (thehardwarestore.ai).

#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <type_traits>

#include "specverify.h"
#include "sv_stream.h"

namespace sv {

// Four resident waves per SIMD: the register budget (128) the folding code
// needs, and enough bytes in flight with the one-chunk prefetch.
#ifndef SV_STATS_WAVES_PER_EU
#define SV_STATS_WAVES_PER_EU 4
#endif

// One wave per (row slot, segment).  The grid is one resident round of
// waves.
template <typename In, int F>
__global__ __launch_bounds__(kBlock)
__attribute__((amdgpu_waves_per_eu(SV_STATS_WAVES_PER_EU))) void k_stats(Params P) {
  __shared__ CandLds<F> s_cand[kWavesPerBlock];
  warm_kernargs();
  const int64_t task = wave_global_id();
  if (task >= P.nslots * P.nparts) return;
  const int64_t slot = task / P.nparts;
  const int seg = (int)(task - slot * P.nparts);
  int b, j;
  slot_to_bj(P, slot, b, j);
  stream_segment<In, F>(P, slot, uniform(b), uniform(j), seg, P.nparts,
                        &s_cand[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)]);
}

// Bounds of an inexact candidate's maximum in logits from its key (see
// inexact_key) and the reciprocal of its scale c: the key's relation
// widened by a margin for the rounding of the terms, the key and this
// product.  A key that is not finite bounds nothing.
template <typename In>
__device__ __forceinline__ void key_bounds(float key, double inv_c, float& lo, float& hi) {
  constexpr double kLowBits = (Elem<In>::VEC == 8) ? 4.0 : 3.0;  // 1 + log2(VEC)
  if (!(finitef(key) && inv_c > 0.0)) { lo = neg_inf(); hi = pos_inf(); return; }
  const double m = 1e-3 + 1e-5 * fabs((double)key);
  lo = (float)(((double)key - kLowBits - m) * inv_c);
  hi = (float)(((double)key + m) * inv_c);
}

// The candidate vectors the segments of row (b, j) passed on (cnt: this
// lane's segment's count, lanes < np), a round of 64 * kRound at a time:
// their positions and keys are loaded first.  A candidate's key is its
// maximum, or for an inexact one a key that bounds the maximum from both
// sides (key_bounds).  The f-th largest of the lower bounds (f distinct
// elements reach it, so it is a lower bound of the row's f-th best) raises
// the threshold kv.  Only the vectors whose upper bound reaches kv are
// re-read; their elements (id < V, id != mask_id) at or above kv go into
// this lane's list.  With nhalf = 2, two waves share the row: wave `half`
// takes every other round.
template <typename In, int F>
__device__ __forceinline__ void fork_candidates(const Params& P, int b, int j, int64_t base,
                                                int np, int cnt, int mask_id, int half,
                                                int nhalf, double cd, TopList<F>& mine) {
  if constexpr (F > 0) {
    constexpr int VEC = Elem<In>::VEC;
    constexpr int kRound = 4;
    const int lane = lane_id();
    const int mycnt = lane < np ? cnt : 0;
    const int incl = wave_inclusive_scan_i(mycnt);
    const int total = readlane_i(incl, kLanes - 1);
    const In* drow = drow_ptr<In>(P, b, j);
    const int V = P.V;
    const double inv_c = cd > 0.0 ? 1.0 / cd : 0.0;
    float kv = neg_inf();
    for (int t0 = half * kLanes * kRound; t0 < total; t0 += nhalf * kLanes * kRound) {
      int pos[kRound];
      float vm[kRound];
#pragma unroll
      for (int q = 0; q < kRound; ++q) {
        const int t = t0 + q * kLanes + lane;
        // segment holding flat index t: the first g < np with incl[g] > t.
        // Few segments: a scan of lane reads; many (small batches): a
        // binary search over the lanes' running counts.  The cross-lane
        // reads run with every lane active (a read from an inactive lane
        // returns 0).
        int lo = 0;
        if (np <= 16) {
          for (int g = 0; g < np; ++g) lo += (readlane_i(incl, g) <= t) ? 1 : 0;
        } else {
          int hi = np;
#pragma unroll
          for (int it = 0; it < 7; ++it) {  // np <= 64
            const int mid = (lo + hi) >> 1;
            const int v = __shfl(incl, min(mid, kLanes - 1));
            if (lo < hi) {
              if (v <= t) lo = mid + 1;
              else hi = mid;
            }
          }
        }
        const int seg = min(lo, np - 1);
        const int before = __shfl(incl, seg) - __shfl(mycnt, seg);
        pos[q] = -1;
        vm[q] = neg_inf();
        if (t < total) {
          const int64_t e = (base + seg) * kDumpCap + (t - before);
          pos[q] = P.ws.cpos[e];
          vm[q] = P.ws.cvm[e];
        }
      }
      float lo[kRound], up[kRound];
#pragma unroll
      for (int q = 0; q < kRound; ++q) {
        lo[q] = up[q] = vm[q];
        if (pos[q] >= 0 && (pos[q] & kCandInexact)) key_bounds<In>(vm[q], inv_c, lo[q], up[q]);
      }
      kv = fmaxf(kv, fth_largest_multi<kRound>(lo, P.f));
      // the round's re-reads are all issued before the first is ranked
      int p0[kRound];
      uint4 v[kRound];
#pragma unroll
      for (int q = 0; q < kRound; ++q) {
        p0[q] = (pos[q] >= 0 && up[q] >= kv) ? (pos[q] & ~kCandInexact) : -1;
        v[q] = make_uint4(Elem<In>::kNegInfWord, Elem<In>::kNegInfWord, Elem<In>::kNegInfWord,
                          Elem<In>::kNegInfWord);
        if (p0[q] >= 0) load_vec<In>(drow, p0[q], V, v[q]);
      }
#pragma unroll
      for (int q = 0; q < kRound; ++q) {
        if (!__ballot(p0[q] >= 0)) continue;
        float thr = fmaxf(kv, mine.v[F - 1]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float x = elem<In>(v[q], e);
          const int id = p0[q] + e;
          if (p0[q] >= 0 && id < V && id != mask_id && x >= thr) {
            mine.insert(x, id);
            thr = fmaxf(kv, mine.v[F - 1]);
          }
        }
      }
    }
  }
}

// A row's merged statistics (LDS, one per row of the sequence).
struct RowStat {
  float tm; int targ; double ts;   // target reference, argmax, sum
  float dm; int darg; double ds;   // draft (unmasked row)
  float qm; double qs;             // draft with the drafted token masked (forks)
  double pd, qd;                   // p(d), q(d) for j < k
  int valid;
  int ftok[kMaxF];                 // forks (f entries)
  float fprob[kMaxF];
};

// The row's forks: the top-f of the segments' lists and of the candidate
// vectors they passed on, with masked-softmax probabilities at tau
// (2^((v - m') c) / S', (1, 0, ...) at temperature 0); lane r < f gets entry
// r in (tok, prob).  With nhalf = 2 this wave ranks its half of the
// candidates (the segments' lists go to half 0) and top is that half's
// top-f, to be merged with the other half's.
template <typename In, int F>
__device__ __forceinline__ void fork_top(const Params& P, int b, int j, const RowPlan& pl,
                                         const float (&lv)[F > 0 ? F : 1],
                                         const int (&li)[F > 0 ? F : 1], int cnt, float qm,
                                         double qs, double cd, int half, int nhalf,
                                         TopList<F>& top, int& tok, float& prob) {
  const int lane = lane_id();
  tok = kEmptyId;
  prob = 0.0f;
  if constexpr (F > 0) {
    TopList<F> mine;
    mine.clear();
    if (half == 0) {
#pragma unroll
      for (int r = 0; r < F; ++r) mine.insert(lv[r], li[r]);
    }
    fork_candidates<In, F>(P, b, j, slot_of(P, b, j) * kMaxSeg, P.nparts, cnt, pl.mask_id, half,
                           nhalf, cd, mine);
    wave_merge_lists<F>(mine, P.f, top);
    float v = neg_inf();
#pragma unroll
    for (int r = 0; r < F; ++r) {
      if (lane == r) { v = top.v[r]; tok = top.i[r]; }
    }
    if (pl.greedy) prob = (lane == 0) ? 1.0f : 0.0f;
    else if (!finitef(qm) || !(v > neg_inf())) prob = 0.0f;
    else prob = (float)(exp2(((double)v - (double)qm) * cd) / qs);
  }
}

// Merges the partials of row (b, j) into rs (written by lanes 0..f-1 and
// lane 0).  One wave; every load is issued before the first is used (the
// partials, the fork lists and the drafted token's logits as seen by
// k_stats are loaded whether or not the row needs them).  With nhalf = 2
// two waves share the row's forks: both merge the statistics, half 0
// writes rs, and each writes its half's top-f list to (hv, hi).
template <typename In, int F>
__device__ __forceinline__ void row_stat(const Params& P, int b, int j, float tau, RowStat* rs,
                                         bool forks_now, int half = 0, int nhalf = 1,
                                         float* hv = nullptr, int* hi = nullptr) {
  const int lane = lane_id();
  const Ws& W = P.ws;
  const int k = P.k;
  const int np = P.nparts;
  const int64_t slot = slot_of(P, b, j);
  const int64_t base = slot * kMaxSeg;
  const float nan = __uint_as_float(0x7fc00000u);

  float tmi = neg_inf(), dmi = neg_inf();
  double tsi = 0.0, dsi = 0.0;
  int tai = kEmptyId, dai = kEmptyId;
  float lv[F > 0 ? F : 1];
  int li[F > 0 ? F : 1];
#pragma unroll
  for (int r = 0; r < (F > 0 ? F : 1); ++r) { lv[r] = neg_inf(); li[r] = kEmptyId; }
  int cnt = 0;
  if (lane < np) {
    const int64_t e = base + lane;
    tmi = W.tm[e]; tsi = W.ts[e]; tai = W.targ[e];
    dmi = W.dm[e]; dsi = W.ds[e]; dai = W.darg[e];
    if constexpr (F > 0) {
#pragma unroll
      for (int r = 0; r < F; ++r) { lv[r] = W.dtv[e * F + r]; li[r] = W.dti[e * F + r]; }
      cnt = W.cn[e];
    }
  }
  const float xd = W.xd[slot], yd = W.yd[slot];

  const RowPlan pl = plan_row(P, b, j, tau);
  const float c = pl.greedy ? 0.0f : scale_of(tau);
  const double cd = (double)c;
  const int d = (int)pl.d_id;
  const bool d_ok = pl.d_id >= 0 && pl.d_id < P.V;
  if (!pl.readT) { tmi = neg_inf(); tsi = 0.0; tai = kEmptyId; }
  if (!pl.readD) { dmi = neg_inf(); dsi = 0.0; dai = kEmptyId; }

  float tm = neg_inf(), dm = neg_inf();
  int targ = kEmptyId, darg = kEmptyId;
  double ts = 0.0, ds = 0.0, pd = nan, qd = nan;
  bool valid = pl.tok && pl.pos_ok;

  if (pl.readT) {
    const Merged t = merge_lanes(tmi, tsi, tai, pl.greedy, cd);
    tm = t.m; ts = t.s; targ = t.arg;
    valid = valid && finitef(t.m);
  }

  TopList<F> top;
  top.clear();
  if (pl.readD) {
    const Merged q = merge_lanes(dmi, dsi, dai, pl.greedy, cd);
    if (lane == 0 && half == 0) { rs->qm = q.m; rs->qs = q.s; }
    if (pl.topf) {
      if constexpr (F > 0) {
        if (forks_now) {
          int tok;
          float prob;
          fork_top<In, F>(P, b, j, pl, lv, li, cnt, q.m, q.s, cd, half, nhalf, top, tok, prob);
          if (nhalf > 1) {
#pragma unroll
            for (int r = 0; r < F; ++r) {
              if (lane == r && r < P.f) { hv[r] = top.v[r]; hi[r] = top.i[r]; }
            }
          } else if (lane < P.f) {
            rs->ftok[lane] = tok;
            rs->fprob[lane] = prob;
          }
        }
      }
      if (j < k) {
        // unmasked draft statistics from the masked ones and y_d
        if (d_ok) {
          const float mfull = fmaxf(q.m, yd);
          dm = mfull;
          if (!pl.greedy && finitef(mfull)) {
            double s = exp2(((double)yd - (double)mfull) * cd);
            if (q.m > neg_inf()) s += q.s * exp2(((double)q.m - (double)mfull) * cd);
            ds = s;
          }
          darg = better(yd, d, top.v[0], top.i[0]) ? d : top.i[0];
        }
        valid = valid && d_ok && finitef(dm);
      } else {
        dm = q.m; ds = q.s; darg = top.i[0];
        valid = valid && finitef(q.m);
      }
    } else {
      dm = q.m; ds = q.s; darg = q.arg;
      valid = valid && finitef(q.m);
    }
  }

  // p(d), q(d) for the acceptance test and the optional outputs
  if (P.mode == kVerify && j < k) {
    valid = valid && d_ok;
    if (valid) {
      if (pl.greedy) {
        pd = (d == targ) ? 1.0 : 0.0;
        qd = pl.readD ? ((d == darg) ? 1.0 : 0.0) : (double)nan;
      } else {
        pd = exp2(((double)xd - (double)tm) * cd) / ts;
        qd = exp2(((double)yd - (double)dm) * cd) / ds;
      }
    }
  }
  if (lane == 0 && half == 0) {
    rs->tm = tm; rs->targ = targ; rs->ts = ts;
    rs->dm = dm; rs->darg = darg; rs->ds = ds;
    rs->pd = pd; rs->qd = qd;
    rs->valid = valid ? 1 : 0;
  }
}

// ================================================================ k_decide

constexpr int kDecideWaves = 16;
constexpr int kDecideBlock = kDecideWaves * kLanes;

struct DecideLds {
  RowStat rs[kMaxK + 1];
  float hv[kMaxK + 1][2][kMaxF];  // fork blocks: each half's top-f per row
  int hi[kMaxK + 1][2][kMaxF];
  float wv[kDecideWaves][kMaxF];  // split fork blocks: each wave's top-f
  int wi[kDecideWaves][kMaxF];
  double ct[kTotRegs * kLanes];   // chunk totals, when one block sums the whole row
  ResidCoef kc;                   // coefficients of the row to sum (decision wave)
  int n, status;
};

// Wave 0 of a k_decide block: validity, acceptance tests, first rejection
// (ballot over positions) and, when write_outputs, the per-sequence outputs.
// Returns the outcome position n and the status (0 error, 1 finished,
// 2 draw pending).
// The per-sequence inputs of the decision, loaded by wave 0 at the start of
// the kernel so that they arrive together with the row partials: lane j < k
// holds the drafted token and the acceptance uniform of position j.
struct SeqIn {
  float tau;
  int d;
  float ua;
  int pos;
};

__device__ __forceinline__ SeqIn load_seq_inputs(const Params& P, int b) {
  const int lane = lane_id();
  SeqIn in;
  in.tau = P.tau[b];
  in.d = 0;
  in.ua = 0.0f;
  in.pos = -1;
  if (lane < P.k) {
    in.d = P.drafts[(int64_t)b * P.k + lane];
    if (P.mode == kVerify) in.ua = P.u_acc[(int64_t)b * P.k + lane];
  }
  if (P.mode == kResidual) in.pos = P.position[b];
  return in;
}

__device__ __forceinline__ void decide_sequence(const Params& P, int b, const DecideLds& S,
                                                const SeqIn& in, bool write_outputs, int& n_out,
                                                int& status) {
  const int lane = lane_id();
  const int k = P.k;
  const int K1 = k + 1;
  const float tau = in.tau;
  const bool tok = tau_ok(tau);
  const bool greedy = tau == 0.0f;

  bool ok = tok;
  int d = 0;
  if (lane < k) {
    d = in.d;
    if (d < 0 || d >= P.V) ok = false;
  }
  int pos = -1;
  if (P.mode == kResidual) {
    pos = in.pos;
    if (pos < 0 || pos > k) ok = false;
  }
  // rows read are valid
  if (P.mode == kResidual && !P.rows_all) {
    if (lane == 0 && pos >= 0 && pos <= k && !S.rs[pos].valid) ok = false;
  } else if (lane < K1) {
    if (!S.rs[lane].valid) ok = false;
  }
  const bool seq_ok = __ballot(!ok) == 0ull;

  n_out = 0;
  status = 0;
  if (!seq_ok) {
    if (write_outputs) write_seq_error(P, b);
    return;
  }
  if (P.mode == kVerify) {
    bool acc = true;
    if (lane < k) {
      const RowStat& r = S.rs[lane];
      if (greedy) {
        acc = (d == r.targ);
      } else {
        // a = min(1, p/q); q = 0: a = 1 if p > 0 else 0.  Accept iff u < a.
        const double p = r.pd, q = r.qd;
        const double a = (q == 0.0) ? (p > 0.0 ? 1.0 : 0.0) : fmin(1.0, p / q);
        acc = (double)in.ua < a;
      }
      if (write_outputs) {
        if (P.p_draft) P.p_draft[(int64_t)b * k + lane] = (float)r.pd;
        if (P.q_draft) P.q_draft[(int64_t)b * k + lane] = (float)r.qd;
      }
    }
    const unsigned long long rej = __ballot(lane < k && !acc);
    const int n = rej ? (__ffsll((long long)rej) - 1) : k;
    n_out = n;
    if (write_outputs && lane == 0) st_dev(P.accept_len + b, n);
    if (greedy) {
      status = 1;
      if (write_outputs && lane == 0) st_dev(P.out_token + b, S.rs[n].targ);
    } else {
      status = 2;
    }
  } else if (P.mode == kResidual) {
    n_out = pos;
    if (greedy) {
      status = 1;
      if (write_outputs && lane == 0) st_dev(P.out_token + b, S.rs[pos].targ);
    } else {
      status = 2;
    }
  } else {
    status = 1;
  }
}

// Speculation-cache lookup of sequence b, once its outcome and its forks
// are written (device-scope loads: they may come from other blocks): the
// index of the outcome token among the forks of the outcome position, else
// -1.  One wave.
__device__ __forceinline__ void write_hit(const Params& P, int b) {
  const int lane = lane_id();
  const int K1 = P.k + 1;
  const int n = uniform(ld_dev(P.accept_len + b));
  const int t = uniform(ld_dev(P.out_token + b));
  int hit = -1;
  if (n >= 0 && n <= P.k && t >= 0) {
    int tok = -1;
    if (lane < P.f) tok = ld_dev(P.fork_tok + ((int64_t)b * K1 + n) * P.f + lane);
    const unsigned long long m = __ballot(lane < P.f && tok == t);
    hit = m ? (__ffsll((long long)m) - 1) : -1;
  }
  if (lane == 0) P.hits[b] = hit;
}

// One of the lookup's two inputs of sequence b (the drawn token, or the
// forks ranked beside the draw) has been written by the calling block, all
// of whose waves have waited for their stores; the second arrival writes
// the lookup.  One wave.
__device__ __forceinline__ void hit_input_ready(const Params& P, int b) {
  if (!P.hits) return;
  if (arrive_last(seq_ctr(P.ws, b, kCtrHits), 2u)) write_hit(P, b);
}

// P.nbs blocks per task row: a task row is a sequence (verify, forks,
// residual at given positions) or a (sequence, position) pair (residual with
// full distributions).  Every block of a task merges the rows' partials and
// decides the sequence (block 0 writes the outputs); for a draw at
// temperature > 0 the blocks split the chunks of the row to sum, publish
// the chunk totals with device-scope stores, and the last block to arrive
// draws the token.
template <typename In, int F>
__global__ __launch_bounds__(kDecideBlock) void k_decide(Params P) {
  __shared__ DecideLds S;
  warm_kernargs();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int K1 = P.k + 1;
  const int64_t ntasks = (P.mode == kResidual && P.rows_all) ? (int64_t)P.B * K1 : P.B;
  if ((int64_t)blockIdx.x >= ntasks * P.nbs && P.fsplit > 1) {
    // a split fork block (small batches): fork block r of the sequence ranks
    // rows r, r + fsplit, ... with nsplit waves each, after a merge-only
    // pass over every row that gives the decision its validity flags
    const int fb = (int)(blockIdx.x - ntasks * P.nbs);
    const int b = fb / P.fsplit;
    const int r0 = fb - b * P.fsplit;
    const float tau = P.tau[b];
    if (!(tau > 0.0f && tau_ok(tau))) return;  // the owner block ranks these
    SeqIn sin;
    if (w == 0) sin = load_seq_inputs(P, b);
    for (int j = w; j < K1; j += kDecideWaves) row_stat<In, F>(P, b, j, tau, &S.rs[j], false);
    __syncthreads();
    const int rpb = (K1 - r0 + P.fsplit - 1) / P.fsplit;  // rows of this block, >= 1
    const int nsplit = min(kDecideWaves / rpb, kLanes / P.f);
    if (w < rpb * nsplit) {
      const int jj = w % rpb, h = w / rpb;
      const int j = r0 + jj * P.fsplit;
      row_stat<In, F>(P, b, j, tau, &S.rs[j], true, h, nsplit, S.wv[w], S.wi[w]);
    }
    __syncthreads();
    if (w == 0) {
      int n, status;
      decide_sequence(P, b, S, sin, false, n, status);
      if (lane == 0) S.status = status;
    }
    __syncthreads();
    if (S.status == 0) return;
    if constexpr (F > 0) {
      if (w < rpb) {
        // the row's nsplit lists merged (lane h * f + r holds entry r of
        // the list of wave h * rpb + w)
        const int j = r0 + w * P.fsplit;
        TopList<F> l, top;
        l.clear();
        if (lane < nsplit * P.f) {
          const int h = lane / P.f, r = lane - h * P.f;
          l.insert(S.wv[h * rpb + w][r], S.wi[h * rpb + w][r]);
        }
        wave_merge_lists<F>(l, P.f, top);
        const float qm = S.rs[j].qm;
        const double qs = S.rs[j].qs;
        const double cd = (double)scale_of(tau);
#pragma unroll
        for (int r = 0; r < F; ++r) {
          if (lane == r && r < P.f) {
            const float v = top.v[r];
            const float prob = (!finitef(qm) || !(v > neg_inf()))
                                   ? 0.0f
                                   : (float)(exp2(((double)v - (double)qm) * cd) / qs);
            const int64_t o = ((int64_t)b * K1 + j) * P.f + r;
            st_dev(P.fork_tok + o, top.i[r]);
            if (P.fork_prob) P.fork_prob[o] = prob;
          }
        }
      }
    }
    if (P.hits) {
      // the sequence's last fork block to finish hands its forks to the lookup
      vm_complete();
      __syncthreads();
      if (w == 0 && arrive_last(seq_ctr(P.ws, b, kCtrForks), (unsigned)P.fsplit))
        hit_input_ready(P, b);
    }
    return;
  }
  if ((int64_t)blockIdx.x >= ntasks * P.nbs) {
    // a fork block: the forks of one sequence at temperature > 0, ranked
    // beside the blocks that sum and draw
    const int b = (int)(blockIdx.x - ntasks * P.nbs);
    const float tau = P.tau[b];
    if (!(tau > 0.0f && tau_ok(tau))) return;  // the owner block ranks these
    // two waves per row when the block has them: wave t ranks half t / K1
    // of row t % K1's candidates
    const int nhalf = (2 * K1 <= kDecideWaves) ? 2 : 1;
    SeqIn sin;
    if (w == 0) sin = load_seq_inputs(P, b);
    for (int t = w; t < K1 * nhalf; t += kDecideWaves) {
      const int j = t % K1, h = t / K1;
      row_stat<In, F>(P, b, j, tau, &S.rs[j], true, h, nhalf, S.hv[j][h], S.hi[j][h]);
    }
    __syncthreads();
    if (w == 0) {
      int n, status;
      decide_sequence(P, b, S, sin, false, n, status);
      if (lane == 0) S.status = status;
    }
    __syncthreads();
    if (S.status == 0) return;
    for (int j = w; j < K1; j += kDecideWaves) {
      if constexpr (F > 0) {
        if (nhalf > 1) {
          // the two halves' lists merged (lane h * f + r holds entry r of half h)
          TopList<F> l, top;
          l.clear();
          if (lane < 2 * P.f) {
            const int h = lane / P.f, r = lane - h * P.f;
            l.insert(S.hv[j][h][r], S.hi[j][h][r]);
          }
          wave_merge_lists<F>(l, P.f, top);
          const float qm = S.rs[j].qm;
          const double qs = S.rs[j].qs;
          const double cd = (double)scale_of(tau);
#pragma unroll
          for (int r = 0; r < F; ++r) {
            if (lane == r && r < P.f) {
              const float v = top.v[r];
              const float prob = (!finitef(qm) || !(v > neg_inf()))
                                     ? 0.0f
                                     : (float)(exp2(((double)v - (double)qm) * cd) / qs);
              const int64_t o = ((int64_t)b * K1 + j) * P.f + r;
              st_dev(P.fork_tok + o, top.i[r]);
              if (P.fork_prob) P.fork_prob[o] = prob;
            }
          }
          continue;
        }
      }
      if (lane < P.f) {
        const int64_t o = ((int64_t)b * K1 + j) * P.f + lane;
        st_dev(P.fork_tok + o, S.rs[j].ftok[lane]);
        if (P.fork_prob) P.fork_prob[o] = S.rs[j].fprob[lane];
      }
    }
    if (P.hits) {
      vm_complete();
      __syncthreads();
      if (w == 0) hit_input_ready(P, b);
    }
    return;
  }
  const int64_t task = blockIdx.x / P.nbs;
  const int part = (int)(blockIdx.x - task * P.nbs);
  int b, jt;  // sequence, and the task's own row in the full-residual mode
  if (P.mode == kResidual && P.rows_all) {
    b = (int)(task / K1);
    jt = (int)(task - (int64_t)b * K1);
  } else {
    b = (int)task;
    jt = -1;
  }
  const float tau = P.tau[b];
  const bool owner = jt <= 0 && part == 0;  // writes the per-sequence outputs

  // 1. row statistics, one wave per row.  Forks are ranked here by the
  // owner at temperature 0 (the greedy q(d) needs the draft's top-1) and for
  // the forks-only call; at temperature > 0 fork blocks of their own do.
  const bool forks_now = owner && (P.mode == kForks || !(tau > 0.0f && tau_ok(tau)));
  SeqIn sin;
  if (w == 0) sin = load_seq_inputs(P, b);
  if (P.mode == kResidual && !P.rows_all) {
    if (w == 0) {
      const int pos = P.position[b];
      if (pos >= 0 && pos <= P.k) row_stat<In, F>(P, b, pos, tau, &S.rs[pos], false);
    }
  } else {
    for (int j = w; j < K1; j += kDecideWaves) row_stat<In, F>(P, b, j, tau, &S.rs[j], forks_now);
  }
  __syncthreads();

  // 2. decision; for a draw, the decision wave also works out the
  // coefficients of the row to sum (fp64), once for the block
  if (w == 0) {
    int n, status;
    decide_sequence(P, b, S, sin, owner, n, status);
    if (lane == 0) { S.n = n; S.status = status; }
    if (owner && lane == 0) { P.ws.seqs[b].n = n; P.ws.seqs[b].status = status; }
    if (status == 2 && P.mode != kForks) {
      const int jr = (jt >= 0) ? jt : n;
      const RowStat& R = S.rs[jr];
      const ResidCoef kc = resid_coef(R.tm, R.ts, R.dm, R.ds, scale_of(tau), jr < P.k);
      if (lane == 0) S.kc = kc;
    }
  }
  __syncthreads();
  const int n = S.n;
  const int status = S.status;

  // 3. forks ranked in step 1
  if (forks_now && status != 0 && P.fork_tok) {
    for (int j = w; j < K1; j += kDecideWaves) {
      if (lane < P.f) {
        const int64_t o = ((int64_t)b * K1 + j) * P.f + lane;
        st_dev(P.fork_tok + o, S.rs[j].ftok[lane]);
        if (P.fork_prob) P.fork_prob[o] = S.rs[j].fprob[lane];
      }
    }
  }
  if (owner && P.hits && status != 2) {
    // greedy or error: the owner wrote the token and the forks (-1 for an
    // error sequence) itself
    vm_complete();
    __syncthreads();
    if (w == 0) write_hit(P, b);
  }
  if (status != 2 || P.mode == kForks) return;

  // 4. this block's chunks of the row to sum: n (verify, residual at a
  // position) or the task's row
  const int jr = (jt >= 0) ? jt : n;
  const bool draw_row = (jt < 0) || (jt == n);
  const bool has_q = jr < P.k;
  const RowStat& R = S.rs[jr];
  const ResidCoef kc = S.kc;
  const In* trow = trow_ptr<In>(P, b, jr);
  const In* drow = has_q ? drow_ptr<In>(P, b, jr) : nullptr;
  double* ctr = P.ws.ctr + task * (int64_t)P.cpr;
  // a row summed by this block alone hands its chunk totals over in LDS
  const bool in_lds = P.nbs == 1 && P.cpr <= kTotRegs * kLanes;
  {
    constexpr int VEC = Elem<In>::VEC;
    constexpr int64_t SLAB = slab_elems<In>();
    // the block's chunks [b0, b1) (32-bit: cpr * nbs is far below 2^31)
    const int b0 = part * P.cpr / P.nbs;
    const int b1 = (part + 1) * P.cpr / P.nbs;
    const int64_t slim = (int64_t)P.V / SLAB;
    uint4 ta[kU], da[kU], tb[kU], db[kU];
    auto load = [&](uint4 (&t)[kU], uint4 (&d)[kU], int ch) {
      const int64_t sl = (int64_t)ch * kU;
      const int nv = (int)min<int64_t>(kU, (int64_t)P.nslab - sl);
      const bool full = sl + kU <= slim;
      const int eb = (int)(sl * SLAB) + lane * VEC;
      load_chunk<In>(trow, eb, nv, P.V, full, t);
      if (has_q) {
        load_chunk<In>(drow, eb, nv, P.V, full, d);
      } else {
#pragma unroll
        for (int u = 0; u < kU; ++u) d[u] = make_uint4(0, 0, 0, 0);
      }
    };
    auto sum = [&](const uint4 (&t)[kU], const uint4 (&d)[kU], int ch) {
      const double cr = wave_sum(chunk_rsum<In>(kc, t, d));
      if (lane == 0) {
        if (in_lds) S.ct[ch] = cr;
        else st_dev(ctr + ch, cr);
      }
    };
    // dealt to the waves in turn (wave w takes b0 + w, b0 + w + 16, ...):
    // consecutive waves sit on different SIMDs, so a block with fewer
    // chunks than waves spreads its sums (VALU-heavy: two exponentials per
    // element) over all four SIMDs.  Each chunk's total does not depend on
    // which wave sums it.
    constexpr int kStep = kDecideWaves;
    int ch = b0 + w;
    if (ch < b1) {
      load(ta, da, ch);
      if (ch + kStep < b1) load(tb, db, ch + kStep);
      sum(ta, da, ch);
      for (ch += kStep; ch < b1; ch += 2 * kStep) {
        if (ch + kStep < b1) load(ta, da, ch + kStep);
        sum(tb, db, ch);
        if (ch + kStep >= b1) break;
        if (ch + 2 * kStep < b1) load(tb, db, ch + 2 * kStep);
        sum(ta, da, ch + kStep);
      }
    }
  }
  if (!in_lds) vm_complete();
  __syncthreads();
  if (w != 0) return;
  if (!in_lds) {
    unsigned* ctr_arrive = (P.mode == kResidual && P.rows_all) ? row_ctr(P.ws, task)
                                                                : seq_ctr(P.ws, task, kCtrDraw);
    if (!arrive_last(ctr_arrive, (unsigned)P.nbs)) return;
  }

  // 5. the last block: totals (chunk order) and the draw
  double z = 0.0;
  double tc[kTotRegs];  // chunk totals g * 64 + lane, for rows of up to 64 * kTotRegs chunks
#pragma unroll
  for (int g = 0; g < kTotRegs; ++g) {
    const int ch = g * kLanes + lane;
    tc[g] = (ch < P.cpr) ? (in_lds ? S.ct[ch] : ld_dev(ctr + ch)) : 0.0;
  }
  if (P.cpr <= kTotRegs * kLanes) {
#pragma unroll
    for (int g = 0; g < kTotRegs; ++g) z += wave_sum(tc[g]);
  } else {
    for (int g = 0; g < P.cpr; g += kLanes) z += wave_sum(g + lane < P.cpr ? ld_dev(ctr + g + lane) : 0.0);
  }
  if (P.mode == kResidual && P.rows_all && lane == 0) {
    RowRec rr;
    rr.tm = R.tm; rr.targ = R.targ; rr.ts = R.ts;
    rr.dm = R.dm; rr.ds = R.ds; rr.valid = R.valid;
    rr.zr = z;
    P.ws.rows[(int64_t)b * K1 + jr] = rr;
  }
  if (!draw_row) return;
  ResidCoef kd = kc;
  if (!(z > 0.0)) {
    // a residual of total zero (p = q throughout): draw from p_n; its chunk
    // totals are summed here, one chunk at a time
    kd.has_q = false;
    z = 0.0;
    for (int ch = 0; ch < P.cpr; ++ch) {
      uint4 t[kU], d[kU];
      const int sl = ch * kU;
      const int nv = min(kU, P.nslab - sl);
      load_chunk<In>(trow, sl * (int)slab_elems<In>() + lane * Elem<In>::VEC, nv, P.V, false, t);
#pragma unroll
      for (int u = 0; u < kU; ++u) d[u] = make_uint4(0, 0, 0, 0);
      const double cr = wave_sum(chunk_rsum<In>(kd, t, d));
      if (lane == 0) st_dev(ctr + ch, cr);
      z += cr;
      if (ch < kTotRegs * kLanes) {
#pragma unroll
        for (int g = 0; g < kTotRegs; ++g)
          if (g * kLanes + lane == ch) tc[g] = cr;
      }
    }
    vm_complete();
  }
  const int tok = resid_draw<In>(P, ctr, tc, trow, drow, kd, z,
                                 (double)P.u_rec[(int64_t)b * K1 + jr]);
  if (lane == 0) st_dev(P.out_token + b, tok);
  if (P.hits) {
    vm_complete();
    hit_input_ready(P, b);
  }
}

// ================================================================ k_write

// Normalised outputs, one wave per chunk of a row: softmax rows
// (sv_softmax_temp; the wave merges its row's partials) or residual
// distributions (sv_residual_sample; from the records of k_decide).
template <typename In>
__global__ __launch_bounds__(kBlock) void k_write(Params P) {
  constexpr int VEC = Elem<In>::VEC;
  constexpr int64_t SLAB = slab_elems<In>();
  const int64_t task = wave_global_id();
  const int64_t nslots = (P.mode == kSoftmax) ? P.nslots : (int64_t)P.B * (P.k + 1);
  if (task >= nslots * P.cpr) return;
  const int64_t slot = task / P.cpr;
  const int chunk = (int)(task - slot * P.cpr);
  const int lane = lane_id();
  const float nan = __uint_as_float(0x7fc00000u);

  int b, j;
  float tau;
  if (P.mode == kSoftmax) {
    b = (int)slot; j = 0;
    tau = P.tau[slot / P.rows_per_temp];
  } else {
    b = (int)(slot / (P.k + 1));
    j = (int)(slot - (int64_t)b * (P.k + 1));
    tau = P.tau[b];
  }
  b = uniform(b); j = uniform(j);
  const int64_t sl = (int64_t)chunk * kU;
  const int nv = (int)min<int64_t>(kU, (int64_t)P.nslab - sl);
  const bool full = sl + kU <= (int64_t)P.V / SLAB;
  const int eb = (int)(sl * SLAB) + lane * VEC;
  // the chunk's loads go out before the row's statistics are merged or
  // read (they do not depend on them), whenever the temperature asks for
  // values
  const bool has_q = (P.mode == kResidual) && j < P.k;
  uint4 traw[kU], draw[kU];
  if (tau > 0.0f && tau_ok(tau)) {
    const In* tr = (P.mode == kSoftmax) ? reinterpret_cast<const In*>(P.T) + slot * P.t_row
                                        : trow_ptr<In>(P, b, j);
    load_chunk<In>(tr, eb, nv, P.V, full, traw);
    if (has_q) load_chunk<In>(drow_ptr<In>(P, b, j), eb, nv, P.V, full, draw);
  }

  float* orow;
  int state;  // 0 NaN, 1 one-hot, 2 values
  float tm, dm = 0.0f;
  double ts, ds = 1.0, zr = 0.0;
  int targ;
  if (P.mode == kSoftmax) {
    orow = P.out + slot * P.out_row;
    const bool greedy = tau == 0.0f || !tau_ok(tau);
    const Merged t = merge_partials(P.ws.tm, P.ws.ts, P.ws.targ, slot * kMaxSeg, P.nparts, greedy,
                                    greedy ? 0.0 : (double)scale_of(tau));
    tm = t.m; ts = t.s; targ = t.arg;
    state = (!tau_ok(tau) || !finitef(t.m)) ? 0 : (tau == 0.0f ? 1 : 2);
  } else {
    orow = P.out + (int64_t)b * P.out_seq + (int64_t)j * P.out_row;
    const int st = P.ws.seqs[b].status;
    state = (st == 0) ? 0 : (tau == 0.0f ? 1 : 2);
    if (state == 2) {
      const RowRec& rr = P.ws.rows[slot];
      tm = rr.tm; ts = rr.ts; targ = rr.targ;
      dm = rr.dm; ds = rr.ds; zr = rr.zr;
    } else {
      // greedy rows were not merged by k_decide: the argmax comes from the
      // partials
      const Merged t = merge_partials(P.ws.tm, P.ws.ts, P.ws.targ, slot * kMaxSeg, P.nparts, true,
                                      0.0);
      tm = t.m; ts = t.s; targ = t.arg;
    }
  }
  state = uniform(state);

  ResidCoef kc;
  float inv_z = 1.0f;
  bool use_r = false;
  if (state == 2) {
    kc = resid_coef(tm, ts, dm, ds, scale_of(tau), has_q);
    use_r = has_q && zr > 0.0;
    if (use_r) inv_z = (float)(1.0 / zr);
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    if (u < nv) {
      const int64_t e0 = eb + (int64_t)u * SLAB;
      float o[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        if (state == 0) {
          o[e] = nan;
        } else if (state == 1) {
          o[e] = (e0 + e == targ) ? 1.0f : 0.0f;
        } else {
          float p, r;
          resid_elem(kc, elem<In>(traw[u], e), kc.has_q ? elem<In>(draw[u], e) : 0.0f, p, r);
          o[e] = use_r ? r * inv_z : p;
        }
      }
      if (e0 + VEC <= P.V) {
#pragma unroll
        for (int h = 0; h < VEC; h += 4)
          *reinterpret_cast<float4*>(orow + e0 + h) =
              make_float4(o[h], o[h + 1], o[h + 2], o[h + 3]);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          if (e0 + e < P.V) orow[e0 + e] = o[e];
      }
    }
  }
}

// ================================================================ hits

// Speculation-cache lookup, one thread per sequence: the index of the
// outcome token among the forks of the outcome position, else -1.
__global__ __launch_bounds__(kBlock) void k_hits(int32_t B, int32_t k, int32_t f,
                                                 const int32_t* __restrict__ forks,
                                                 const int32_t* __restrict__ accept_len,
                                                 const int32_t* __restrict__ out_token,
                                                 int32_t* __restrict__ hits) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int n = accept_len[b];
  const int t = out_token[b];
  int hit = -1;
  if (n >= 0 && n <= k && t >= 0) {
    const int32_t* row = forks + (b * (k + 1) + n) * f;
    for (int r = f - 1; r >= 0; --r)
      if (row[r] == t) hit = r;
  }
  hits[b] = hit;
}

static hipError_t launch_hits(int32_t B, int32_t k, int32_t f, const int32_t* forks,
                              const int32_t* accept_len, const int32_t* out_token, int32_t* hits,
                              hipStream_t s) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(k_hits, dim3((unsigned)((B + kBlock - 1) / kBlock)), dim3(kBlock), 0, s, B,
                     k, f, forks, accept_len, out_token, hits);
  return hipGetLastError();
}

// ================================================================ fill

__global__ __launch_bounds__(kBlock) void k_fill_zero(uint8_t* p, size_t bytes) {
  const size_t n16 = bytes / 16;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    reinterpret_cast<uint4*>(p)[i] = make_uint4(0, 0, 0, 0);
  const size_t tail = bytes - n16 * 16;
  if (blockIdx.x == 0 && threadIdx.x < tail) p[n16 * 16 + threadIdx.x] = 0;
}

// ================================================================ host side

struct Layout {
  size_t tm, ts, targ, dm, ds, darg, dtv, dti, rows, seqs, xd, yd, cn, cpos, cvm, ctr, total;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Candidate-list length of the stream for fan-out f: 4 covers f <= 4, 16
// covers the rest (the top-F contain the top-f).
static int fork_F(int f) {
  if (f <= 0) return 0;
  return f <= 4 ? 4 : 16;
}

// Workspace layout for R row slots, B sequences and rows of cpr chunks,
// after the control header (kCtlBytes, same offset for every call).
static Layout make_layout(int64_t R, int64_t B, int64_t cpr, int F) {
  Layout L;
  size_t o = (size_t)kCtlBytes;
  auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
  const size_t RS = (size_t)(R * kMaxSeg);
  const size_t Fa = (size_t)(F > 0 ? F : 1);
  L.tm = take(sizeof(float) * RS);
  L.ts = take(sizeof(double) * RS);
  L.targ = take(sizeof(int) * RS);
  L.dm = take(sizeof(float) * RS);
  L.ds = take(sizeof(double) * RS);
  L.darg = take(sizeof(int) * RS);
  L.dtv = take(sizeof(float) * RS * Fa);
  L.dti = take(sizeof(int) * RS * Fa);
  L.rows = take(sizeof(RowRec) * R);
  L.seqs = take(sizeof(SeqRec) * B);
  L.xd = take(sizeof(float) * R);
  L.yd = take(sizeof(float) * R);
  L.cn = take(F > 0 ? sizeof(int) * RS : 0);
  L.cpos = take(F > 0 ? sizeof(int) * RS * kDumpCap : 0);
  L.cvm = take(F > 0 ? sizeof(float) * RS * kDumpCap : 0);
  L.ctr = take(sizeof(double) * R * cpr);
  L.total = o;
  return L;
}

static Ws bind_ws(void* base, const Layout& L) {
  uint8_t* p = static_cast<uint8_t*>(base);
  Ws w;
  w.seqctl = reinterpret_cast<unsigned*>(p);
  w.rowctl = reinterpret_cast<unsigned*>(p + kMaxBatch * kSeqCtlBytes);
  w.tm = reinterpret_cast<float*>(p + L.tm);
  w.ts = reinterpret_cast<double*>(p + L.ts);
  w.targ = reinterpret_cast<int*>(p + L.targ);
  w.dm = reinterpret_cast<float*>(p + L.dm);
  w.ds = reinterpret_cast<double*>(p + L.ds);
  w.darg = reinterpret_cast<int*>(p + L.darg);
  w.dtv = reinterpret_cast<float*>(p + L.dtv);
  w.dti = reinterpret_cast<int*>(p + L.dti);
  w.rows = reinterpret_cast<RowRec*>(p + L.rows);
  w.seqs = reinterpret_cast<SeqRec*>(p + L.seqs);
  w.xd = reinterpret_cast<float*>(p + L.xd);
  w.yd = reinterpret_cast<float*>(p + L.yd);
  w.cn = reinterpret_cast<int*>(p + L.cn);
  w.cpos = reinterpret_cast<int*>(p + L.cpos);
  w.cvm = reinterpret_cast<float*>(p + L.cvm);
  w.ctr = reinterpret_cast<double*>(p + L.ctr);
  return w;
}

static int64_t slabs_per_row(int dtype, int64_t V) {
  const int64_t s = (dtype == SV_BF16) ? slab_elems<uint16_t>() : slab_elems<float>();
  return (V + s - 1) / s;
}
static int64_t chunks_per_row(int dtype, int64_t V) {
  return (slabs_per_row(dtype, V) + kU - 1) / kU;
}

static size_t workspace_bytes(int64_t R, int64_t B, int64_t V, int f) {
  return make_layout(R, B, chunks_per_row(SV_F32, V), fork_F(f)).total;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static int elem_bytes(int dtype) { return dtype == SV_BF16 ? 2 : 4; }

static bool rows_aligned(const void* base, int dtype, int64_t s1, int64_t s2) {
  const int64_t eb = elem_bytes(dtype);
  return aligned16(base) && ((s1 * eb) % 16 == 0) && ((s2 * eb) % 16 == 0);
}

static sv_status check_batch(const sv_batch* in, bool need_target, bool need_draft) {
  if (!in) return SV_ERR_INVALID_ARG;
  if (in->B < 0 || in->k < 1 || in->k > kMaxK || in->V < 2 || in->V > kMaxV)
    return SV_ERR_INVALID_ARG;
  if (in->dtype != SV_F32 && in->dtype != SV_BF16) return SV_ERR_INVALID_ARG;
  if (in->B > kMaxBatch || (int64_t)in->B * (in->k + 1) > kMaxRows) return SV_ERR_INVALID_ARG;
  if (in->B == 0) return SV_OK;
  if (!in->temperature || !in->draft_tokens) return SV_ERR_INVALID_ARG;
  if (need_target) {
    if (!in->target) return SV_ERR_INVALID_ARG;
    if (!rows_aligned(in->target, in->dtype, in->t_seq_stride, in->t_row_stride))
      return SV_ERR_MISALIGNED;
  }
  if (need_draft) {
    if (!in->draft) return SV_ERR_INVALID_ARG;
    if (!rows_aligned(in->draft, in->dtype, in->d_seq_stride, in->d_row_stride))
      return SV_ERR_MISALIGNED;
  }
  return SV_OK;
}

static Params base_params(const sv_batch* in) {
  Params P;
  memset(&P, 0, sizeof(P));
  P.T = in->target; P.t_seq = in->t_seq_stride; P.t_row = in->t_row_stride;
  P.D = in->draft; P.d_seq = in->d_seq_stride; P.d_row = in->d_row_stride;
  P.drafts = in->draft_tokens;
  P.tau = in->temperature;
  P.B = in->B; P.k = in->k; P.V = in->V;
  P.nslab = (int32_t)slabs_per_row(in->dtype, in->V);
  P.cpr = (int32_t)chunks_per_row(in->dtype, in->V);
  P.rows_per_temp = 1;
  return P;
}

static dim3 grid_for(int64_t waves) {
  return dim3((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock));
}

static int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      v <= 0)
    v = 256;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// Waves of a kernel that fit on the device at once (occupancy query,
// cached per kernel and device).
template <typename In, int F>
static int64_t resident_waves() {
  static std::atomic<int64_t> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int64_t v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int blocks = 0;
  const void* fn = (const void*)k_stats<In, F>;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, kBlock, 0) != hipSuccess ||
      blocks <= 0)
    blocks = 4;
  v = (int64_t)device_cus() * blocks * kWavesPerBlock;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// Segments per row: one resident round of waves, each with an equal share
// of its row's slabs (at most 64 partials per row).
template <typename In, int F>
static void plan_segments(Params& P) {
  const int64_t res = resident_waves<In, F>();
  int64_t g = res / std::max<int64_t>(P.nslots, 1);
  g = std::max<int64_t>(1, std::min<int64_t>(g, std::min<int64_t>(kMaxSeg, P.nslab)));
  P.nparts = (int32_t)g;
}

template <typename In, int F>
static hipError_t launch_stats_F(Params& P, hipStream_t s) {
  plan_segments<In, F>(P);
  const int64_t waves = P.nslots * P.nparts;
  if (waves == 0) return hipSuccess;
  hipLaunchKernelGGL((k_stats<In, F>), grid_for(waves), dim3(kBlock), 0, s, P);
  return hipGetLastError();
}

// k_decide: enough blocks per task row to cover the device (one 1024-thread
// block per CU), at least four chunks of the summed row per block (one
// chunk sum per SIMD), plus the fork blocks when verify asks for forks (one
// per sequence, or up to one per row at small batches).
template <typename In, int F>
static hipError_t launch_decide_F(Params P, hipStream_t s) {
  const int64_t tasks = (P.mode == kResidual && P.rows_all) ? (int64_t)P.B * (P.k + 1) : P.B;
  if (tasks == 0) return hipSuccess;
  // fork blocks per sequence: one, or (small batches, k + 1 <= 16) up to one
  // per row while they take at most a quarter of the CUs
  const bool forks = P.mode == kVerify && P.fork_tok;
  int fsplit = 1;
  if (forks && P.k + 1 <= kDecideWaves) {
    while (fsplit * 2 <= P.k + 1 && (int64_t)P.B * fsplit * 2 <= device_cus() / 4) fsplit *= 2;
  }
  P.fsplit = fsplit;
  const int64_t fork_blocks = forks ? (int64_t)P.B * fsplit : 0;
  int64_t nbs = (device_cus() - fork_blocks) / tasks;
  nbs = std::max<int64_t>(1, std::min<int64_t>(nbs, std::max<int64_t>(1, P.cpr / 4)));
  P.nbs = (int32_t)nbs;
  hipLaunchKernelGGL((k_decide<In, F>), dim3((unsigned)(tasks * nbs + fork_blocks)),
                     dim3(kDecideBlock), 0, s, P);
  return hipGetLastError();
}

template <typename In>
static hipError_t launch_write(const Params& P, hipStream_t s) {
  const int64_t nslots = (P.mode == kSoftmax) ? P.nslots : (int64_t)P.B * (P.k + 1);
  const int64_t waves = nslots * P.cpr;
  if (waves == 0) return hipSuccess;
  if (!P.out) return hipErrorInvalidValue;  // every wave stores into the output rows
  hipLaunchKernelGGL((k_write<In>), grid_for(waves), dim3(kBlock), 0, s, P);
  return hipGetLastError();
}

template <typename In>
static hipError_t launch_stats(Params& P, hipStream_t s) {
  switch (P.F) {
    case 0: return launch_stats_F<In, 0>(P, s);
    case 4: return launch_stats_F<In, 4>(P, s);
    default: return launch_stats_F<In, 16>(P, s);
  }
}
template <typename In>
static hipError_t launch_decide(const Params& P, hipStream_t s) {
  switch (P.F) {
    case 0: return launch_decide_F<In, 0>(P, s);
    case 4: return launch_decide_F<In, 4>(P, s);
    default: return launch_decide_F<In, 16>(P, s);
  }
}

// The statistics launch plans its blocks into P (k_decide and k_write read
// P.nparts).
static hipError_t dispatch_stats(int dtype, Params& P, hipStream_t s) {
  return dtype == SV_BF16 ? launch_stats<uint16_t>(P, s) : launch_stats<float>(P, s);
}
static hipError_t dispatch_decide(int dtype, const Params& P, hipStream_t s) {
  return dtype == SV_BF16 ? launch_decide<uint16_t>(P, s) : launch_decide<float>(P, s);
}
static hipError_t dispatch_write(int dtype, const Params& P, hipStream_t s) {
  return dtype == SV_BF16 ? launch_write<uint16_t>(P, s) : launch_write<float>(P, s);
}

static sv_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (!ws || ws_bytes < need) return SV_ERR_WORKSPACE;
  if (!aligned16(ws)) return SV_ERR_MISALIGNED;
  return SV_OK;
}

}  // namespace sv

using namespace sv;

// ================================================================ scratch
// The workspace of sv_verify_noalloc: one array per device, in the code
// object's zero-initialised data, held until the process ends.  Host code
// never passes the array's name to a kernel or a copy (on the host it is
// only a stand-in for the symbol): it uses the device address that
// hipGetSymbolAddress returns on each device.
static __device__ __align__(256) uint8_t scratch[SV_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch[kMaxDevices];  // the array's address on each device
}  // namespace

// The current device's scratch address.  The first call on a device looks
// it up (with that device current) and zero-fills the array on `stream`, so
// that the arrival counters at its start begin at zero; later calls reuse
// both.
static sv_status scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SV_ERR_HIP;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* a = nullptr;
      if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return SV_ERR_HIP;
      const size_t n16 = SV_NOALLOC_SCRATCH_BYTES / 16;
      const unsigned blocks = (unsigned)std::min<size_t>((n16 + kBlock - 1) / kBlock, 4096);
      hipLaunchKernelGGL(k_fill_zero, dim3(blocks), dim3(kBlock), 0, stream, (uint8_t*)a,
                         (size_t)SV_NOALLOC_SCRATCH_BYTES);
      if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
      p = a;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SV_OK;
}

extern "C" {

size_t sv_workspace_size(int32_t B, int32_t k, int32_t V, int32_t f) {
  if (B < 0 || k < 0 || k > kMaxK || V < 2 || V > kMaxV || f < 0 || f > kMaxF) return 0;
  const int64_t R = (int64_t)B * (k + 1);
  return workspace_bytes(R > 0 ? R : 1, B > 0 ? B : 1, V, f);
}

sv_status sv_workspace_init(void* ws, size_t bytes, void* stream) {
  if (!ws) return SV_ERR_INVALID_ARG;
  if (bytes == 0) return SV_OK;
  if (!aligned16(ws)) return SV_ERR_MISALIGNED;
  const size_t n16 = (bytes + 15) / 16;
  const unsigned blocks = (unsigned)std::min<size_t>((n16 + kBlock - 1) / kBlock, 4096);
  hipLaunchKernelGGL(k_fill_zero, dim3(blocks), dim3(kBlock), 0, (hipStream_t)stream,
                     (uint8_t*)ws, bytes);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

const char* sv_status_string(int32_t s) {
  switch (s) {
    case SV_OK: return "SV_OK";
    case SV_ERR_INVALID_ARG: return "SV_ERR_INVALID_ARG";
    case SV_ERR_MISALIGNED: return "SV_ERR_MISALIGNED";
    case SV_ERR_WORKSPACE: return "SV_ERR_WORKSPACE";
    case SV_ERR_HIP: return "SV_ERR_HIP";
    default: return "SV_UNKNOWN_STATUS";
  }
}

const char* sv_version(void) { return "libspecverify 0.3.0 gfx950"; }

sv_status sv_softmax_temp(const void* logits, int32_t dtype, int64_t rows, int32_t V,
                          int64_t row_stride, const float* temperature, int64_t rows_per_temp,
                          float* probs, int64_t out_row_stride, void* ws, size_t ws_bytes,
                          void* stream) {
  if (rows < 0 || V < 2 || V > kMaxV || rows_per_temp < 1) return SV_ERR_INVALID_ARG;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_INVALID_ARG;
  if (rows == 0) return SV_OK;
  if (rows > ((int64_t)1 << 31) / 64) return SV_ERR_INVALID_ARG;
  if (!logits || !temperature || !probs) return SV_ERR_INVALID_ARG;
  if (!rows_aligned(logits, dtype, row_stride, row_stride)) return SV_ERR_MISALIGNED;
  if (!aligned16(probs) || (out_row_stride * 4) % 16 != 0) return SV_ERR_MISALIGNED;
  if (row_stride < V || out_row_stride < V) return SV_ERR_INVALID_ARG;
  sv_status st = check_ws(ws, ws_bytes, workspace_bytes(rows, 1, V, 0));
  if (st != SV_OK) return st;
  Params P;
  memset(&P, 0, sizeof(P));
  P.T = logits; P.t_row = row_stride; P.t_seq = row_stride;
  P.tau = temperature;
  P.B = (int32_t)std::min<int64_t>(rows, 0x7fffffff); P.k = 0; P.V = V; P.f = 0; P.F = 0;
  P.nslab = (int32_t)slabs_per_row(dtype, V);
  P.cpr = (int32_t)chunks_per_row(dtype, V);
  P.mode = kSoftmax;
  P.nslots = rows;
  P.rows_per_temp = rows_per_temp;
  P.out = probs; P.out_row = out_row_stride;
  P.ws = bind_ws(ws, make_layout(rows, 1, chunks_per_row(SV_F32, V), 0));
  hipStream_t s = (hipStream_t)stream;
  if (dispatch_stats(dtype, P, s) != hipSuccess) return SV_ERR_HIP;
  if (dispatch_write(dtype, P, s) != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

sv_status sv_verify_ex(const sv_batch* in, const float* u_accept, const float* u_recover,
                       int32_t* accept_len, int32_t* out_token, float* p_draft, float* q_draft,
                       const sv_forks* forks, void* ws, size_t ws_bytes, void* stream,
                       const sv_opts* opts) {
  const int f = forks ? forks->f : 0;
  if (forks && (f < 1 || f > kMaxF || (in && f > in->V - 1))) return SV_ERR_INVALID_ARG;
  // Draft rows are needed at temperature > 0 (unknown on the host), for q_draft
  // and for forks.
  sv_status st = check_batch(in, true, true);
  if (st != SV_OK || in->B == 0) return st;
  if (!u_accept || !u_recover || !accept_len || !out_token) return SV_ERR_INVALID_ARG;
  if (forks && !forks->tokens) return SV_ERR_INVALID_ARG;
  st = check_ws(ws, ws_bytes, sv_workspace_size(in->B, in->k, in->V, f));
  if (st != SV_OK) return st;
  Params P = base_params(in);
  P.mode = kVerify;
  P.f = f; P.F = fork_F(f);
  P.want_q = q_draft != nullptr;
  P.u_acc = u_accept; P.u_rec = u_recover;
  P.accept_len = accept_len; P.out_token = out_token;
  P.p_draft = p_draft; P.q_draft = q_draft;
  P.fork_tok = forks ? forks->tokens : nullptr;
  P.fork_prob = forks ? forks->probs : nullptr;
  P.hits = forks ? forks->hits : nullptr;
  P.nslots = (int64_t)in->B * (in->k + 1);
  P.ws = bind_ws(ws, make_layout(P.nslots, in->B, chunks_per_row(SV_F32, in->V), P.F));
  hipStream_t s = (hipStream_t)stream;
  if (opts && opts->ev_stats_begin) {
    if (hipEventRecord((hipEvent_t)opts->ev_stats_begin, s) != hipSuccess) return SV_ERR_HIP;
  }
  if (dispatch_stats(in->dtype, P, s) != hipSuccess) return SV_ERR_HIP;
  if (opts && opts->ev_stats_end) {
    if (hipEventRecord((hipEvent_t)opts->ev_stats_end, s) != hipSuccess) return SV_ERR_HIP;
  }
  if (dispatch_decide(in->dtype, P, s) != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

sv_status sv_verify(const sv_batch* in, const float* u_accept, const float* u_recover,
                    int32_t* accept_len, int32_t* out_token, float* p_draft, float* q_draft,
                    const sv_forks* forks, void* ws, size_t ws_bytes, void* stream) {
  return sv_verify_ex(in, u_accept, u_recover, accept_len, out_token, p_draft, q_draft, forks,
                      ws, ws_bytes, stream, nullptr);
}

sv_status sv_verify_noalloc(const sv_batch* in, const float* u_accept, const float* u_recover,
                            int32_t* accept_len, int32_t* out_token, float* p_draft,
                            float* q_draft, const sv_forks* forks, void* stream) {
  if (!in) return SV_ERR_INVALID_ARG;
  const int f = forks ? forks->f : 0;
  if (forks && (f < 1 || f > kMaxF)) return SV_ERR_INVALID_ARG;
  const size_t need = sv_workspace_size(in->B, in->k, in->V, f);
  if (need == 0) return SV_ERR_INVALID_ARG;
  if (need > (size_t)SV_NOALLOC_SCRATCH_BYTES) return SV_ERR_WORKSPACE;
  void* ws = nullptr;
  const sv_status st = scratch_address((hipStream_t)stream, &ws);
  if (st != SV_OK) return st;
  return sv_verify_ex(in, u_accept, u_recover, accept_len, out_token, p_draft, q_draft, forks, ws,
                      (size_t)SV_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

sv_status sv_residual_sample(const sv_batch* in, const int32_t* position,
                             const float* u_recover, int32_t* token_out, float* residual,
                             int64_t res_seq_stride, int64_t res_row_stride, void* ws,
                             size_t ws_bytes, void* stream) {
  sv_status st = check_batch(in, true, true);
  if (st != SV_OK || in->B == 0) return st;
  if (!position || !u_recover || !token_out) return SV_ERR_INVALID_ARG;
  if (residual && (!aligned16(residual) || (res_seq_stride * 4) % 16 != 0 ||
                   (res_row_stride * 4) % 16 != 0))
    return SV_ERR_MISALIGNED;
  st = check_ws(ws, ws_bytes, sv_workspace_size(in->B, in->k, in->V, 0));
  if (st != SV_OK) return st;
  Params P = base_params(in);
  P.mode = kResidual;
  P.rows_all = residual != nullptr;
  P.position = position;
  P.u_rec = u_recover;
  P.out_token = token_out;
  P.out = residual; P.out_seq = res_seq_stride; P.out_row = res_row_stride;
  P.nslots = P.rows_all ? (int64_t)in->B * (in->k + 1) : in->B;
  P.ws = bind_ws(ws, make_layout((int64_t)in->B * (in->k + 1), in->B,
                                 chunks_per_row(SV_F32, in->V), 0));
  hipStream_t s = (hipStream_t)stream;
  if (dispatch_stats(in->dtype, P, s) != hipSuccess) return SV_ERR_HIP;
  if (dispatch_decide(in->dtype, P, s) != hipSuccess) return SV_ERR_HIP;
  // the distributions are written only when asked for (the token-only call
  // has no output rows)
  if (residual && dispatch_write(in->dtype, P, s) != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

sv_status sv_forked_topf(const sv_batch* in, const sv_forks* forks, void* ws, size_t ws_bytes,
                         void* stream) {
  if (!forks) return SV_ERR_INVALID_ARG;
  const int f = forks->f;
  if (f < 1 || f > kMaxF || (in && f > in->V - 1)) return SV_ERR_INVALID_ARG;
  sv_status st = check_batch(in, false, true);
  if (st != SV_OK || in->B == 0) return st;
  if (!forks->tokens) return SV_ERR_INVALID_ARG;
  st = check_ws(ws, ws_bytes, sv_workspace_size(in->B, in->k, in->V, f));
  if (st != SV_OK) return st;
  Params P = base_params(in);
  P.mode = kForks;
  P.f = f; P.F = fork_F(f);
  P.fork_tok = forks->tokens;
  P.fork_prob = forks->probs;
  P.nslots = (int64_t)in->B * (in->k + 1);
  P.ws = bind_ws(ws, make_layout(P.nslots, in->B, chunks_per_row(SV_F32, in->V), P.F));
  hipStream_t s = (hipStream_t)stream;
  if (dispatch_stats(in->dtype, P, s) != hipSuccess) return SV_ERR_HIP;
  if (dispatch_decide(in->dtype, P, s) != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

sv_status sv_cache_hit(int32_t B, int32_t k, int32_t f, const int32_t* fork_tokens,
                       const int32_t* accept_len, const int32_t* out_token, int32_t* hits,
                       void* stream) {
  if (B < 0 || k < 1 || k > kMaxK || f < 1 || f > kMaxF) return SV_ERR_INVALID_ARG;
  if (B == 0) return SV_OK;
  if (!fork_tokens || !accept_len || !out_token || !hits) return SV_ERR_INVALID_ARG;
  return launch_hits(B, k, f, fork_tokens, accept_len, out_token, hits, (hipStream_t)stream) ==
                 hipSuccess
             ? SV_OK
             : SV_ERR_HIP;
}

}  // extern "C"
