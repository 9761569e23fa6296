// libspecverify: kernels and the C ABI entry points (gfx950).
//
// Kernel chain of sv_verify (one stream, no host synchronisation):
//   k_stats   one wavefront per (row, chunk): streams the target and draft
//             chunk once with 16-byte loads, writes chunk partials; the last
//             wave to finish a row merges its partials (row max, sum, argmax,
//             fork top-f, p(d), q(d)); the last row to finish a sequence
//             decides it (acceptance tests, first rejection by ballot, greedy
//             token).
//   k_resid   one wavefront per chunk of row n of every sequence still to be
//             drawn (temperature > 0): residual chunk sums in fp64; the last
//             wave of the row finds the chunk holding u*Z and draws the token
//             inside it.
// sv_residual_sample runs the same pair (plus k_write for the full residual
// distributions); sv_softmax_temp runs k_stats then k_write; sv_forked_topf
// runs k_stats alone.
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
#include <stdint.h>
#include <string.h>

#include "specverify.h"
#include "sv_device.h"
#include "sv_stats.h"

namespace sv {

constexpr double kLog2e = 1.4426950408889634074;

enum Mode : int { kVerify = 0, kForks = 1, kResidual = 2, kSoftmax = 3 };

// Arrival counters sit 256 bytes apart: device-scope atomics to one memory
// line are serialised, and many rows finishing together must not queue on a
// shared line.
constexpr int64_t kCtrStride = 64;

// Per-row results of the statistics pass (72 bytes).
struct RowRec {
  float tm;     // target row max
  int targ;     // target argmax (temperature 0)
  double ts;    // target sum of 2^((x - tm) c)
  float dm;     // draft row max (drafted token included)
  int darg;     // draft argmax (temperature 0)
  double ds;    // draft sum of 2^((y - dm) c)
  double pd;    // p(d), q(d) of the drafted token (j < k)
  double qd;
  double zr;    // residual total sum max(0, p - q) (residual kernel)
  double zp;    // target total sum p (residual kernel)
  int valid;    // rows read are finite and inputs in range
  int pad;
};
static_assert(sizeof(RowRec) == 72, "RowRec layout");

__device__ __forceinline__ void store_row(RowRec* p, const RowRec& r) {
  st_dev(&p->tm, r.tm); st_dev(&p->targ, r.targ); st_dev(&p->ts, r.ts);
  st_dev(&p->dm, r.dm); st_dev(&p->darg, r.darg); st_dev(&p->ds, r.ds);
  st_dev(&p->pd, r.pd); st_dev(&p->qd, r.qd); st_dev(&p->zr, r.zr); st_dev(&p->zp, r.zp);
  st_dev(&p->valid, r.valid); st_dev(&p->pad, r.pad);
}

struct SeqRec {
  int n;        // outcome position
  int status;   // 0 error, 1 finished (greedy), 2 residual draw pending
};

struct Ws {
  unsigned* row_ctr;   // [R], one per kCtrStride words
  unsigned* seq_ctr;   // [B], one per kCtrStride words
  unsigned* k2_ctr;    // [R], one per kCtrStride words
  float* tm; double* ts; int* targ;     // [R * cpr] target chunk partials
  float* dm; double* ds; int* darg;     // [R * cpr] draft chunk partials
  float* dtv; int* dti;                 // [R * cpr * F] draft chunk top-f
  int* ftok; float* fprob;              // [R * F] a row's forks, staged for the sequence
  RowRec* rows;        // [R]
  SeqRec* seqs;        // [B]
  double* kr; double* kp;               // [R * cpr * kU] residual slab sums
};

struct Params {
  const void* T; int64_t t_seq, t_row;
  const void* D; int64_t d_seq, d_row;
  const int32_t* drafts;
  const float* tau;
  const float* u_acc;
  const float* u_rec;
  const int32_t* position;
  int32_t B, k, V, f, F, cpr, mode, rows_all, want_q;
  int32_t nseg;            // k_stats: segments per row (one wave each)
  int32_t seg_chunks;      // k_stats: chunks per segment
  int64_t nslots;          // row slots of k_stats
  int64_t rows_per_temp;   // softmax
  int32_t* accept_len;
  int32_t* out_token;
  float* p_draft;
  float* q_draft;
  int32_t* fork_tok;
  float* fork_prob;
  float* out; int64_t out_seq, out_row;
  Ws ws;
};

__device__ __forceinline__ bool tau_ok(float t) { return t >= 0.0f && t < pos_inf(); }

__device__ __forceinline__ float slot_tau(const Params& P, int64_t slot, int b) {
  if (P.mode == kSoftmax) return P.tau[slot / P.rows_per_temp];
  return P.tau[b];
}

// Row slot -> (sequence, position) in k_stats.
__device__ __forceinline__ void slot_to_bj(const Params& P, int64_t slot, int& b, int& j) {
  if (P.mode == kSoftmax) { b = (int)slot; j = 0; return; }
  if (P.mode == kResidual && !P.rows_all) { b = (int)slot; j = P.position[b]; return; }
  b = (int)(slot / (P.k + 1));
  j = (int)(slot - (int64_t)b * (P.k + 1));
}

template <typename In>
__device__ __forceinline__ const In* trow_ptr(const Params& P, int b, int j) {
  return reinterpret_cast<const In*>(P.T) + (int64_t)b * P.t_seq + (int64_t)j * P.t_row;
}
template <typename In>
__device__ __forceinline__ const In* drow_ptr(const Params& P, int b, int j) {
  return reinterpret_cast<const In*>(P.D) + (int64_t)b * P.d_seq + (int64_t)j * P.d_row;
}
template <typename In>
__device__ __forceinline__ float load_logit(const In* row, int64_t t) {
  if constexpr (sizeof(In) == 4) return row[t];
  else return __uint_as_float(((uint32_t)row[t]) << 16);
}

__device__ __forceinline__ float scale_of(float tau) {
  return (float)(kLog2e / (double)tau);
}

// Which tensors / statistics a row needs.
struct RowPlan {
  bool pos_ok, readT, readD, topf, greedy, tok;
  int64_t mask_id;
};

__device__ __forceinline__ RowPlan plan_row(const Params& P, int b, int j, float tau) {
  RowPlan r;
  r.tok = tau_ok(tau);
  r.greedy = (tau == 0.0f) || !r.tok;
  r.pos_ok = (j >= 0 && j <= P.k);
  const bool forks = (P.mode == kForks) || (P.mode == kVerify && P.f > 0);
  r.topf = forks && r.pos_ok;
  r.readT = r.pos_ok && P.mode != kForks;
  if (P.mode == kForks) r.readD = r.pos_ok;
  else if (P.mode == kVerify)
    r.readD = r.pos_ok && (j < P.k ? (tau != 0.0f || P.want_q || P.f > 0) : (P.f > 0));
  else if (P.mode == kResidual) r.readD = r.pos_ok && j < P.k;
  else r.readD = false;
  r.mask_id = -1;
  if (r.topf && j < P.k) {
    const int d = P.drafts[(int64_t)b * P.k + j];
    r.mask_id = d;  // out-of-range ids match no element
  }
  return r;
}

// ------------------------------------------------------------ merge helpers

struct Merged {
  float m; double s; int arg;
};

// Row max / sum / argmax from the chunk partials of one slot.
__device__ __forceinline__ Merged merge_chunks(const float* pm, const double* ps, const int* parg,
                                               int64_t base, int cpr, bool greedy, double cd) {
  const int lane = lane_id();
  float m = neg_inf();
  for (int ch = lane; ch < cpr; ch += kLanes) m = fmaxf(m, ld_dev(pm + base + ch));
  const float M = wave_max(m);
  double s = 0.0;
  int arg = kEmptyId;
  for (int ch = lane; ch < cpr; ch += kLanes) {
    const float mc = ld_dev(pm + base + ch);
    if (greedy) {
      if (mc == M) arg = min(arg, ld_dev(parg + base + ch));
    } else if (finitef(M) && mc > neg_inf()) {
      s += ld_dev(ps + base + ch) * exp2(((double)mc - (double)M) * cd);
    }
  }
  Merged r;
  r.m = M;
  r.s = wave_sum(s);
  r.arg = wave_min(arg);
  return r;
}

// Overwrites the per-sequence outputs of an error sequence.
__device__ __forceinline__ void write_seq_error(const Params& P, int b) {
  const int lane = lane_id();
  const float nan = __uint_as_float(0x7fc00000u);
  const int K1 = P.k + 1;
  if (P.fork_tok) {
    for (int t = lane; t < K1 * P.f; t += kLanes) {
      P.fork_tok[(int64_t)b * K1 * P.f + t] = -1;
      if (P.fork_prob) P.fork_prob[(int64_t)b * K1 * P.f + t] = nan;
    }
  }
  if (P.mode == kVerify) {
    for (int t = lane; t < P.k; t += kLanes) {
      if (P.p_draft) P.p_draft[(int64_t)b * P.k + t] = nan;
      if (P.q_draft) P.q_draft[(int64_t)b * P.k + t] = nan;
    }
  }
  if (lane == 0) {
    if (P.accept_len) P.accept_len[b] = -1;
    if (P.out_token) P.out_token[b] = -1;
  }
}

// The last row of sequence b to finish decides it.
__device__ __forceinline__ void finalize_sequence(const Params& P, int b) {
  const int lane = lane_id();
  const int k = P.k;
  const int K1 = k + 1;
  const float tau = P.tau[b];
  const bool tok = tau_ok(tau);
  const bool greedy = tau == 0.0f;

  // drafted ids in range
  bool ok = tok;
  int d = 0;
  if (lane < k) {
    d = P.drafts[(int64_t)b * k + lane];
    if (d < 0 || d >= P.V) ok = false;
  }
  int pos = -1;
  if (P.mode == kResidual) {
    pos = P.position[b];
    if (pos < 0 || pos > k) ok = false;
  }
  // rows read are valid
  if (P.mode == kResidual && !P.rows_all) {
    if (lane == 0 && !ld_dev(&P.ws.rows[b].valid)) ok = false;
  } else if (lane < K1) {
    if (!ld_dev(&P.ws.rows[(int64_t)b * K1 + lane].valid)) ok = false;
  }
  const bool seq_ok = __ballot(!ok) == 0ull;

  SeqRec sr;
  sr.n = 0;
  sr.status = 0;
  if (!seq_ok) {
    write_seq_error(P, b);
  } else if (P.mode == kVerify) {
    bool acc = true;
    if (lane < k) {
      const RowRec* rr = &P.ws.rows[(int64_t)b * K1 + lane];
      if (greedy) {
        acc = (d == ld_dev(&rr->targ));
      } else {
        // a = min(1, p/q); q = 0: a = 1 if p > 0 else 0.  Accept iff u < a.
        const double p = ld_dev(&rr->pd), q = ld_dev(&rr->qd);
        const double a = (q == 0.0) ? (p > 0.0 ? 1.0 : 0.0) : fmin(1.0, p / q);
        acc = (double)P.u_acc[(int64_t)b * k + lane] < a;
      }
    }
    if (lane < k) {
      const RowRec* rr = &P.ws.rows[(int64_t)b * K1 + lane];
      if (P.p_draft) P.p_draft[(int64_t)b * k + lane] = (float)ld_dev(&rr->pd);
      if (P.q_draft) P.q_draft[(int64_t)b * k + lane] = (float)ld_dev(&rr->qd);
    }
    const unsigned long long rej = __ballot(lane < k && !acc);
    const int n = rej ? (__ffsll((long long)rej) - 1) : k;
    sr.n = n;
    if (greedy) {
      sr.status = 1;
      if (lane == 0) P.out_token[b] = ld_dev(&P.ws.rows[(int64_t)b * K1 + n].targ);
    } else {
      sr.status = 2;
    }
    if (lane == 0) P.accept_len[b] = n;
  } else if (P.mode == kResidual) {
    sr.n = pos;
    if (greedy) {
      sr.status = 1;
      const int64_t rs = P.rows_all ? (int64_t)b * K1 + pos : (int64_t)b;
      if (lane == 0) P.out_token[b] = ld_dev(&P.ws.rows[rs].targ);
    } else {
      sr.status = 2;
    }
  } else {
    sr.status = 1;
  }
  if (seq_ok && P.fork_tok) {
    // forks staged by the row merges: rows b*(k+1) .. b*(k+1)+k
    for (int t = lane; t < K1 * P.f; t += kLanes) {
      const int jj = t / P.f, r = t - jj * P.f;
      const int64_t src = ((int64_t)b * K1 + jj) * P.F + r;
      P.fork_tok[(int64_t)b * K1 * P.f + t] = ld_dev(P.ws.ftok + src);
      if (P.fork_prob) P.fork_prob[(int64_t)b * K1 * P.f + t] = ld_dev(P.ws.fprob + src);
    }
  }
  if (lane == 0) P.ws.seqs[b] = sr;
}

// ------------------------------------------------------------ k_stats

template <typename In, int F>
__device__ __forceinline__ void row_merge(const Params& P, int64_t slot, int b, int j, float tau,
                          const RowPlan& pl) {
  const int lane = lane_id();
  const int np = P.nseg;               // one partial per segment
  const int64_t base = slot * P.cpr;   // partial arrays have a stride of cpr per row
  const float c = pl.greedy ? 0.0f : scale_of(tau);
  const double cd = (double)c;
  const Ws& W = P.ws;
  const int k = P.k;
  const int K1 = k + 1;
  const float nan = __uint_as_float(0x7fc00000u);

  RowRec rec;
  rec.tm = neg_inf(); rec.targ = kEmptyId; rec.ts = 0.0;
  rec.dm = neg_inf(); rec.darg = kEmptyId; rec.ds = 0.0;
  rec.pd = nan; rec.qd = nan; rec.zr = 0.0; rec.zp = 0.0;
  rec.pad = 0;
  bool valid = pl.tok && pl.pos_ok;

  int d = -1;
  bool d_ok = false;
  if (P.mode != kSoftmax && pl.pos_ok && j < k) {
    d = P.drafts[(int64_t)b * k + j];
    d_ok = (d >= 0 && d < P.V);
  }

  if (pl.readT) {
    const Merged t = merge_chunks(W.tm, W.ts, W.targ, base, np, pl.greedy, cd);
    rec.tm = t.m; rec.ts = t.s; rec.targ = t.arg;
    valid = valid && finitef(t.m);
  }

  float xd = 0.0f, yd = 0.0f;
  if (d_ok) {
    if (pl.readT) xd = load_logit<In>(trow_ptr<In>(P, b, j), d);
    if (pl.readD) yd = load_logit<In>(drow_ptr<In>(P, b, j), d);
  }

  if (pl.readD) {
    const Merged q = merge_chunks(W.dm, W.ds, W.darg, base, np, pl.greedy, cd);
    if (pl.topf) {
      // Fork candidates: merge the chunks' lists, keep the top f.
      TopList<F> mine;
      mine.clear();
      for (int ch = lane; ch < np; ch += kLanes) {
#pragma unroll
        for (int r = 0; r < F; ++r)
          mine.insert(ld_dev(W.dtv + (base + ch) * F + r), ld_dev(W.dti + (base + ch) * F + r));
      }
      TopList<F> top;
      wave_merge_lists<F>(mine, P.f, top);
      // Masked softmax at tau of the selected tokens: 2^((v - m') c) / S'.
      // Staged in the workspace; the sequence's last wave writes the outputs.
      if (lane == 0) {
#pragma unroll
        for (int r = 0; r < F; ++r) {
          if (r < P.f) {
            float pr;
            if (pl.greedy) pr = (r == 0) ? 1.0f : 0.0f;
            else if (!finitef(q.m) || !(top.v[r] > neg_inf())) pr = 0.0f;
            else pr = (float)(exp2(((double)top.v[r] - (double)q.m) * cd) / q.s);
            st_dev(W.ftok + slot * F + r, top.i[r]);
            st_dev(W.fprob + slot * F + r, pr);
          }
        }
      }
      if (j < k) {
        // Unmasked draft statistics from the masked ones and y_d.
        if (d_ok) {
          const float mfull = fmaxf(q.m, yd);
          rec.dm = mfull;
          if (!pl.greedy && finitef(mfull)) {
            double s = exp2(((double)yd - (double)mfull) * cd);
            if (q.m > neg_inf()) s += q.s * exp2(((double)q.m - (double)mfull) * cd);
            rec.ds = s;
          }
          rec.darg = (better(yd, d, top.v[0], top.i[0])) ? d : top.i[0];
        }
        valid = valid && d_ok && finitef(rec.dm);
      } else {
        rec.dm = q.m; rec.ds = q.s; rec.darg = top.i[0];
        valid = valid && finitef(q.m);
      }
    } else {
      rec.dm = q.m; rec.ds = q.s; rec.darg = q.arg;
      valid = valid && finitef(q.m);
    }
  }

  // p(d), q(d) for the acceptance test and the optional outputs.
  if (P.mode == kVerify && j < k) {
    valid = valid && d_ok;
    if (valid) {
      if (pl.greedy) {
        rec.pd = (d == rec.targ) ? 1.0 : 0.0;
        rec.qd = pl.readD ? ((d == rec.darg) ? 1.0 : 0.0) : (double)nan;
      } else {
        rec.pd = exp2(((double)xd - (double)rec.tm) * cd) / rec.ts;
        rec.qd = exp2(((double)yd - (double)rec.dm) * cd) / rec.ds;
      }
    }
  }
  rec.valid = valid ? 1 : 0;
  if (lane == 0) store_row(&W.rows[slot], rec);

  if (P.mode == kSoftmax) return;
  const unsigned rows_per_seq = (P.mode == kResidual && !P.rows_all) ? 1u : (unsigned)K1;
  if (!arrive_last(&W.seq_ctr[(int64_t)b * kCtrStride], rows_per_seq)) return;
  finalize_sequence(P, b);
}

// The drafted token leaves the draft row's masked statistics: the element
// is set to -inf in the lane that holds it (rare: one chunk per row).
template <typename In>
struct Vec4 {
  uint4 v[kU];
};

template <typename In>
__device__ __noinline__ Vec4<In> mask_token(uint4 v0, uint4 v1, uint4 v2, uint4 v3, int64_t cstart,
                                            int64_t mask_id) {
  constexpr int VEC = Elem<In>::VEC;
  static_assert(kU == 4, "mask_token takes four vectors");
  Vec4<In> r;
  r.v[0] = v0; r.v[1] = v1; r.v[2] = v2; r.v[3] = v3;
  const int lane = lane_id();
#pragma unroll
  for (int u = 0; u < kU; ++u) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      if (cstart + (int64_t)(u * kLanes + lane) * VEC + e == mask_id) set_neg_inf<In>(r.v[u], e);
    }
  }
  return r;
}

// Fork-candidate state of one wave (the buffer lives in LDS).
struct WaveCand {
  float* cv;
  int* ci;
  CandState st;
};

// One chunk of one row segment, already in registers.  RT / RD: the target
// / draft row is read; GREEDY: temperature 0.
template <typename In, int F, bool RT, bool RD, bool GREEDY>
__device__ __forceinline__ void stats_chunk(const Params& P, const RowPlan& pl, uint4 (&traw)[kU],
                                            uint4 (&draw)[kU], int ch, bool first, float c,
                                            LaneStats& ta, LaneStats& da, WaveCand& wc) {
  constexpr int CH = chunk_elems<In>();
  const int64_t cstart = (int64_t)ch * CH;
  if constexpr (RT) {
    if constexpr (GREEDY) {
      float m8[kU], mc;
      fold_greedy<In>(ta, traw, cstart, true, m8, mc);
    } else {
      float vs[kU], lm;
      fold_warm<In>(ta, traw, c, first, vs, lm);
    }
  }
  if constexpr (RD) {
    if (pl.mask_id >= cstart && pl.mask_id < cstart + CH) {
      const Vec4<In> m = mask_token<In>(draw[0], draw[1], draw[2], draw[3], cstart, pl.mask_id);
#pragma unroll
      for (int u = 0; u < kU; ++u) draw[u] = m.v[u];
    }
    unsigned candbits = 0;
    if constexpr (GREEDY) {
      float m8[kU], mc;
      fold_greedy<In>(da, draw, cstart, !pl.topf, m8, mc);
      if constexpr (F > 0) {
        if (pl.topf) {
          if (first) wc.st.kv = wave_fth_largest<F>(mc, F);
#pragma unroll
          for (int u = 0; u < kU; ++u) candbits |= (m8[u] >= wc.st.kv) ? (1u << u) : 0u;
        }
      }
    } else {
      float vs[kU], lm;
      fold_warm<In>(da, draw, c, first, vs, lm);
      if constexpr (F > 0) {
        if (pl.topf) {
          if (first) {
            // every element of the chunk's top-F reaches the F-th largest lane
            // maximum; the first chunk's candidates are all its vectors there
            wc.st.kv = wave_fth_largest<F>(lm, F);
            candbits = 0xFu;
          } else {
            // an element at or above kv has a term 2^(x c - hi) of at least
            // 2^(kv c - hi); a vector whose sum of terms is below that (less a
            // margin for rounding) has no such element
            const float eth = __builtin_amdgcn_exp2f(fmaf(wc.st.kv, c, -da.hi)) * 0.999999f;
#pragma unroll
            for (int u = 0; u < kU; ++u) candbits |= (vs[u] >= eth) ? (1u << u) : 0u;
          }
        }
      }
    }
    if constexpr (F > 0) {
      if (pl.topf) {
        if (__ballot(candbits != 0u))
          wc.st = cand_chunk<In, F>(draw[0], draw[1], draw[2], draw[3], candbits, cstart, P.V,
                                    pl.mask_id, wc.cv, wc.ci, wc.st);
        if (first) wc.st = cand_compact<F>(wc.cv, wc.ci, wc.st);
      }
    }
  }
}

// A row segment [c0, c1): full chunks [c0, cfull), then at most one partial
// chunk.  Target and draft loads of a chunk are issued together.
template <typename In, int F, bool RT, bool RD, bool GREEDY>
__device__ __forceinline__ void stats_segment(const Params& P, const RowPlan& pl, const In* trow,
                                              const In* drow, int c0, int c1, int cfull, float c,
                                              LaneStats& ta, LaneStats& da, WaveCand& wc) {
  constexpr int CH = chunk_elems<In>();
  for (int ch = c0; ch < c1; ++ch) {
    const bool full = ch < cfull;
    uint4 t[kU], d[kU];
    if constexpr (RT) load_chunk<In>(trow, (int64_t)ch * CH, P.V, full, t);
    if constexpr (RD) load_chunk<In>(drow, (int64_t)ch * CH, P.V, full, d);
    stats_chunk<In, F, RT, RD, GREEDY>(P, pl, t, d, ch, ch == c0, c, ta, da, wc);
  }
}

// Occupancy target of the statistics kernel (waves per SIMD); 0 leaves the
// register budget to the compiler.
#ifndef SV_STATS_WAVES_PER_EU
#define SV_STATS_WAVES_PER_EU 0
#endif
#if SV_STATS_WAVES_PER_EU > 0
#define SV_STATS_ATTR __attribute__((amdgpu_waves_per_eu(SV_STATS_WAVES_PER_EU, 8)))
#else
#define SV_STATS_ATTR
#endif

template <typename In, int F>
__global__ __launch_bounds__(kBlock) SV_STATS_ATTR void k_stats(Params P) {
  constexpr int CH = chunk_elems<In>();
  const int64_t task = wave_global_id();
  if (task >= P.nslots * P.nseg) return;
  const int64_t slot = task / P.nseg;
  const int seg = (int)(task - slot * P.nseg);
  int b, j;
  slot_to_bj(P, slot, b, j);
  b = uniform(b);
  j = uniform(j);
  const float tau = uniform(slot_tau(P, slot, b));
  const RowPlan pl = plan_row(P, b, j, tau);
  const float c = pl.greedy ? 0.0f : scale_of(tau);
  const int lane = lane_id();
  const Ws& W = P.ws;
  const int c0 = seg * P.seg_chunks;
  const int c1 = min(c0 + P.seg_chunks, P.cpr);
  const int cfull = min(c1, max(c0, P.V / CH));  // chunks [c0, cfull) lie inside the row
  const In* trow = pl.readT ? trow_ptr<In>(P, b, j) : nullptr;
  const In* drow = pl.readD ? drow_ptr<In>(P, b, j) : nullptr;

  LaneStats ta, da;
  lane_init(ta);
  lane_init(da);
  __shared__ float s_cv[kWavesPerBlock * kCandCap];
  __shared__ int s_ci[kWavesPerBlock * kCandCap];
  const int wib = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  WaveCand cb;
  cb.cv = s_cv + wib * kCandCap;
  cb.ci = s_ci + wib * kCandCap;
  cb.st.n = 0;
  cb.st.kv = neg_inf();
  // specialised loops: which rows are read and whether the row is greedy
  if (pl.readT && pl.readD) {
    if (pl.greedy) stats_segment<In, F, true, true, true>(P, pl, trow, drow, c0, c1, cfull, c, ta, da, cb);
    else stats_segment<In, F, true, true, false>(P, pl, trow, drow, c0, c1, cfull, c, ta, da, cb);
  } else if (pl.readT) {
    if (pl.greedy) stats_segment<In, F, true, false, true>(P, pl, trow, drow, c0, c1, cfull, c, ta, da, cb);
    else stats_segment<In, F, true, false, false>(P, pl, trow, drow, c0, c1, cfull, c, ta, da, cb);
  } else if (pl.readD) {
    if (pl.greedy) stats_segment<In, F, false, true, true>(P, pl, trow, drow, c0, c1, cfull, c, ta, da, cb);
    else stats_segment<In, F, false, true, false>(P, pl, trow, drow, c0, c1, cfull, c, ta, da, cb);
  }
  TopList<F> wl;
  wl.clear();
  if constexpr (F > 0) {
    if (pl.topf) {
      CandBuf buf;
      buf.v = cb.cv;
      buf.id = cb.ci;
      buf.n = cb.st.n;
      buf.kv = cb.st.kv;
      cand_select<F>(buf, wl);
    }
  }

  const int64_t part = slot * P.cpr + seg;
  if (pl.readT) {
    const WaveStats w = wave_finish(ta, c, pl.greedy);
    if (lane == 0) { st_dev(W.tm + part, w.m); st_dev(W.ts + part, w.s); st_dev(W.targ + part, w.arg); }
  }
  if (pl.readD) {
    const WaveStats w = wave_finish(da, c, pl.greedy);
    if (lane == 0) {
      st_dev(W.dm + part, w.m); st_dev(W.ds + part, w.s); st_dev(W.darg + part, w.arg);
      if constexpr (F > 0) {
#pragma unroll
        for (int r = 0; r < F; ++r) {
          st_dev(W.dtv + part * F + r, wl.v[r]);
          st_dev(W.dti + part * F + r, wl.i[r]);
        }
      }
    }
  }

  if (!arrive_last(&W.row_ctr[slot * kCtrStride], (unsigned)P.nseg)) return;
  row_merge<In, F>(P, slot, b, j, tau, pl);
}

// ------------------------------------------------------------ k_resid

// Per-element residual weight r = max(0, p - q) and target probability p,
// from the merged row statistics (fp32; references split exactly as in
// chunk_stats).
struct ResidCoef {
  float c, thi, tscale, dhi, dscale;
  bool has_q;
};

__device__ __forceinline__ ResidCoef resid_coef(const RowRec& rr, float c, bool has_q) {
  ResidCoef k;
  k.c = c;
  k.thi = rr.tm * c;
  const float tlo = fmaf(rr.tm, c, -k.thi);
  k.tscale = (float)(exp2(-(double)tlo) / rr.ts);
  k.has_q = has_q;
  k.dhi = 0.0f;
  k.dscale = 0.0f;
  if (has_q) {
    k.dhi = rr.dm * c;
    const float dlo = fmaf(rr.dm, c, -k.dhi);
    k.dscale = (float)(exp2(-(double)dlo) / rr.ds);
  }
  return k;
}

__device__ __forceinline__ void resid_elem(const ResidCoef& k, float x, float y, float& p, float& r) {
  p = __builtin_amdgcn_exp2f(fmaf(x, k.c, -k.thi)) * k.tscale;
  if (k.has_q) {
    const float q = __builtin_amdgcn_exp2f(fmaf(y, k.c, -k.dhi)) * k.dscale;
    r = fmaxf(p - q, 0.0f);
  } else {
    r = p;
  }
}

// Weights of one 16-byte vector: w[e] = r (residual) or p, e in element order.
template <typename In>
__device__ __forceinline__ void resid_vec(const ResidCoef& kc, const uint4& tv, const uint4& dv,
                                          float (&r)[Elem<In>::VEC], float (&p)[Elem<In>::VEC]) {
#pragma unroll
  for (int e = 0; e < Elem<In>::VEC; ++e)
    resid_elem(kc, elem<In>(tv, e), kc.has_q ? elem<In>(dv, e) : 0.0f, p[e], r[e]);
}

// Pairwise fp32 sum of one vector's weights (fixed order).
template <int N>
__device__ __forceinline__ float vec_sum(const float (&w)[N]) {
  float a[N];
#pragma unroll
  for (int e = 0; e < N; ++e) a[e] = w[e];
#pragma unroll
  for (int h = N / 2; h > 0; h >>= 1) {
#pragma unroll
    for (int e = 0; e < h; ++e) a[e] = a[e] + a[e + h];
  }
  return a[0];
}

// k_resid slot -> (b, j, record slot).
__device__ __forceinline__ void resid_slot(const Params& P, int64_t slot, int& b, int& j,
                                           int64_t& rslot, bool& draw_row) {
  const int K1 = P.k + 1;
  if (P.mode == kResidual && P.rows_all) {
    b = (int)(slot / K1);
    j = (int)(slot - (int64_t)b * K1);
    rslot = slot;
    draw_row = (j == P.ws.seqs[b].n);
  } else {
    b = (int)slot;
    j = P.ws.seqs[b].n;
    rslot = (P.mode == kVerify) ? (int64_t)b * K1 + j : (int64_t)b;
    draw_row = true;
  }
}

// The draw of one row, by the wave that finished its residual sums.  Token
// order inside a chunk is slab by slab: slab u holds vector u of lanes
// 0..63, i.e. 64 consecutive 16-byte vectors.  The chunk holding the target
// is found from the chunk sums, the slab from that chunk's slab sums, the
// lane from a scan of one re-read slab, and the token inside the lane's
// vector.  Every step keeps to tokens of positive weight: the token is the
// first one whose running total passes u*Z, or the last positive one if
// rounding leaves none.
template <typename In>
__device__ __forceinline__ void resid_draw(const Params& P, int64_t slot, int b, int j,
                                           const ResidCoef& kc, double Zr, double Zp) {
  constexpr int VEC = Elem<In>::VEC;
  constexpr int CH = chunk_elems<In>();
  const int lane = lane_id();
  const int cpr = P.cpr;
  const bool use_r = (j < P.k) && Zr > 0.0;
  const double Z = use_r ? Zr : Zp;
  const double* slabs = use_r ? P.ws.kr : P.ws.kp;
  const double target = (double)P.u_rec[(int64_t)b * (P.k + 1) + j] * Z;
  const int64_t sbase = slot * (int64_t)cpr * kU;

  // 1. chunk: first whose inclusive prefix passes the target
  int cstar = -1, clast = -1;
  double before = 0.0, before_last = 0.0, carry = 0.0;
  double sl[kU], sl_last[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) { sl[u] = 0.0; sl_last[u] = 0.0; }
  for (int g = 0; g < cpr; g += kLanes) {
    const int ch = g + lane;
    double v[kU];
    double w = 0.0;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      v[u] = ch < cpr ? ld_dev(slabs + sbase + (int64_t)ch * kU + u) : 0.0;
      w += v[u];
    }
    const double incl = carry + wave_inclusive_scan(w);
    double excl = __shfl_up(incl, 1);
    if (lane == 0) excl = carry;
    const unsigned long long hit = __ballot(ch < cpr && w > 0.0 && incl > target);
    if (cstar < 0 && hit) {
      const int l = __ffsll((long long)hit) - 1;
      cstar = g + l;
      before = readlane_d(excl, l);
#pragma unroll
      for (int u = 0; u < kU; ++u) sl[u] = readlane_d(v[u], l);
    }
    const unsigned long long posm = __ballot(ch < cpr && w > 0.0);
    if (posm) {
      const int l = 63 - __clzll((long long)posm);
      clast = g + l;
      before_last = readlane_d(excl, l);
#pragma unroll
      for (int u = 0; u < kU; ++u) sl_last[u] = readlane_d(v[u], l);
    }
    carry = readlane_d(incl, kLanes - 1);
  }
  if (cstar < 0) {
    cstar = clast;
    before = before_last;
#pragma unroll
    for (int u = 0; u < kU; ++u) sl[u] = sl_last[u];
  }
  if (cstar < 0) { cstar = 0; before = 0.0; }

  // 2. slab inside that chunk (uniform)
  int ustar = -1, ulast = 0;
  double ubefore = before, ubefore_last = before, run = before;
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    if (sl[u] > 0.0) {
      if (ustar < 0 && run + sl[u] > target) { ustar = u; ubefore = run; }
      ulast = u;
      ubefore_last = run;
    }
    run += sl[u];
  }
  if (ustar < 0) { ustar = ulast; ubefore = ubefore_last; }

  // 3. re-read that slab (one vector per lane) and find the lane
  const int64_t cstart = (int64_t)cstar * CH;
  const int64_t e0 = cstart + (int64_t)(ustar * kLanes + lane) * VEC;
  float w[VEC];
  {
    uint4 tv = make_uint4(0, 0, 0, 0), dv = make_uint4(0, 0, 0, 0);
    const In* tr = trow_ptr<In>(P, b, j);
    const In* dr = kc.has_q ? drow_ptr<In>(P, b, j) : nullptr;
    load_vec<In>(tr, e0, P.V, tv);
    if (kc.has_q) load_vec<In>(dr, e0, P.V, dv);
    float r[VEC], p[VEC];
    resid_vec<In>(kc, tv, dv, r, p);
#pragma unroll
    for (int e = 0; e < VEC; ++e) w[e] = (e0 + e < P.V) ? (use_r ? r[e] : p[e]) : 0.0f;
  }
  const float vt = vec_sum<VEC>(w);
  const double incl = ubefore + wave_inclusive_scan((double)vt);
  double excl = __shfl_up(incl, 1);
  if (lane == 0) excl = ubefore;
  const unsigned long long hit = __ballot(vt > 0.0f && incl > target);
  const unsigned long long posm = __ballot(vt > 0.0f);
  const int lstar = hit ? (__ffsll((long long)hit) - 1) : (posm ? 63 - __clzll((long long)posm) : 0);

  // 4. the token inside lane lstar's vector
  int t = -1, vlast = -1;
  float acc = 0.0f;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    acc += w[e];
    if (w[e] > 0.0f) {
      vlast = (int)(e0 + e);
      if (t < 0 && excl + (double)acc > target) t = (int)(e0 + e);
    }
  }
  if (t < 0) t = vlast;
  const int tok = readlane_i(t, lstar);
  if (lane == 0) P.out_token[b] = tok;
}

template <typename In>
__global__ __launch_bounds__(kBlock) void k_resid(Params P) {
  constexpr int CH = chunk_elems<In>();
  constexpr int VEC = Elem<In>::VEC;
  const int64_t task = wave_global_id();
  const int64_t nslots = (P.mode == kResidual && P.rows_all) ? (int64_t)P.B * (P.k + 1) : P.B;
  if (task >= nslots * P.cpr) return;
  const int64_t slot = task / P.cpr;
  const int chunk = (int)(task - slot * P.cpr);
  int b = (int)((P.mode == kResidual && P.rows_all) ? slot / (P.k + 1) : slot);
  b = uniform(b);
  if (P.ws.seqs[b].status != 2) return;
  int j;
  int64_t rslot;
  bool draw_row;
  resid_slot(P, slot, b, j, rslot, draw_row);
  j = uniform(j);
  const RowRec rr = P.ws.rows[rslot];
  const float c = scale_of(P.tau[b]);
  const bool has_q = j < P.k;
  const ResidCoef kc = resid_coef(rr, c, has_q);

  const int64_t cstart = (int64_t)chunk * CH;
  const bool full = cstart + CH <= P.V;
  uint4 traw[kU], draw[kU];
  load_chunk<In>(trow_ptr<In>(P, b, j), cstart, P.V, full, traw);
  if (has_q) load_chunk<In>(drow_ptr<In>(P, b, j), cstart, P.V, full, draw);
  // slab sums of r and p (padding reads -inf: weight 0)
  const int64_t sbase = (slot * (int64_t)P.cpr + chunk) * kU;
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    float r[VEC], p[VEC];
    resid_vec<In>(kc, traw[u], draw[u], r, p);
    const double sr = wave_sum((double)vec_sum<VEC>(r));
    const double sp = wave_sum((double)vec_sum<VEC>(p));
    if (lane_id() == 0) {
      st_dev(P.ws.kr + sbase + u, sr);
      st_dev(P.ws.kp + sbase + u, sp);
    }
  }
  if (!arrive_last(&P.ws.k2_ctr[slot * kCtrStride], (unsigned)P.cpr)) return;

  // Row totals, in chunk order.
  const int lane = lane_id();
  double carry_r = 0.0, carry_p = 0.0;
  const int64_t rbase = slot * (int64_t)P.cpr * kU;
  for (int g = 0; g < P.cpr; g += kLanes) {
    const int ch = g + lane;
    double wr = 0.0, wp = 0.0;
    if (ch < P.cpr) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        wr += ld_dev(P.ws.kr + rbase + (int64_t)ch * kU + u);
        wp += ld_dev(P.ws.kp + rbase + (int64_t)ch * kU + u);
      }
    }
    carry_r = readlane_d(carry_r + wave_inclusive_scan(wr), kLanes - 1);
    carry_p = readlane_d(carry_p + wave_inclusive_scan(wp), kLanes - 1);
  }
  if (lane == 0) {
    P.ws.rows[rslot].zr = carry_r;
    P.ws.rows[rslot].zp = carry_p;
  }
  if (draw_row) resid_draw<In>(P, slot, b, j, kc, carry_r, carry_p);
}

// ------------------------------------------------------------ k_write

// Normalised outputs: softmax rows (sv_softmax_temp) or residual
// distributions (sv_residual_sample).
template <typename In>
__global__ __launch_bounds__(kBlock) void k_write(Params P) {
  constexpr int VEC = Elem<In>::VEC;
  constexpr int CH = chunk_elems<In>();
  const int64_t task = wave_global_id();
  const int64_t nslots = (P.mode == kSoftmax) ? P.nslots : (int64_t)P.B * (P.k + 1);
  if (task >= nslots * P.cpr) return;
  const int64_t slot = task / P.cpr;
  const int chunk = (int)(task - slot * P.cpr);
  const int lane = lane_id();
  const float nan = __uint_as_float(0x7fc00000u);

  int b, j;
  float* orow;
  int state;  // 0 NaN, 1 one-hot, 2 values
  float tau;
  if (P.mode == kSoftmax) {
    b = (int)slot; j = 0;
    tau = P.tau[slot / P.rows_per_temp];
    orow = P.out + slot * P.out_row;
    const RowRec& rr = P.ws.rows[slot];
    state = !rr.valid ? 0 : (tau == 0.0f ? 1 : 2);
  } else {
    b = (int)(slot / (P.k + 1));
    j = (int)(slot - (int64_t)b * (P.k + 1));
    tau = P.tau[b];
    orow = P.out + (int64_t)b * P.out_seq + (int64_t)j * P.out_row;
    const int st = P.ws.seqs[b].status;
    state = (st == 0) ? 0 : (tau == 0.0f ? 1 : 2);
  }
  b = uniform(b); j = uniform(j); state = uniform(state);
  const RowRec rr = P.ws.rows[slot];
  const int64_t cstart = (int64_t)chunk * CH;
  const bool full = cstart + CH <= P.V;

  uint4 traw[kU], draw[kU];
  ResidCoef kc;
  float inv_z = 1.0f;
  bool use_r = false;
  if (state == 2) {
    const bool has_q = (P.mode == kResidual) && j < P.k;
    kc = resid_coef(rr, scale_of(tau), has_q);
    use_r = has_q && rr.zr > 0.0;
    if (use_r) inv_z = (float)(1.0 / rr.zr);
    const In* tr = (P.mode == kSoftmax)
        ? reinterpret_cast<const In*>(P.T) + slot * P.t_row
        : trow_ptr<In>(P, b, j);
    load_chunk<In>(tr, cstart, P.V, full, traw);
    if (has_q) load_chunk<In>(drow_ptr<In>(P, b, j), cstart, P.V, full, draw);
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t e0 = cstart + (int64_t)(u * kLanes + lane) * VEC;
    float o[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      if (state == 0) {
        o[e] = nan;
      } else if (state == 1) {
        o[e] = (e0 + e == rr.targ) ? 1.0f : 0.0f;
      } else {
        float p, r;
        resid_elem(kc, elem<In>(traw[u], e), kc.has_q ? elem<In>(draw[u], e) : 0.0f, p, r);
        o[e] = use_r ? r * inv_z : p;
      }
    }
    if (full || e0 + VEC <= P.V) {
#pragma unroll
      for (int h = 0; h < VEC; h += 4)
        *reinterpret_cast<float4*>(orow + e0 + h) = make_float4(o[h], o[h + 1], o[h + 2], o[h + 3]);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        if (e0 + e < P.V) orow[e0 + e] = o[e];
    }
  }
}

// ------------------------------------------------------------ fill

__global__ __launch_bounds__(kBlock) void k_fill_zero(uint8_t* p, size_t bytes) {
  const size_t n16 = bytes / 16;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    reinterpret_cast<uint4*>(p)[i] = make_uint4(0, 0, 0, 0);
  const size_t tail = bytes - n16 * 16;
  if (blockIdx.x == 0 && threadIdx.x < tail) p[n16 * 16 + threadIdx.x] = 0;
}

// ------------------------------------------------------------ host side

struct Layout {
  size_t row_ctr, seq_ctr, k2_ctr, tm, ts, targ, dm, ds, darg, dtv, dti, ftok, fprob, rows, seqs,
      kr, kp, total;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Candidate-list length of the statistics kernel for fan-out f: 4 covers
// f <= 4, 16 covers the rest (the top-F contain the top-f).
static int fork_F(int f) {
  if (f <= 0) return 0;
  return f <= 4 ? 4 : 16;
}

// Workspace layout for R row slots, B sequences, cpr chunks per row and top
// lists of F entries.
static Layout make_layout(int64_t R, int64_t B, int64_t cpr, int F) {
  Layout L;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
  const size_t RC = (size_t)(R * cpr);
  const size_t Fa = (size_t)(F > 0 ? F : 1);
  L.row_ctr = take(sizeof(unsigned) * kCtrStride * R);
  L.seq_ctr = take(sizeof(unsigned) * kCtrStride * B);
  L.k2_ctr = take(sizeof(unsigned) * kCtrStride * R);
  L.tm = take(sizeof(float) * RC);
  L.ts = take(sizeof(double) * RC);
  L.targ = take(sizeof(int) * RC);
  L.dm = take(sizeof(float) * RC);
  L.ds = take(sizeof(double) * RC);
  L.darg = take(sizeof(int) * RC);
  L.dtv = take(sizeof(float) * RC * Fa);
  L.dti = take(sizeof(int) * RC * Fa);
  L.ftok = take(sizeof(int) * R * Fa);
  L.fprob = take(sizeof(float) * R * Fa);
  L.rows = take(sizeof(RowRec) * R);
  L.seqs = take(sizeof(SeqRec) * B);
  L.kr = take(sizeof(double) * RC * kU);
  L.kp = take(sizeof(double) * RC * kU);
  L.total = o;
  return L;
}

static Ws bind_ws(void* base, const Layout& L) {
  uint8_t* p = static_cast<uint8_t*>(base);
  Ws w;
  w.row_ctr = reinterpret_cast<unsigned*>(p + L.row_ctr);
  w.seq_ctr = reinterpret_cast<unsigned*>(p + L.seq_ctr);
  w.k2_ctr = reinterpret_cast<unsigned*>(p + L.k2_ctr);
  w.tm = reinterpret_cast<float*>(p + L.tm);
  w.ts = reinterpret_cast<double*>(p + L.ts);
  w.targ = reinterpret_cast<int*>(p + L.targ);
  w.dm = reinterpret_cast<float*>(p + L.dm);
  w.ds = reinterpret_cast<double*>(p + L.ds);
  w.darg = reinterpret_cast<int*>(p + L.darg);
  w.dtv = reinterpret_cast<float*>(p + L.dtv);
  w.dti = reinterpret_cast<int*>(p + L.dti);
  w.ftok = reinterpret_cast<int*>(p + L.ftok);
  w.fprob = reinterpret_cast<float*>(p + L.fprob);
  w.rows = reinterpret_cast<RowRec*>(p + L.rows);
  w.seqs = reinterpret_cast<SeqRec*>(p + L.seqs);
  w.kr = reinterpret_cast<double*>(p + L.kr);
  w.kp = reinterpret_cast<double*>(p + L.kp);
  return w;
}

// Chunks per row for a dtype.
static int64_t chunks_per_row(int dtype, int64_t V) {
  const int64_t ch = (dtype == SV_BF16) ? chunk_elems<uint16_t>() : chunk_elems<float>();
  return (V + ch - 1) / ch;
}

constexpr int64_t kMaxV = (int64_t)1 << 26;

static size_t workspace_bytes(int64_t R, int64_t B, int64_t V, int f) {
  const int64_t cpr = chunks_per_row(SV_F32, V);  // fp32 has the smaller chunks
  return make_layout(R, B, cpr, fork_F(f)).total;
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
  P.cpr = (int32_t)chunks_per_row(in->dtype, in->V);
  P.rows_per_temp = 1;
  return P;
}

// Segments: each k_stats wave folds seg_chunks consecutive chunks of one row.
// The segment size is chosen so that the grid is about one resident round
// of waves (CUs x 24: six waves per SIMD at the kernel's register use);
// more chunks per wave amortise the per-wave cross-lane work.
static void plan_segments(Params& P) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
  }
  const int64_t target = (int64_t)cus * 24;
  const int64_t chunks = P.nslots * (int64_t)P.cpr;
  int64_t g = (chunks + target - 1) / target;
  if (g < 1) g = 1;
  if (g > P.cpr) g = P.cpr;
  P.seg_chunks = (int32_t)g;
  P.nseg = (int32_t)((P.cpr + g - 1) / g);
}

static dim3 grid_for(int64_t waves) {
  return dim3((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock));
}

template <typename In, int F>
static hipError_t launch_stats_F(const Params& P, hipStream_t s) {
  const int64_t waves = P.nslots * P.nseg;
  if (waves == 0) return hipSuccess;
  hipLaunchKernelGGL((k_stats<In, F>), grid_for(waves), dim3(kBlock), 0, s, P);
  return hipGetLastError();
}

template <typename In>
static hipError_t launch_stats(const Params& P, hipStream_t s) {
  switch (P.F) {
    case 0: return launch_stats_F<In, 0>(P, s);
    case 4: return launch_stats_F<In, 4>(P, s);
    default: return launch_stats_F<In, 16>(P, s);
  }
}

template <typename In>
static hipError_t launch_resid(const Params& P, hipStream_t s) {
  const int64_t nslots = (P.mode == kResidual && P.rows_all) ? (int64_t)P.B * (P.k + 1) : P.B;
  const int64_t waves = nslots * P.cpr;
  if (waves == 0) return hipSuccess;
  hipLaunchKernelGGL((k_resid<In>), grid_for(waves), dim3(kBlock), 0, s, P);
  return hipGetLastError();
}

template <typename In>
static hipError_t launch_write(const Params& P, hipStream_t s) {
  const int64_t nslots = (P.mode == kSoftmax) ? P.nslots : (int64_t)P.B * (P.k + 1);
  const int64_t waves = nslots * P.cpr;
  if (waves == 0) return hipSuccess;
  hipLaunchKernelGGL((k_write<In>), grid_for(waves), dim3(kBlock), 0, s, P);
  return hipGetLastError();
}

static hipError_t dispatch_stats(int dtype, const Params& P0, hipStream_t s) {
  Params P = P0;
  plan_segments(P);
  return dtype == SV_BF16 ? launch_stats<uint16_t>(P, s) : launch_stats<float>(P, s);
}
static hipError_t dispatch_resid(int dtype, const Params& P, hipStream_t s) {
  return dtype == SV_BF16 ? launch_resid<uint16_t>(P, s) : launch_resid<float>(P, s);
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

const char* sv_version(void) { return "libspecverify 0.1.0 gfx950"; }

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
  if (dispatch_resid(in->dtype, P, s) != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

sv_status sv_verify(const sv_batch* in, const float* u_accept, const float* u_recover,
                    int32_t* accept_len, int32_t* out_token, float* p_draft, float* q_draft,
                    const sv_forks* forks, void* ws, size_t ws_bytes, void* stream) {
  return sv_verify_ex(in, u_accept, u_recover, accept_len, out_token, p_draft, q_draft, forks,
                      ws, ws_bytes, stream, nullptr);
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
  if (dispatch_resid(in->dtype, P, s) != hipSuccess) return SV_ERR_HIP;
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
  if (dispatch_stats(in->dtype, P, (hipStream_t)stream) != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

}  // extern "C"
