// Shared device code of libspecverify (gfx950): launch parameters, the
// workspace, per-row plans, the streaming statistics of one segment of a
// row, the merge of segment partials, and the residual weights and draw.
//
// The speculative-sampling rule (accept iff u < min(1, p/q), first
// rejection, draw from max(0, p - q), bonus draw from p_k) follows the
// speculative-sampling project page ("How It Works", "Highlighted
// Details", sourcepulse.org project 1842340) and the exactness requirement
// of "What changes in SSD" (hysenlabs.com editorial); the forked top-f with
// the drafted token masked follows the async-SD utilities file described in
// the tanishqkumar/ssd repository summary (thehardwarestore.ai).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "sv_device.h"
#include "sv_stats.h"

namespace sv {

constexpr double kLog2e = 1.4426950408889634074;

enum Mode : int { kVerify = 0, kForks = 1, kResidual = 2, kSoftmax = 3 };

// Largest vocabulary: the draw keeps one chunk total per chunk of a row
// (fp32 chunks hold 1024 elements).
constexpr int kMaxChunks = 1024;
constexpr int64_t kMaxV = (int64_t)kMaxChunks * kU * kLanes * 4;
constexpr int kMaxSeg = 64;   // partials per row (one lane each when merged)
constexpr int kDumpCap = 128;  // fork candidate vectors a segment passes on

// ---------------------------------------------------------------- control
// The arrival counters sit in a control header at the start of every
// workspace, at offsets that do not depend on the call's sizes, so a
// workspace zero-filled once can be reused by any entry point and any
// sizes.  Every counter is returned to zero by its last arrival, so a call
// that runs to completion leaves the header as it found it.  Counters sit
// on lines of their own: device-scope atomics to one line are serialised.
constexpr int64_t kMaxBatch = 8192;  // sequences per call
constexpr int64_t kMaxRows = 32768;  // (sequence, position) rows per call
constexpr int64_t kSeqCtlBytes = 128;
constexpr int64_t kRowCtlBytes = 64;
constexpr int64_t kCtlBytes = kMaxBatch * kSeqCtlBytes + kMaxRows * kRowCtlBytes;

// Per-sequence counters (one block of kSeqCtlBytes per sequence).
enum SeqCounter : int {
  kCtrDraw = 0,   // blocks that summed their share of the drawn row
  kCtrForks = 1,  // fork blocks that wrote their rows
  kCtrHits = 2    // inputs of the cache lookup that are written (token, forks)
};

// Row record: merged statistics of one (sequence, position) row, written
// once per call by the wave that merges the row.
struct RowRec {
  float tm;     // target reference (temperature > 0) or maximum
  int targ;     // target argmax
  double ts;    // target sum of 2^((x - tm) c)
  float dm;     // draft reference (unmasked row)
  int valid;
  double ds;    // draft sum of 2^((y - dm) c)
  double zr;    // total weight: sum of max(0, p - q), or of p at j = k
  double pd;    // p(d), q(d) at the row's drafted token (j < k)
  double qd;
};

struct SeqRec {
  int n;        // outcome position
  int status;   // 0 error, 1 finished (greedy), 2 drawn at temperature > 0
};

struct Ws {
  unsigned* seqctl;                     // control header: [kMaxBatch] blocks of kSeqCtlBytes
  unsigned* rowctl;                     // then [kMaxRows] counters kRowCtlBytes apart
  float* tm; double* ts; int* targ;     // [R * kMaxSeg] target segment partials
  float* dm; double* ds; int* darg;     // [R * kMaxSeg] draft segment partials
  float* dtv; int* dti;                 // [R * kMaxSeg * F] draft segment top-F
  RowRec* rows;                         // [R]
  SeqRec* seqs;                         // [B]
  float* xd; float* yd;                 // [R] the drafted token's logits, seen by the stream
  int* cn; int* cpos; float* cvm;       // [R * kMaxSeg], [R * kMaxSeg * kDumpCap] x 2: fork
                                        // candidate vectors (position, maximum)
  double* ctr;                          // [R * cpr] chunk totals of residual weights
};

__device__ __forceinline__ unsigned* seq_ctr(const Ws& W, int64_t b, int which) {
  return reinterpret_cast<unsigned*>(reinterpret_cast<char*>(W.seqctl) + b * kSeqCtlBytes) +
         which;
}
__device__ __forceinline__ unsigned* row_ctr(const Ws& W, int64_t slot) {
  return reinterpret_cast<unsigned*>(reinterpret_cast<char*>(W.rowctl) + slot * kRowCtlBytes);
}

struct Params {
  const void* T; int64_t t_seq, t_row;
  const void* D; int64_t d_seq, d_row;
  const int32_t* drafts;
  const float* tau;
  const float* u_acc;
  const float* u_rec;
  const int32_t* position;
  int32_t B, k, V, f, F, mode, rows_all, want_q;
  int32_t cpr;             // chunks per row
  int32_t nslab;           // slabs per row
  int32_t nparts;          // segments (partials) per row
  int32_t nbs;             // block-level decide: blocks per task row
  int32_t fsplit;          // block-level decide: fork blocks per sequence
  int64_t nslots;          // row slots of the stream
  int64_t rows_per_temp;   // softmax
  int32_t* accept_len;
  int32_t* out_token;
  float* p_draft;
  float* q_draft;
  int32_t* fork_tok;
  float* fork_prob;
  int32_t* hits;
  float* out; int64_t out_seq, out_row;
  Ws ws;
};

// Touches every 64-byte line of the kernel's argument block with scalar
// loads issued together, so that the argument loads the code makes later,
// some of them only after earlier ones return, find the lines in the
// scalar cache.
__device__ __forceinline__ void warm_kernargs() {
  typedef __attribute__((address_space(4))) const uint32_t KWord;
  KWord* kp = (KWord*)__builtin_amdgcn_kernarg_segment_ptr();
  uint32_t acc = 0;
#pragma unroll
  for (int off = 0; off < (int)sizeof(Params); off += 64) acc |= kp[off / 4];
  asm volatile("" ::"s"(acc));
}

__device__ __forceinline__ bool tau_ok(float t) { return t >= 0.0f && t < pos_inf(); }

__device__ __forceinline__ float slot_tau(const Params& P, int64_t slot, int b) {
  if (P.mode == kSoftmax) return P.tau[slot / P.rows_per_temp];
  return P.tau[b];
}

// Row slot -> (sequence, position) of k_stats.
__device__ __forceinline__ void slot_to_bj(const Params& P, int64_t slot, int& b, int& j) {
  if (P.mode == kSoftmax) { b = (int)slot; j = 0; return; }
  if (P.mode == kResidual && !P.rows_all) { b = (int)slot; j = P.position[b]; return; }
  b = (int)(slot / (P.k + 1));
  j = (int)(slot - (int64_t)b * (P.k + 1));
}

// Slot of row (b, j) in the partial arrays.
__device__ __forceinline__ int64_t slot_of(const Params& P, int b, int j) {
  if (P.mode == kResidual && !P.rows_all) return b;
  return (int64_t)b * (P.k + 1) + j;
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
  int mask_id;  // element left out of the draft's masked statistics (-1: none)
  int d_id;     // the drafted token of the row (-1: none)
  int nf;       // forks asked for (f <= F)
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
  r.d_id = -1;
  r.nf = P.f;
  if (r.pos_ok && j < P.k && P.mode != kSoftmax) {
    const int d = P.drafts[(int64_t)b * P.k + j];
    r.d_id = d;  // out-of-range ids match no element
    if (r.topf) r.mask_id = d;
  }
  return r;
}

// ================================================================ k_stats

// The drafted token leaves the draft row's masked statistics: the element
// is set to -inf in the lane that holds it (one chunk per row).
template <typename In>
struct Vec4 {
  uint4 v[kU];
};

template <typename In>
__device__ __noinline__ Vec4<In> mask_token(uint4 v0, uint4 v1, uint4 v2, uint4 v3, int e_base,
                                            int mask_id) {
  constexpr int VEC = Elem<In>::VEC;
  static_assert(kU == 4, "mask_token takes four vectors");
  Vec4<In> r;
  r.v[0] = v0; r.v[1] = v1; r.v[2] = v2; r.v[3] = v3;
#pragma unroll
  for (int u = 0; u < kU; ++u) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      if (e_base + u * slab_elems<In>() + e == mask_id) set_neg_inf<In>(r.v[u], e);
    }
  }
  return r;
}

// The value of element `id` if this lane holds it in the chunk (else -inf),
// and whether it does.
template <typename In>
__device__ __noinline__ float2 pick_elem(uint4 v0, uint4 v1, uint4 v2, uint4 v3, int e_base,
                                         int id) {
  constexpr int VEC = Elem<In>::VEC;
  static_assert(kU == 4, "pick_elem takes four vectors");
  const uint4 raw[kU] = {v0, v1, v2, v3};
  float x = neg_inf(), found = 0.0f;
#pragma unroll
  for (int u = 0; u < kU; ++u) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      if (e_base + u * slab_elems<In>() + e == id) { x = elem<In>(raw[u], e); found = 1.0f; }
    }
  }
  return make_float2(x, found);
}

struct WaveState {
  Warm tw, dw;    // temperature > 0
  Greedy tg, dg;  // temperature 0
  int nc;         // fork candidate slots in use (this lane)
  float kv;       // fork candidate threshold (wave-uniform)
  float eth;      // this lane's term of an element at kv, 2^(kv c - hi), less a margin
};

// Recomputes st.eth after kv or the draft reference changed.
__device__ __forceinline__ void refresh_eth(WaveState& st, float c) {
  st.eth = __builtin_amdgcn_exp2f(fmaf(st.kv, c, -st.dw.hi)) * 0.999999f;
}

// Writes element id of a chunk (held by one lane, if any) to *out.
template <typename In>
__device__ __forceinline__ void capture(const uint4 (&raw)[kU], int e_base, int id, float* out) {
  const float2 r = pick_elem<In>(raw[0], raw[1], raw[2], raw[3], e_base, id);
  if (r.y != 0.0f) *out = r.x;
}

// One chunk of a segment, already in registers.  RT / RD: the target / draft
// row is read; GREEDY: temperature 0; FIRST: the segment's first chunk.
// cs: the chunk's first element (wave-uniform); e_base = cs + lane * VEC;
// nv: vectors of the chunk inside the segment (the others read as -inf).
// The drafted token's logits are written to xd / yd when the chunk holds it.
template <typename In, int F, bool RT, bool RD, bool GREEDY, bool FIRST>
__device__ __forceinline__ void stats_chunk(const RowPlan& pl, int V, const In* drow,
                                            const uint4 (&traw)[kU], uint4 (&draw)[kU],
                                            int cs, int e_base, int nv, float c, WaveState& st,
                                            CandLds<F>* L, float* xd, float* yd) {
  constexpr int SLAB = slab_elems<In>();
  constexpr int CH = chunk_elems<In>();
  // only vectors [0, nv) of the chunk belong to this segment
  const bool has_d = pl.d_id >= cs && pl.d_id < cs + nv * SLAB;
  if constexpr (RT) {
    if (has_d) capture<In>(traw, e_base, pl.d_id, xd);
  }
  if constexpr (RD) {
    if (has_d) capture<In>(draw, e_base, pl.d_id, yd);
    if (pl.mask_id >= cs && pl.mask_id < cs + CH) {
      const Vec4<In> m = mask_token<In>(draw[0], draw[1], draw[2], draw[3], e_base, pl.mask_id);
#pragma unroll
      for (int u = 0; u < kU; ++u) draw[u] = m.v[u];
    }
  }
  // fold: running maxima at temperature 0 (with forks the draft's (masked)
  // argmax is kept too: it gives the unmasked argmax together with the
  // drafted token's logit), sums of terms above it
  float m8[kU], vs[kU];  // the draft chunk's vector maxima and sums of terms
  bool d_fixed = false;  // some draft lane's reference was raised
  if constexpr (RT) {
    float m8t[kU];
    if constexpr (GREEDY) greedy_fold<In>(st.tg, traw, e_base, true, m8t);
    else warm_fold<In, FIRST>(st.tw, traw, c, m8t);
  }
  if constexpr (RD) {
    if constexpr (GREEDY) greedy_fold<In>(st.dg, draw, e_base, true, m8);
    else warm_fold_vs<In, FIRST>(st.dw, draw, c, m8, vs, d_fixed);
  }
  if constexpr (RD && F > 0) {
    if (pl.topf) {
      unsigned bits = 0;
      constexpr bool have_m8 = FIRST || GREEDY;
      if constexpr (FIRST) {
        // at least f vectors reach the f-th largest lane maximum, so every
        // element of the segment's top-f does; the first chunk's
        // candidates are the vectors there
        float lm = m8[0];
#pragma unroll
        for (int u = 1; u < kU; ++u) lm = fmaxf(lm, m8[u]);
        st.kv = wave_fth_largest<F>(lm, pl.nf);
#pragma unroll
        for (int u = 0; u < kU; ++u) bits |= (m8[u] >= st.kv) ? (1u << u) : 0u;
        if constexpr (!GREEDY) refresh_eth(st, c);
      } else if (!(st.kv > neg_inf())) {
        bits = (1u << kU) - 1u;  // fewer than f elements seen: all are candidates
      } else if constexpr (GREEDY) {
#pragma unroll
        for (int u = 0; u < kU; ++u) bits |= (m8[u] > st.kv) ? (1u << u) : 0u;
      } else {
        // an element above kv has a term 2^(x c - hi) of more than
        // 2^(kv c - hi) (st.eth, less a margin for rounding); a vector whose
        // sum of terms is below that holds no such element.  The chunk's
        // largest vector sum is tested first.
        if (d_fixed) refresh_eth(st, c);
        const float vmax = fmaxf(fmaxf(vs[0], vs[1]), fmaxf(vs[2], vs[3]));
        if (__ballot(vmax >= st.eth)) {
#pragma unroll
          for (int u = 0; u < kU; ++u) bits |= (vs[u] >= st.eth) ? (1u << u) : 0u;
        }
      }
      bits &= (1u << nv) - 1u;  // vectors past the segment belong to the next one
      if (__ballot(bits != 0u)) {
        // the maxima are exact where they were computed (first chunk,
        // temperature 0); elsewhere the candidate is passed on as inexact,
        // with the key that bounds its maximum
        if constexpr (!have_m8) {
#pragma unroll
          for (int u = 0; u < kU; ++u) m8[u] = inexact_key(vs[u], st.dw.hi);
        }
        cand_append<F>(L, bits, e_base, SLAB, m8, have_m8, st.nc);
        if (__ballot(st.nc > kCandSlots - kU)) {
          cand_reduce<In, F, 2>(L, drow, V, pl.mask_id, st.nc, st.kv);
          if constexpr (!GREEDY) refresh_eth(st, c);
        }
      }
    }
  }
}

// A segment of slabs [s0, s1) of one row, a chunk (kU slabs) at a time; the
// next chunk's loads are issued before the current chunk is folded.
template <typename In, int F, bool RT, bool RD, bool GREEDY>
__device__ __forceinline__ void stats_segment(const RowPlan& pl, int V, const In* trow,
                                              const In* drow, int s0, int s1, float c,
                                              WaveState& st, CandLds<F>* L, float* xd,
                                              float* yd) {
  constexpr int SLAB = slab_elems<In>();
  constexpr int VEC = Elem<In>::VEC;
  const int lane = lane_id();
  const int nch = (s1 - s0 + kU - 1) / kU;
  const int slim = min(s1, V / SLAB);  // slabs [.., slim) lie inside the row
  uint4 ta[kU], da[kU], tb[kU], db[kU];
  auto load = [&](uint4 (&t)[kU], uint4 (&d)[kU], int i) {
    const int sl = s0 + i * kU;
    const int nv = min(kU, s1 - sl);
    const bool full = sl + kU <= slim;
    const int eb = sl * SLAB + lane * VEC;
    if constexpr (RT) load_chunk<In>(trow, eb, nv, V, full, t);
    if constexpr (RD) load_chunk<In>(drow, eb, nv, V, full, d);
  };
  auto fold = [&](const uint4 (&t)[kU], uint4 (&d)[kU], int i, auto first) {
    const int sl = s0 + i * kU;
    const int nv = min(kU, s1 - sl);
    stats_chunk<In, F, RT, RD, GREEDY, decltype(first)::value>(pl, V, drow, t, d, sl * SLAB,
                                                               sl * SLAB + lane * VEC, nv, c,
                                                               st, L, xd, yd);
  };
  load(ta, da, 0);
  if (nch > 1) load(tb, db, 1);
  fold(ta, da, 0, std::true_type{});
  for (int i = 1; i < nch; i += 2) {
    if (i + 1 < nch) load(ta, da, i + 1);
    fold(tb, db, i, std::false_type{});
    if (i + 1 >= nch) break;
    if (i + 2 < nch) load(tb, db, i + 2);
    fold(ta, da, i + 1, std::false_type{});
  }
}


// Segment `seg` of row slot `slot` (sequence b, position j) cut into
// `nparts`: slabs [seg * nslab / nparts, (seg + 1) * nslab / nparts) of the target and
// draft rows the plan reads.  Writes the segment's partial statistics
// (reference or maximum, fp64 sum, argmax) for each tensor read, the
// drafted token's logits when the segment holds it, and the draft's fork
// candidates (positions and vector maxima, compacted, with the list of any
// in-wave reduction), read by the next launch.  One wave; L is the wave's
// own LDS slots.
template <typename In, int F>
__device__ __forceinline__ void stream_segment(const Params& P, int64_t slot, int b, int j,
                                               int seg, int nparts, CandLds<F>* L) {
  const float tau = uniform(slot_tau(P, slot, b));
  const RowPlan pl = plan_row(P, b, j, tau);
  const float c = pl.greedy ? 0.0f : scale_of(tau);
  const int lane = lane_id();
  const Ws& W = P.ws;
  const int s0 = (int)((int64_t)seg * P.nslab / nparts);
  const int s1 = (int)((int64_t)(seg + 1) * P.nslab / nparts);
  const In* trow = pl.readT ? trow_ptr<In>(P, b, j) : nullptr;
  const In* drow = pl.readD ? drow_ptr<In>(P, b, j) : nullptr;

  WaveState st;
  warm_init(st.tw); warm_init(st.dw);
  greedy_init(st.tg); greedy_init(st.dg);
  st.nc = 0;
  st.kv = neg_inf();
  st.eth = 0.0f;
  if constexpr (F > 0) {
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < F; ++r) { L->wv[r] = neg_inf(); L->wi[r] = kEmptyId; }
    }
  }
  float* xd = W.xd + slot;
  float* yd = W.yd + slot;
  if (s1 > s0) {
    const int V = P.V;
    if (pl.readT && pl.readD) {
      if (pl.greedy) stats_segment<In, F, true, true, true>(pl, V, trow, drow, s0, s1, c, st, L, xd, yd);
      else stats_segment<In, F, true, true, false>(pl, V, trow, drow, s0, s1, c, st, L, xd, yd);
    } else if (pl.readT) {
      if (pl.greedy) stats_segment<In, F, true, false, true>(pl, V, trow, drow, s0, s1, c, st, L, xd, yd);
      else stats_segment<In, F, true, false, false>(pl, V, trow, drow, s0, s1, c, st, L, xd, yd);
    } else if (pl.readD) {
      if (pl.greedy) stats_segment<In, F, false, true, true>(pl, V, trow, drow, s0, s1, c, st, L, xd, yd);
      else stats_segment<In, F, false, true, false>(pl, V, trow, drow, s0, s1, c, st, L, xd, yd);
    }
  }
  // the output pointers are read from the kernel arguments again, past an
  // empty asm statement, so that they are not held in scalar registers
  // while the segment streams (P is the kernel's only argument, at the
  // start of its argument segment)
  typedef __attribute__((address_space(4))) const Params KParams;
  KParams* kp = (KParams*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(kp));
  Ws WE;
  WE.cpos = kp->ws.cpos; WE.cvm = kp->ws.cvm; WE.cn = kp->ws.cn;
  WE.tm = kp->ws.tm; WE.ts = kp->ws.ts; WE.targ = kp->ws.targ;
  WE.dm = kp->ws.dm; WE.ds = kp->ws.ds; WE.darg = kp->ws.darg;
  WE.dtv = kp->ws.dtv; WE.dti = kp->ws.dti;
  const int64_t part = slot * kMaxSeg + seg;
  if constexpr (F > 0) {
    if (pl.topf && pl.readD) {
      // pass the candidates on, compacted; rank them here only if they do
      // not fit
      int incl = wave_inclusive_scan_i(st.nc);
      int total = readlane_i(incl, kLanes - 1);
      if (total > kDumpCap) {
        cand_reduce<In, F, 8>(L, drow, P.V, pl.mask_id, st.nc, st.kv);
        incl = 0;
        total = 0;
      }
      int* dst = WE.cpos + part * kDumpCap + (incl - st.nc);
      float* dvm = WE.cvm + part * kDumpCap + (incl - st.nc);
      for (int i = 0; i < st.nc; ++i) {
        dst[i] = L->pos[i][lane];
        dvm[i] = L->vm[i][lane];
      }
      if (lane == 0) WE.cn[part] = total;
    }
  }

  if (pl.readT) {
    const WaveStats ws = pl.greedy ? wave_finish_greedy(st.tg) : wave_finish_warm(st.tw, c);
    if (lane == 0) { WE.tm[part] = ws.m; WE.ts[part] = ws.s; WE.targ[part] = ws.arg; }
  }
  if (pl.readD) {
    const WaveStats ws = pl.greedy ? wave_finish_greedy(st.dg) : wave_finish_warm(st.dw, c);
    if (lane == 0) { WE.dm[part] = ws.m; WE.ds[part] = ws.s; WE.darg[part] = ws.arg; }
    if constexpr (F > 0) {
      if (pl.topf && lane < F) {
        WE.dtv[part * F + lane] = L->wv[lane];
        WE.dti[part * F + lane] = L->wi[lane];
      }
    }
  }
}

// ================================================================ merging

struct Merged {
  float m; double s; int arg;
};

// Row reference / sum / argmax from the segment partials of one slot; every
// lane gets the result.  (k_write; k_decide merges from registers.)
__device__ __forceinline__ Merged merge_partials(const float* pm, const double* ps,
                                                 const int* parg, int64_t base, int np,
                                                 bool greedy, double cd) {
  const int lane = lane_id();
  float mi = neg_inf();
  double si = 0.0;
  int ai = kEmptyId;
  if (lane < np) { mi = pm[base + lane]; si = ps[base + lane]; ai = parg[base + lane]; }
  const float M = wave_max(mi);
  double s = 0.0;
  int arg = kEmptyId;
  if (greedy) {
    if (lane < np && mi == M) arg = ai;
  } else if (finitef(M) && mi > neg_inf()) {
    s = si * merge_scale(mi, M, (float)cd);
  }
  Merged r;
  r.m = M;
  r.s = wave_sum(s);
  r.arg = wave_min(arg);
  return r;
}

// The same from values already in the lanes (lane i holds partial i, empty
// lanes hold -inf).
__device__ __forceinline__ Merged merge_lanes(float mi, double si, int ai, bool greedy, double cd) {
  const float M = wave_max(mi);
  double s = 0.0;
  int arg = kEmptyId;
  if (greedy) {
    if (mi == M) arg = ai;
  } else if (finitef(M) && mi > neg_inf()) {
    s = si * merge_scale(mi, M, (float)cd);
  }
  Merged r;
  r.m = M;
  r.s = wave_sum(s);
  r.arg = wave_min(arg);
  return r;
}

// ================================================================ residual

// Per-element residual weight r = max(0, p - q) and target probability p
// from the merged row statistics (fp32 terms; references split exactly as
// in the statistics pass).
struct ResidCoef {
  float c, thi, tscale, dhi, dscale;
  bool has_q;
};

__device__ __forceinline__ ResidCoef resid_coef(float tm, double ts, float dm, double ds,
                                                float c, bool has_q) {
  ResidCoef k;
  k.c = c;
  k.thi = tm * c;
  const float tlo = fmaf(tm, c, -k.thi);
  k.tscale = (float)(exp2(-(double)tlo) / ts);
  k.has_q = has_q;
  k.dhi = 0.0f;
  k.dscale = 0.0f;
  if (has_q) {
    k.dhi = dm * c;
    const float dlo = fmaf(dm, c, -k.dhi);
    k.dscale = (float)(exp2(-(double)dlo) / ds);
  }
  return k;
}

// p and q are each rounded to fp32 before the difference is taken (no
// contraction of a product into the subtraction), so that equal target and
// draft rows give a residual of exactly zero.
__device__ __forceinline__ void resid_elem(const ResidCoef& k, float x, float y, float& p,
                                           float& r) {
#pragma clang fp contract(off)
  p = __builtin_amdgcn_exp2f(fmaf(x, k.c, -k.thi)) * k.tscale;
  if (k.has_q) {
    const float q = __builtin_amdgcn_exp2f(fmaf(y, k.c, -k.dhi)) * k.dscale;
    r = fmaxf(p - q, 0.0f);
  } else {
    r = p;
  }
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

// The weights of a lane's chunk summed: per vector the fp32 sum of r (which
// is p where there is no q), the vectors added in fp64.
template <typename In>
__device__ __forceinline__ double chunk_rsum(const ResidCoef& kc, const uint4 (&t)[kU],
                                             const uint4 (&d)[kU]) {
  constexpr int VEC = Elem<In>::VEC;
  double acc = 0.0;
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    float r[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float p;
      resid_elem(kc, elem<In>(t[u], e), kc.has_q ? elem<In>(d[u], e) : 0.0f, p, r[e]);
    }
    acc += (double)vec_sum<VEC>(r);
  }
  return acc;
}

constexpr int kTotRegs = 4;  // chunk totals the drawing wave keeps in registers (x 64)

// Overwrites the per-sequence outputs of an error sequence.
__device__ __forceinline__ void write_seq_error(const Params& P, int b) {
  const int lane = lane_id();
  const float nan = __uint_as_float(0x7fc00000u);
  const int K1 = P.k + 1;
  if (P.fork_tok) {
    for (int t = lane; t < K1 * P.f; t += kLanes) {
      st_dev(P.fork_tok + (int64_t)b * K1 * P.f + t, -1);
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
    if (P.accept_len) st_dev(P.accept_len + b, -1);
    if (P.out_token) st_dev(P.out_token + b, -1);
  }
}


// The draw by one wave: the chunk from the per-chunk totals (device-scope
// loads), then the vector (slab by slab, lanes inside), then the element;
// each time the first whose running total passes u*Z among positive
// weights, or the last positive one if rounding leaves none.
template <typename In>
__device__ __forceinline__ int resid_draw(const Params& P, const double* tot,
                                          const double (&tc)[kTotRegs], const In* trow,
                                          const In* drow, const ResidCoef& kc, double Z,
                                          double u) {
  constexpr int VEC = Elem<In>::VEC;
  constexpr int64_t SLAB = slab_elems<In>();
  const int lane = lane_id();
  const int cpr = P.cpr;
  const double target = u * Z;

  // 1. chunk
  int cstar = -1, clast = -1;
  double before = 0.0, before_last = 0.0, carry = 0.0;
  for (int g = 0; g < cpr; g += kLanes) {
    const int ch = g + lane;
    double w = 0.0;
    if (cpr <= kTotRegs * kLanes) {
#pragma unroll
      for (int q = 0; q < kTotRegs; ++q)
        if (q * kLanes == g) w = tc[q];
    } else if (ch < cpr) {
      w = ld_dev(tot + ch);
    }
    const double incl = carry + wave_inclusive_scan(w);
    double excl = __shfl_up(incl, 1);
    if (lane == 0) excl = carry;
    const unsigned long long hit = __ballot(ch < cpr && w > 0.0 && incl > target);
    if (cstar < 0 && hit) {
      const int l = __ffsll((long long)hit) - 1;
      cstar = g + l;
      before = readlane_d(excl, l);
    }
    const unsigned long long posm = __ballot(ch < cpr && w > 0.0);
    if (posm) {
      const int l = 63 - __clzll((long long)posm);
      clast = g + l;
      before_last = readlane_d(excl, l);
    }
    carry = readlane_d(incl, kLanes - 1);
  }
  if (cstar < 0) { cstar = clast; before = before_last; }
  if (cstar < 0) { cstar = 0; before = 0.0; }

  // 2. re-read that chunk; vector sums scanned slab by slab
  const int64_t sl = (int64_t)cstar * kU;
  const int nv = (int)min<int64_t>(kU, (int64_t)P.nslab - sl);
  const int eb = (int)(sl * SLAB) + lane * VEC;
  uint4 t[kU], d[kU];
  load_chunk<In>(trow, eb, nv, P.V, false, t);
  if (kc.has_q) {
    load_chunk<In>(drow, eb, nv, P.V, false, d);
  } else {
#pragma unroll
    for (int u = 0; u < kU; ++u) d[u] = make_uint4(0, 0, 0, 0);
  }
  float w[kU][VEC];
  float vsum[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    float r[VEC], p[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e)
      resid_elem(kc, elem<In>(t[u], e), kc.has_q ? elem<In>(d[u], e) : 0.0f, p[e], r[e]);
#pragma unroll
    for (int e = 0; e < VEC; ++e) w[u][e] = r[e];
    vsum[u] = vec_sum<VEC>(r);
  }
  int ustar = -1, lstar = 0, ulast = -1, llast = 0;
  double my_ex[kU];  // this lane's running total before its vector, per slab
  carry = before;
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const double incl = carry + wave_inclusive_scan((double)vsum[u]);
    double excl = __shfl_up(incl, 1);
    if (lane == 0) excl = carry;
    my_ex[u] = excl;
    const unsigned long long hit = __ballot(vsum[u] > 0.0f && incl > target);
    if (ustar < 0 && hit) {
      ustar = u;
      lstar = __ffsll((long long)hit) - 1;
    }
    const unsigned long long posm = __ballot(vsum[u] > 0.0f);
    if (posm) {
      ulast = u;
      llast = 63 - __clzll((long long)posm);
    }
    carry = readlane_d(incl, kLanes - 1);
  }
  if (ustar < 0) { ustar = ulast; lstar = llast; }
  if (ustar < 0) { ustar = 0; lstar = 0; }

  // 3. the element inside lane lstar's vector ustar
  int tokv = -1;
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    if (u == ustar) {
      int tk = -1, vlast = -1;
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        acc += w[u][e];
        if (w[u][e] > 0.0f) {
          const int id = (int)(eb + (int64_t)u * SLAB + e);
          vlast = id;
          if (tk < 0 && my_ex[u] + (double)acc > target) tk = id;
        }
      }
      tokv = tk < 0 ? vlast : tk;
    }
  }
  return readlane_i(tokv, lstar);
}


}  // namespace sv
