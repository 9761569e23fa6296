"""CPU oracle for the speculative-decoding verify-and-speculate step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP path.

It is a plain, slow, float64 restatement of what the step computes, one
sequence at a time, with the decision code (acceptance test, first rejection,
residual, inverse CDF) written over generic numbers so that it also runs on
``fractions.Fraction`` for exact enumeration.

Sources (cited by page title and section throughout):

* [SpecSampling] speculative-sampling project page (sourcepulse.org,
  project 1842340), sections "How It Works" and "Highlighted Details": a
  small model drafts tokens, the target checks them in parallel, keeps the
  correct ones and re-generates from the first divergence; both the Google
  and the DeepMind variants of speculative sampling are implemented; draft
  and target share one vocabulary ("Quick Start & Requirements").
* [SSD-editorial] "SSD: drafting and verification on separate GPUs, in
  parallel" (hysenlabs.com), section "What changes in SSD": the target
  verifies all drafted tokens in one forward pass, and the method is exact:
  the output distribution is the target model's.
* [SSD-summary] tanishqkumar/ssd repository summary (thehardwarestore.ai),
  the highlighted sampler file (greedy or stochastic sampling chosen by the
  temperature) and the async-SD utilities file (forked recovery tokens:
  top-k selection over logits with masking).
* [SSD-README-zh] SSD README translation (m.111cn.net), section 基准测试:
  benchmark commands with k=6 (synchronous) and k=7, f=3 (SSD), where f is
  the number of alternatives speculated per position.

The pages name the speculative-sampling rule but do not write it out.  This
oracle takes its textbook form, the plainest reading consistent with the
exactness requirement: accept drafted token d at position j iff
``u < min(1, p_j(d)/q_j(d))``; at the first rejection n sample from the
normalised residual ``max(0, p_n - q_n)``; if nothing is rejected sample the
bonus token from ``p_k``.  Readings of the points the pages leave open:

1. ``u < a`` (strict), so a token with p = 0 is never accepted.
2. q(d) = 0: a = 1 if p(d) > 0 else 0.
3. ``u_accept[b, j]`` drives the test at position j; ``u_recover[b, n]``
   drives the draw at the outcome position n (n = k: the bonus draw).
4. Inverse CDF in token-id order: the first t with C_t > u*Z, C the running
   sum of the weights and Z their total; if rounding leaves none, the last
   token of positive weight.
5. A residual of total zero (p = q exactly) falls back to p_n.
6. Temperature 0 is greedy: accept iff d_j is the target's argmax; the token
   is the target's argmax at n.  Ties go to the lowest token id.  Its
   probability outputs are one-hot at that argmax.
7. Forks at position j: the f highest draft logits with the drafted token
   d_j excluded (nothing excluded at the bonus position j = k), ties to the
   lower id; their probabilities come from the softmax of the masked draft
   logits at the sequence temperature (one-hot (1, 0, ...) at temperature 0).
8. A draw is flagged when its uniform lies within 1e-6 of a decision
   boundary (the acceptance probability, or a CDF breakpoint of the chosen
   token); a sequence is flagged when any acceptance test up to and including
   the first rejection, or its final draw, is flagged.  The weights of the
   verify draw are probabilities, or differences of two, that the GPU path
   holds in fp32, so each cumulative sum is known there only to within
   2^-23 of the unit probability mass; a verify draw whose target lies that
   close to a breakpoint is flagged as well (the band is 1e-6 Z + 2^-23 in
   weight units).  This also flags a residual whose whole mass is below
   fp32's resolution, which the GPU path sees as zero.
9. Errors: a temperature that is NaN, negative or infinite, a drafted id
   outside [0, V), or a logits row that is read and whose maximum is not
   finite (+inf, or every entry -inf) make the whole sequence an error.
   NaN logits are outside the contract (this oracle raises).
10. Speculation-cache lookup: the outcome (n, token) hits when the token is
   one of the f forks at position n, and the hit is its index there; an
   error outcome never hits.
"""

from __future__ import annotations

import bisect
import dataclasses
import itertools
import math
from fractions import Fraction
from typing import List, Optional, Sequence

import numpy as np

FLAG_BAND = 1e-6
# Absolute band of the verify draw, in units of the unit probability mass:
# the resolution of a cumulative sum of fp32 probabilities (reading 8).
DRAW_ABS_BAND = 2.0 ** -23

F32 = "f32"
BF16 = "bf16"


class RowError(Exception):
    """A logits row whose maximum is not finite."""


# --------------------------------------------------------------------------
# Input decoding (exact)
# --------------------------------------------------------------------------

def widen(row, dtype: str) -> np.ndarray:
    """Logits row as float64.  bf16 rows arrive as their 16-bit patterns; a
    bfloat16 value is the float32 whose upper half is those 16 bits, so the
    widening is exact.  float32 to float64 is exact as well."""
    a = np.asarray(row)
    if dtype == BF16:
        if a.dtype != np.uint16:
            raise TypeError("bf16 logits must be given as uint16 bit patterns")
        bits32 = a.astype(np.uint32) << np.uint32(16)
        return bits32.view(np.float32).astype(np.float64)
    if dtype == F32:
        return a.astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


def _check_row(x: np.ndarray) -> None:
    if np.isnan(x).any():
        raise ValueError("NaN logits are outside the contract")
    m = x.max()
    if not np.isfinite(m):
        raise RowError("row maximum is not finite")


# --------------------------------------------------------------------------
# O1: temperature softmax, greedy at temperature 0
#     ([SSD-summary] sampler: greedy or stochastic by temperature)
# --------------------------------------------------------------------------

def argmax_first(x) -> int:
    """Lowest index holding the maximum value."""
    x = np.asarray(x)
    m = x.max()
    return int(np.flatnonzero(x == m)[0])


def softmax_temp(x: np.ndarray, tau: float) -> np.ndarray:
    """softmax(x / tau) in float64; one-hot at the first maximum when tau = 0.

    exp((x_t - m)/tau) with m = max x, divided by the correctly rounded sum
    of those terms.
    """
    x = np.asarray(x, dtype=np.float64)
    _check_row(x)
    if tau == 0.0:
        p = np.zeros_like(x)
        p[argmax_first(x)] = 1.0
        return p
    m = x.max()
    e = np.exp((x - m) / tau)
    s = math.fsum(e.tolist())
    return e / s


# --------------------------------------------------------------------------
# O2-O5: acceptance, first rejection, residual, inverse CDF
#        ([SpecSampling] "How It Works"; [SSD-editorial] "What changes in SSD")
#        Written over generic numbers (float or Fraction).
# --------------------------------------------------------------------------

def _total(xs):
    xs = list(xs)
    if xs and isinstance(xs[0], Fraction):
        return sum(xs, Fraction(0))
    return math.fsum(xs)


def acceptance_probability(p, q):
    """a = min(1, p/q); a = 1 if q = 0 < p; a = 0 if p = q = 0."""
    if q == 0:
        return 1 if p > 0 else 0
    r = p / q
    return r if r < 1 else 1


def first_rejection(accepted: Sequence[bool]) -> int:
    """Index of the first rejected position, or len(accepted) if none."""
    for j, ok in enumerate(accepted):
        if not ok:
            return j
    return len(accepted)


def residual_weights(P: Sequence, Q: Sequence) -> list:
    """max(0, p_t - q_t) per token, or p itself if those sum to zero."""
    w = [p - q if p > q else 0 * p for p, q in zip(P, Q)]
    if _total(w) == 0:
        return list(P)
    return w


def inverse_cdf(w: Sequence, u, abs_band=0.0):
    """Sample from unnormalised weights w with the uniform u.

    Returns (token, flagged).  C_t is the running sum of w in token-id order
    and Z = C_{V-1}; the token is the first t with C_t > u*Z (the running
    sums never decrease, so that is bisect_right); if rounding leaves none,
    the last token of positive weight.  The draw is flagged when u lies
    within FLAG_BAND + abs_band / Z of C_{tok-1}/Z or C_tok/Z (abs_band in
    the units of w).
    """
    C = list(itertools.accumulate(w))
    Z = C[-1]
    if not Z > 0:
        raise ValueError("weights sum to zero")
    target = u * Z
    tok = bisect.bisect_right(C, target)
    if tok >= len(C):
        tok = max(t for t, x in enumerate(w) if x > 0)
    lo = C[tok - 1] if tok > 0 else 0 * Z
    hi = C[tok]
    flagged = min(abs(u - lo / Z), abs(u - hi / Z)) < FLAG_BAND + abs_band / Z
    return tok, bool(flagged)


@dataclasses.dataclass
class ProbVerdict:
    accept_len: int
    token: int
    accept_flags: List[bool]
    draw_flag: bool

    @property
    def flagged(self) -> bool:
        n = self.accept_len
        return any(self.accept_flags[: n + 1]) or self.draw_flag


def verify_from_probs(P_rows, Q_rows, drafts, u_accept, u_recover) -> ProbVerdict:
    """Stochastic verification of one sequence given its distributions.

    P_rows[j] (j = 0..k) and Q_rows[j] (j = 0..k-1) are the target and draft
    distributions at each position (any number type); drafts[j] the drafted
    tokens.  Position j's drafted token is accepted iff
    u_accept[j] < min(1, p_j(d_j)/q_j(d_j)); n is the first rejection; the
    emitted token at n is drawn with u_recover[n] from the residual
    max(0, p_n - q_n) (n < k) or from p_k (n = k, the bonus token).
    """
    k = len(drafts)
    accepted, flags = [], []
    for j in range(k):
        d = drafts[j]
        a = acceptance_probability(P_rows[j][d], Q_rows[j][d])
        accepted.append(u_accept[j] < a)
        flags.append(bool(abs(u_accept[j] - a) < FLAG_BAND))
    n = first_rejection(accepted)
    w = residual_weights(P_rows[n], Q_rows[n]) if n < k else list(P_rows[k])
    tok, dflag = inverse_cdf(w, u_recover[n], DRAW_ABS_BAND)
    return ProbVerdict(accept_len=n, token=tok, accept_flags=flags,
                       draw_flag=dflag)


def verify_greedy(T_rows, drafts) -> ProbVerdict:
    """Temperature 0: accept while d_j equals the target's argmax; the
    emitted token is the target's argmax at the first mismatch (or at the
    bonus position).  Nothing is flagged."""
    k = len(drafts)
    accepted = [drafts[j] == argmax_first(T_rows[j]) for j in range(k)]
    n = first_rejection(accepted)
    return ProbVerdict(accept_len=n, token=argmax_first(T_rows[n]),
                       accept_flags=[False] * k, draw_flag=False)


# --------------------------------------------------------------------------
# O6: forked recovery tokens ([SSD-summary] async-SD utilities: top-k over
#     logits with masking; [SSD-README-zh] 基准测试: f alternatives)
# --------------------------------------------------------------------------

def forked_topf(y: np.ndarray, tau: float, f: int, exclude: Optional[int]):
    """Top-f draft tokens with ``exclude`` masked out, and their
    probabilities under the softmax of the masked logits at tau.

    Order: descending logit, ties to the lower token id (a stable sort of
    the negated logits keeps equal keys in ascending id order).
    """
    y = np.asarray(y, dtype=np.float64)
    V = y.shape[0]
    keep = np.ones(V, dtype=bool)
    if exclude is not None:
        keep[exclude] = False
    ids = np.flatnonzero(keep)
    vals = y[ids]
    order = np.argsort(-vals, kind="stable")
    top = ids[order[:f]]
    if tau == 0.0:
        probs = np.zeros(f)
        probs[0] = 1.0
        return top.astype(np.int64), probs
    m = vals.max()
    if not np.isfinite(m):  # every unmasked logit is -inf
        return top.astype(np.int64), np.zeros(f)
    s = math.fsum(np.exp((vals - m) / tau).tolist())
    probs = np.exp((y[top] - m) / tau) / s
    return top.astype(np.int64), probs


# --------------------------------------------------------------------------
# Residual distributions (normalised), one per position
# --------------------------------------------------------------------------

def residual_distribution(P: np.ndarray, Q: Optional[np.ndarray]) -> np.ndarray:
    """max(0, p - q) / sum (p if that sum is zero); p itself when Q is None
    (the bonus position)."""
    if Q is None:
        return np.asarray(P, dtype=np.float64).copy()
    w = np.array(residual_weights(P.tolist(), Q.tolist()), dtype=np.float64)
    return w / math.fsum(w.tolist())


# --------------------------------------------------------------------------
# One sequence, from logits
# --------------------------------------------------------------------------

@dataclasses.dataclass
class SequenceResult:
    accept_len: int
    token: int
    p_draft: np.ndarray  # [k]
    q_draft: np.ndarray  # [k]
    fork_tokens: np.ndarray  # [k+1, f]
    fork_probs: np.ndarray  # [k+1, f]
    residual: Optional[np.ndarray]  # [k+1, V]
    accept_flags: List[bool]
    draw_flag: bool
    flagged: bool
    error: bool


def _tau_ok(tau: float) -> bool:
    return math.isfinite(tau) and tau >= 0.0


def _error_result(k, f, V, want_residual) -> SequenceResult:
    return SequenceResult(
        accept_len=-1, token=-1, p_draft=np.full(k, np.nan),
        q_draft=np.full(k, np.nan), fork_tokens=np.full((k + 1, f), -1),
        fork_probs=np.full((k + 1, f), np.nan),
        residual=np.full((k + 1, V), np.nan) if want_residual else None,
        accept_flags=[False] * k, draw_flag=False, flagged=False, error=True)


def verify_sequence(T, D, dtype, drafts, tau, u_accept, u_recover, f=0,
                    want_q=True, want_residual=False) -> SequenceResult:
    """Verify one sequence from its logits.

    T: [k+1, V] target logits; D: [k+1, V] draft logits (row k is read only
    for forks); drafts: [k]; tau: the sequence temperature; u_accept: [k];
    u_recover: [k+1].  f = 0 asks for no forks.  want_q asks for the draft
    probabilities of the drafted tokens also at temperature 0 (at tau > 0 the
    draft rows are always read).
    """
    k = len(drafts)
    V = np.asarray(T).shape[-1]
    tau = float(tau)
    drafts = [int(x) for x in drafts]
    if not _tau_ok(tau) or any(not (0 <= d < V) for d in drafts):
        return _error_result(k, f, V, want_residual)
    read_d_rows = k if (tau > 0 or want_q or f > 0 or want_residual) else 0
    try:
        Tw = [widen(T[j], dtype) for j in range(k + 1)]
        P = [softmax_temp(Tw[j], tau) for j in range(k + 1)]
        Dw = [widen(D[j], dtype) for j in range(read_d_rows)]
        if f > 0:
            Dw.append(widen(D[k], dtype))
        Q = [softmax_temp(Dw[j], tau) for j in range(read_d_rows)]
        if f > 0:
            _check_row(Dw[k])
    except RowError:
        return _error_result(k, f, V, want_residual)

    if tau == 0.0:
        verdict = verify_greedy(Tw, drafts)
    else:
        verdict = verify_from_probs(
            [p.tolist() for p in P], [q.tolist() for q in Q], drafts,
            [float(u) for u in u_accept], [float(u) for u in u_recover])

    p_d = np.array([P[j][drafts[j]] for j in range(k)])
    q_d = (np.array([Q[j][drafts[j]] for j in range(k)]) if read_d_rows
           else np.full(k, np.nan))

    ft = np.zeros((k + 1, f), dtype=np.int64)
    fp = np.zeros((k + 1, f))
    for j in range(k + 1 if f > 0 else 0):
        ft[j], fp[j] = forked_topf(Dw[j], tau, f, drafts[j] if j < k else None)

    res = None
    if want_residual:
        res = np.stack([residual_distribution(P[j], Q[j]) for j in range(k)]
                       + [residual_distribution(P[k], None)])

    return SequenceResult(accept_len=verdict.accept_len, token=verdict.token,
                          p_draft=p_d, q_draft=q_d, fork_tokens=ft,
                          fork_probs=fp, residual=res,
                          accept_flags=verdict.accept_flags,
                          draw_flag=verdict.draw_flag,
                          flagged=verdict.flagged, error=False)


def sample_at_position(T, D, dtype, drafts, tau, position, u_recover,
                       want_residual=False):
    """The recovery (position < k) or bonus (position = k) draw of one
    sequence at a given position, and optionally every position's residual
    distribution.  Returns (token, flagged, residual or None, error)."""
    k = len(drafts)
    V = np.asarray(T).shape[-1]
    tau = float(tau)
    drafts = [int(x) for x in drafts]
    n = int(position)
    if (not _tau_ok(tau) or any(not (0 <= d < V) for d in drafts)
            or not (0 <= n <= k)):
        return -1, False, (np.full((k + 1, V), np.nan) if want_residual else None), True
    rows = range(k + 1) if want_residual else [n]
    try:
        P = {j: softmax_temp(widen(T[j], dtype), tau) for j in rows}
        Q = {j: softmax_temp(widen(D[j], dtype), tau) for j in rows if j < k}
    except RowError:
        return -1, False, (np.full((k + 1, V), np.nan) if want_residual else None), True
    if tau == 0.0:
        tok, flag = argmax_first(widen(T[n], dtype)), False
    else:
        w = residual_weights(P[n].tolist(), Q[n].tolist()) if n < k else P[n].tolist()
        tok, flag = inverse_cdf(w, float(u_recover[n]), DRAW_ABS_BAND)
    res = None
    if want_residual:
        res = np.stack([residual_distribution(P[j], Q[j]) for j in range(k)]
                       + [residual_distribution(P[k], None)])
    return tok, flag, res, False


# --------------------------------------------------------------------------
# Batch drivers (loops over sequences)
# --------------------------------------------------------------------------

@dataclasses.dataclass
class BatchResult:
    seqs: np.ndarray
    accept_len: np.ndarray
    token: np.ndarray
    p_draft: np.ndarray
    q_draft: np.ndarray
    fork_tokens: np.ndarray
    fork_probs: np.ndarray
    residual: Optional[np.ndarray]
    flagged: np.ndarray  # bool [B]
    n_flagged_draws: int
    error: np.ndarray  # bool [B]


def verify_batch(target, draft, dtype, draft_tokens, temperature, u_accept,
                 u_recover, f=0, want_q=True, want_residual=False,
                 seqs=None) -> BatchResult:
    """verify_sequence over the sequences ``seqs`` (default: all)."""
    B = np.asarray(target).shape[0]
    seqs = np.arange(B) if seqs is None else np.asarray(seqs)
    out = [verify_sequence(target[b], draft[b], dtype, draft_tokens[b],
                           temperature[b], u_accept[b], u_recover[b], f=f,
                           want_q=want_q, want_residual=want_residual)
           for b in seqs]
    return BatchResult(
        seqs=seqs,
        accept_len=np.array([r.accept_len for r in out], dtype=np.int64),
        token=np.array([r.token for r in out], dtype=np.int64),
        p_draft=np.stack([r.p_draft for r in out]),
        q_draft=np.stack([r.q_draft for r in out]),
        fork_tokens=np.stack([r.fork_tokens for r in out]),
        fork_probs=np.stack([r.fork_probs for r in out]),
        residual=(np.stack([r.residual for r in out]) if want_residual else None),
        flagged=np.array([r.flagged for r in out], dtype=bool),
        n_flagged_draws=int(sum(sum(r.accept_flags[: max(r.accept_len, 0) + 1])
                                + int(r.draw_flag) for r in out)),
        error=np.array([r.error for r in out], dtype=bool))


def softmax_rows(logits, dtype, temperatures) -> np.ndarray:
    """softmax_temp over each row of a [rows, V] array, with one temperature
    per row.  Rows whose maximum is not finite, or whose temperature is not a
    finite non-negative number, come back as NaN."""
    logits = np.asarray(logits)
    out = np.empty(logits.shape, dtype=np.float64)
    for r in range(logits.shape[0]):
        tau = float(temperatures[r])
        try:
            if not _tau_ok(tau):
                raise RowError
            out[r] = softmax_temp(widen(logits[r], dtype), tau)
        except RowError:
            out[r] = np.nan
    return out


def forked_topf_batch(draft, dtype, draft_tokens, temperature, f):
    """forked_topf at every position of every sequence: ([B,k+1,f] tokens,
    [B,k+1,f] probabilities).  Error sequences get -1 / NaN."""
    draft = np.asarray(draft)
    B, K1, V = draft.shape
    k = K1 - 1
    toks = np.full((B, K1, f), -1, dtype=np.int64)
    probs = np.full((B, K1, f), np.nan)
    for b in range(B):
        tau = float(temperature[b])
        ds = [int(x) for x in draft_tokens[b]]
        if not _tau_ok(tau) or any(not (0 <= d < V) for d in ds):
            continue
        try:
            rows = [widen(draft[b, j], dtype) for j in range(K1)]
            for r in rows:
                _check_row(r)
        except RowError:
            continue
        for j in range(K1):
            toks[b, j], probs[b, j] = forked_topf(rows[j], tau, f,
                                                  ds[j] if j < k else None)
    return toks, probs

def cache_hit(fork_tokens_n, token) -> int:
    """Speculation-cache lookup of one verification outcome.

    [SSD-editorial] "What changes in SSD": the drafter speculates ahead of
    time for the likely verification outcomes, and when one of its guesses
    is right the speculation is returned at once.  [SSD-summary], the
    async-SD utilities file: the forked recovery tokens (top-k with the
    drafted token masked) are what handles the cache hits and misses.  The
    outcome of a step is (n, token); the drafter speculated, at position n,
    for the f forked tokens ``fork_tokens_n``.  The outcome hits when
    ``token`` is one of them: the result is its index r (the forks are
    distinct, so there is at most one), else -1.
    """
    for r, t in enumerate(fork_tokens_n):
        if int(t) == int(token):
            return r
    return -1


def cache_hits_batch(fork_tokens, accept_len, token) -> np.ndarray:
    """cache_hit for every sequence of a batch: fork_tokens [B, k+1, f],
    accept_len [B] (the outcome position n), token [B].  A sequence whose
    outcome is an error (n or token negative) gets -1."""
    fork_tokens = np.asarray(fork_tokens)
    B, K1, _ = fork_tokens.shape
    out = np.full(B, -1, dtype=np.int64)
    for b in range(B):
        n, t = int(accept_len[b]), int(token[b])
        if 0 <= n < K1 and t >= 0:
            out[b] = cache_hit(fork_tokens[b, n], t)
    return out


def sample_temp(x, tau: float, u):
    """The drafter's own draw from one logits row: greedy at temperature 0,
    stochastic above it.

    [SSD-summary], the highlighted sampler file: sampling is greedy or
    stochastic according to the temperature.  At tau = 0 the token is the
    lowest id holding the maximum; above it, the inverse-CDF draw (reading 4)
    from softmax(x / tau) with the uniform u.  Returns (token, flagged); a
    row whose maximum is not finite, or an invalid temperature, raises
    RowError.
    """
    x = np.asarray(x, dtype=np.float64)
    if not _tau_ok(float(tau)):
        raise RowError("temperature")
    _check_row(x)
    if tau == 0.0:
        return argmax_first(x), False
    return inverse_cdf(softmax_temp(x, tau).tolist(), float(u))


def sample_rows(logits, dtype, temperatures, uniforms):
    """sample_temp over the rows of a [rows, V] array (one temperature and
    one uniform per row): (tokens [rows], flagged [rows]); error rows get
    -1."""
    logits = np.asarray(logits)
    R = logits.shape[0]
    toks = np.full(R, -1, dtype=np.int64)
    flags = np.zeros(R, dtype=bool)
    for r in range(R):
        try:
            toks[r], flags[r] = sample_temp(widen(logits[r], dtype), float(temperatures[r]),
                                            float(uniforms[r]))
        except RowError:
            pass
    return toks, flags
