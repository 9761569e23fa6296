"""Pins of the oracle against library routines, closed forms, limits,
invariants and hand-worked cases (CPU only)."""

import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from workloads import Config, f32_to_bf16_bits, make_workload


# ---------------------------------------------------------------- decoding

def test_bf16_widening_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(4096) * 30).astype(np.float32)
    bits = f32_to_bf16_bits(x)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oracle.widen(bits, "bf16"), ref)
    # torch's own float32 -> bfloat16 rounding is round-to-nearest-even too
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, tb)


# ---------------------------------------------------------------- softmax

@pytest.mark.parametrize("tau", [0.3, 0.7, 1.0, 2.5])
def test_softmax_matches_scipy_and_torch(tau):
    rng = np.random.default_rng(1)
    x = rng.standard_normal(5000) * 3
    p = oracle.softmax_temp(x, tau)
    np.testing.assert_allclose(p, scipy.special.softmax(x / tau), rtol=1e-13, atol=0)
    pt = torch.softmax(torch.from_numpy(x) / tau, dim=0).numpy()
    np.testing.assert_allclose(p, pt, rtol=1e-12, atol=0)
    assert abs(math.fsum(p) - 1) < 1e-14


def test_softmax_shift_invariance_and_masking():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(1000)
    np.testing.assert_allclose(oracle.softmax_temp(x, 0.8),
                               oracle.softmax_temp(x + 17.25, 0.8), rtol=1e-12)
    y = x.copy()
    y[::3] = -np.inf
    p = oracle.softmax_temp(y, 0.8)
    assert np.all(p[::3] == 0)
    q = scipy.special.softmax(x[np.isfinite(y)] / 0.8)
    np.testing.assert_allclose(p[np.isfinite(y)], q, rtol=1e-13)


def test_softmax_greedy_and_row_errors():
    x = np.array([1.0, 3.0, 3.0, 2.0])
    np.testing.assert_array_equal(oracle.softmax_temp(x, 0.0), [0, 1, 0, 0])
    with pytest.raises(oracle.RowError):
        oracle.softmax_temp(np.array([-np.inf, -np.inf]), 1.0)
    with pytest.raises(oracle.RowError):
        oracle.softmax_temp(np.array([0.0, np.inf]), 1.0)


# ---------------------------------------------------------------- inverse CDF

def test_inverse_cdf_matches_searchsorted():
    """Token-id order and the 'first C_t > uZ' boundary, against numpy."""
    rng = np.random.default_rng(4)
    for _ in range(300):
        V = int(rng.integers(1, 60))
        w = rng.random(V)
        w[rng.random(V) < 0.4] = 0.0
        if w.sum() == 0:
            w[int(rng.integers(V))] = 0.5
        u = float(rng.integers(0, 2**24)) * 2.0**-24
        tok, _ = oracle.inverse_cdf(w.tolist(), u)
        c = np.cumsum(w)
        ref = int(np.searchsorted(c, u * c[-1], side="right"))
        if ref >= V:
            ref = int(np.flatnonzero(w > 0)[-1])
        assert tok == ref
        assert w[tok] > 0


def test_inverse_cdf_edges():
    w = [0.0, 0.25, 0.0, 0.75, 0.0]
    assert oracle.inverse_cdf(w, 0.0)[0] == 1
    assert oracle.inverse_cdf(w, 0.2499)[0] == 1
    assert oracle.inverse_cdf(w, 0.25)[0] == 3  # C_1/Z = 0.25 is not > 0.25
    assert oracle.inverse_cdf(w, 1 - 2**-24)[0] == 3
    # flags near a breakpoint
    assert oracle.inverse_cdf(w, 0.25 - 5e-7)[1]
    assert not oracle.inverse_cdf(w, 0.5)[1]


# ---------------------------------------------------------------- greedy

def test_greedy_is_prefix_match():
    """Temperature 0 reduces to greedy verification: the accepted length is
    the length of the common prefix of the drafts and the target argmaxes,
    and the emitted token is the target argmax there."""
    rng = np.random.default_rng(5)
    for _ in range(200):
        k, V = int(rng.integers(1, 6)), int(rng.integers(2, 7))
        T = rng.integers(0, 3, (k + 1, V)).astype(np.float64)  # many ties
        am = [min(t for t in range(V) if T[j, t] == T[j].max()) for j in range(k + 1)]
        drafts = [am[j] if rng.random() < 0.6 else int(rng.integers(V)) for j in range(k)]
        n = 0
        while n < k and drafts[n] == am[n]:
            n += 1
        v = oracle.verify_greedy(list(T), drafts)
        assert (v.accept_len, v.token) == (n, am[n])


def test_small_temperature_limit_matches_greedy():
    """As tau -> 0 the stochastic rule becomes the greedy one: with logits
    separated by >= 1 and tau = 0.01 every probability other than the argmax
    is below e^-100, far inside the flag band."""
    rng = np.random.default_rng(6)
    for _ in range(100):
        k, V = 3, 6
        T = np.stack([rng.permutation(V).astype(np.float64) for _ in range(k + 1)])
        D = np.stack([rng.permutation(V).astype(np.float64) for _ in range(k + 1)])
        am = T.argmax(1)
        drafts = np.array([am[j] if rng.random() < 0.7 else D[j].argmax() for j in range(k)])
        ua = rng.random(k) * 0.98 + 0.01
        ur = rng.random(k + 1) * 0.98 + 0.01
        g = oracle.verify_sequence(T, D, "f32", drafts, 0.0, ua, ur)
        s = oracle.verify_sequence(T, D, "f32", drafts, 0.01, ua, ur)
        assert (g.accept_len, g.token) == (s.accept_len, s.token)


# ---------------------------------------------------------------- forks

def test_forks_match_sorted_key():
    rng = np.random.default_rng(7)
    for _ in range(100):
        V = int(rng.integers(2, 40))
        y = rng.integers(-3, 4, V).astype(np.float64)
        f = int(rng.integers(1, V))
        ex = int(rng.integers(V)) if rng.random() < 0.8 else None
        toks, _ = oracle.forked_topf(y, 1.0, f, ex)
        ref = sorted((t for t in range(V) if t != ex), key=lambda t: (-y[t], t))[:f]
        assert list(toks) == ref


def test_fork_probs_are_masked_softmax():
    rng = np.random.default_rng(8)
    y = rng.standard_normal(300) * 2
    toks, probs = oracle.forked_topf(y, 0.7, 5, 17)
    z = y.copy()
    z[17] = -np.inf
    ref = scipy.special.softmax(z / 0.7)
    np.testing.assert_allclose(probs, ref[toks], rtol=1e-13)
    toks0, probs0 = oracle.forked_topf(y, 0.0, 3, None)
    np.testing.assert_array_equal(probs0, [1, 0, 0])


# ---------------------------------------------------------------- residual

def test_residual_distribution_properties():
    rng = np.random.default_rng(9)
    P = scipy.special.softmax(rng.standard_normal(500))
    Q = scipy.special.softmax(rng.standard_normal(500))
    r = oracle.residual_distribution(P, Q)
    assert abs(r.sum() - 1) < 1e-14
    assert np.all(r[P <= Q] == 0)
    pos = P > Q
    np.testing.assert_allclose(r[pos], (P - Q)[pos] / (P - Q)[pos].sum(), rtol=1e-12)
    np.testing.assert_array_equal(oracle.residual_distribution(P, P), P)


# ---------------------------------------------------------------- invariants

def _small_zipf(B, k, V, tau, seed, f=3):
    return make_workload(Config("t", B=B, k=k, V=V, f=f, dtype="bf16",
                                profile="zipf", seed=seed, tau=tau,
                                sigma_range=(0.3, 1.2)))


@pytest.mark.parametrize("tau", [0.0, 0.7, 1.3])
def test_invariants_on_synthetic_batches(tau):
    w = _small_zipf(12, 5, 3000, tau, 11)
    r = oracle.verify_batch(w.target, w.draft, "bf16", w.draft_tokens,
                            w.temperature, w.u_accept, w.u_recover, f=3)
    assert np.all((r.accept_len >= 0) & (r.accept_len <= w.k))
    for i in range(w.B):
        n = r.accept_len[i]
        if n < w.k:
            assert r.token[i] != w.draft_tokens[i, n]  # rejected draft never re-emitted
        for j in range(w.k + 1):
            ft = list(r.fork_tokens[i, j])
            assert len(set(ft)) == 3
            if j < w.k:
                assert w.draft_tokens[i, j] not in ft
            y = oracle.widen(w.draft[i, j], "bf16")[ft]
            assert np.all(np.diff(y) <= 0)
            assert np.all(np.diff(r.fork_probs[i, j]) <= 0 if tau > 0 else True)


def test_identical_drafter_accepts_everything():
    w = _small_zipf(6, 4, 2000, 0.9, 12)
    r = oracle.verify_batch(w.target, w.target, "bf16", w.draft_tokens,
                            w.temperature, w.u_accept, w.u_recover)
    assert np.all(r.accept_len == w.k)


def test_disjoint_support_rejects_first():
    V, k = 50, 3
    T = np.full((k + 1, V), -np.inf)
    D = np.full((k + 1, V), -np.inf)
    T[:, :25] = 0.0
    D[:, 25:] = 0.0
    r = oracle.verify_sequence(T, D, "f32", [30, 31, 32], 1.0, [0.0] * k, [0.5] * (k + 1))
    assert r.accept_len == 0 and r.token < 25
    assert r.p_draft[0] == 0 and r.q_draft[0] == pytest.approx(1 / 25)


def test_error_sequences():
    T = np.zeros((3, 8))
    D = np.zeros((3, 8))
    assert oracle.verify_sequence(T, D, "f32", [1, 9], 1.0, [0.1, 0.1], [0.1] * 3).error
    assert oracle.verify_sequence(T, D, "f32", [1, 2], -1.0, [0.1, 0.1], [0.1] * 3).error
    assert oracle.verify_sequence(T, D, "f32", [1, 2], float("nan"), [0.1, 0.1], [0.1] * 3).error
    T2 = T.copy()
    T2[2] = -np.inf
    assert oracle.verify_sequence(T2, D, "f32", [1, 2], 1.0, [0.1, 0.1], [0.1] * 3).error
    # row k of the drafter is read only for forks
    D2 = D.copy()
    D2[2, 3] = np.inf
    assert not oracle.verify_sequence(T, D2, "f32", [1, 2], 1.0, [0.1, 0.1], [0.1] * 3).error
    assert oracle.verify_sequence(T, D2, "f32", [1, 2], 1.0, [0.1, 0.1], [0.1] * 3, f=2).error


# ---------------------------------------------------------------- hand-worked

LN = np.log


def test_hand_worked_reject_then_residual():
    """p0 = (1/2, 1/4, 1/4), q0 = (1/4, 1/2, 1/4), drafted token 1:
    a = (1/4)/(1/2) = 1/2.  u = 0.75 >= 1/2 rejects at position 0; the
    residual max(0, p - q) = (1/4, 0, 0) puts all its mass on token 0."""
    T = np.array([[LN(.5), LN(.25), LN(.25)], [0.0, 0.0, 0.0]])
    D = np.array([[LN(.25), LN(.5), LN(.25)], [0.0, 0.0, 0.0]])
    r = oracle.verify_sequence(T, D, "f32", [1], 1.0, [0.75], [0.3, 0.9])
    assert (r.accept_len, r.token) == (0, 0)
    assert r.p_draft[0] == pytest.approx(0.25, rel=1e-6)
    assert r.q_draft[0] == pytest.approx(0.5, rel=1e-6)


def test_hand_worked_accept_then_bonus():
    """Same position 0 with u = 0.25 < 1/2: accepted; the bonus token is
    drawn from p1 = (0.1, 0.2, 0.7) with u = 0.35: C = (0.1, 0.3, 1.0), the
    first C_t > 0.35 is t = 2."""
    T = np.array([[LN(.5), LN(.25), LN(.25)], [LN(.1), LN(.2), LN(.7)]])
    D = np.array([[LN(.25), LN(.5), LN(.25)], [0.0, 0.0, 0.0]])
    r = oracle.verify_sequence(T.astype(np.float32), D.astype(np.float32), "f32",
                               [1], 1.0, [0.25], [0.99, 0.35])
    assert (r.accept_len, r.token) == (1, 2)


def test_hand_worked_recover_uses_uniform_of_rejected_position():
    """k = 2.  Position 0: p = q, accepted for any u.  Position 1:
    p1 = (1/4, 1/2, 1/4), q1 = (0, 1/4, 3/4), drafted token 2:
    a = (1/4)/(3/4) = 1/3, and u = 0.5 rejects.  The residual is
    (1/4, 1/4, 0) with Z = 1/2, so C/Z = (0.5, 1, 1): u_recover[1] = 0.7
    gives token 1, while the other entries (0.1) would give token 0."""
    T = np.array([[0, 0, 0], [LN(.25), LN(.5), LN(.25)], [0, 0, 0]], dtype=np.float64)
    D = np.array([[0, 0, 0], [-np.inf, LN(.25), LN(.75)], [0, 0, 0]], dtype=np.float64)
    r = oracle.verify_sequence(T, D, "f32", [0, 2], 1.0, [0.9, 0.5], [0.1, 0.7, 0.1])
    assert (r.accept_len, r.token) == (1, 1)


def test_hand_worked_greedy_ties():
    """tau = 0: target row (1, 3, 3, 2) has argmax 1 (lowest of the tie);
    drafted token 2 is rejected and token 1 is emitted."""
    T = np.array([[1, 3, 3, 2], [0, 0, 0, 0]], dtype=np.float64)
    D = np.array([[0, 0, 5, 0], [0, 0, 0, 0]], dtype=np.float64)
    r = oracle.verify_sequence(T, D, "f32", [2], 0.0, [0.0], [0.0, 0.0])
    assert (r.accept_len, r.token) == (0, 1)
    np.testing.assert_array_equal(r.p_draft, [0.0])
    np.testing.assert_array_equal(r.q_draft, [1.0])


def test_hand_worked_forks():
    """Draft row (0.5, 2, 2, 1, 2), drafted token 1 masked, f = 3: order by
    (-y, t) gives 2, 4, 3.  At tau = 1 their probabilities are e^2/S, e^2/S,
    e/S with S = e^0.5 + 2e^2 + e (the masked row's softmax)."""
    y = np.array([0.5, 2, 2, 1, 2])
    toks, probs = oracle.forked_topf(y, 1.0, 3, 1)
    assert list(toks) == [2, 4, 3]
    S = math.exp(0.5) + 2 * math.exp(2) + math.exp(1)
    np.testing.assert_allclose(probs, [math.exp(2) / S, math.exp(2) / S, math.e / S], rtol=1e-14)


def test_sample_at_position_agrees_with_verify():
    w = _small_zipf(8, 4, 2500, 0.8, 13, f=0)
    r = oracle.verify_batch(w.target, w.draft, "bf16", w.draft_tokens,
                            w.temperature, w.u_accept, w.u_recover)
    for i in range(w.B):
        tok, flag, _, err = oracle.sample_at_position(
            w.target[i], w.draft[i], "bf16", w.draft_tokens[i],
            w.temperature[i], r.accept_len[i], w.u_recover[i])
        assert not err and tok == r.token[i]


# ---------------------------------------------------------------- cache hits

def test_cache_hit_matches_numpy_search():
    """The hit index is the position of the outcome token in the forks of the
    outcome position (numpy's search over the same table), -1 on a miss or
    an error outcome."""
    rng = np.random.default_rng(5)
    B, K1, f, V = 40, 6, 3, 20
    forks = np.stack([np.stack([rng.choice(V, f, replace=False) for _ in range(K1)])
                      for _ in range(B)])
    n = rng.integers(-1, K1, B)
    tok = rng.integers(-1, V, B)
    got = oracle.cache_hits_batch(forks, n, tok)
    for b in range(B):
        if n[b] < 0 or tok[b] < 0:
            assert got[b] == -1
            continue
        idx = np.flatnonzero(forks[b, n[b]] == tok[b])
        assert got[b] == (idx[0] if idx.size else -1)
    assert (got >= 0).any() and (got == -1).any()


def test_hand_worked_cache_hit_and_miss():
    """k = 1, V = 6.  The target puts almost all mass on token 4 and the
    drafter most of its mass on token 1 (logit 5 against at most 3), so
    drafted token 1 is rejected at position 0 (p/q < e^-19) and the residual
    max(0, p - q), which is positive only at token 4, draws token 4 for any
    u.  Forks at position 0 (token 1 masked, f = 2): draft row
    (-1, 5, 3, 2, 2.5, -3) gives 2 then 4, so the outcome (0, 4) hits at
    index 1; with the row (-1, 5, 3, 2, 0, -3) the forks are 2 then 3 and
    the same outcome misses."""
    T = np.array([[-10, -10, -10, -10, 10, -10], [0, 0, 0, 0, 0, 0]], dtype=np.float64)
    for drow, want_forks, want_hit in (([-1, 5, 3, 2, 2.5, -3], [2, 4], 1),
                                       ([-1, 5, 3, 2, 0, -3], [2, 3], -1)):
        D = np.array([drow, [0, 0, 0, 0, 0, 0]], dtype=np.float64)
        r = oracle.verify_sequence(T, D, "f32", [1], 1.0, [0.5], [0.5, 0.5], f=2)
        assert (r.accept_len, r.token) == (0, 4)
        assert list(r.fork_tokens[0]) == want_forks
        assert oracle.cache_hit(r.fork_tokens[0], r.token) == want_hit


@pytest.mark.parametrize("tau", [0.0, 0.8])
def test_cache_hit_invariants_on_synthetic_batches(tau):
    """A hit names the outcome token among the forks of the outcome
    position; it never names the rejected draft, which the forks exclude."""
    w = _small_zipf(12, 5, 3000, tau, 23)
    r = oracle.verify_batch(w.target, w.draft, "bf16", w.draft_tokens,
                            w.temperature, w.u_accept, w.u_recover, f=3)
    hits = oracle.cache_hits_batch(r.fork_tokens, r.accept_len, r.token)
    for i in range(w.B):
        n = r.accept_len[i]
        if hits[i] >= 0:
            assert r.fork_tokens[i, n, hits[i]] == r.token[i]
        else:
            assert r.token[i] not in list(r.fork_tokens[i, n])
        if n < w.k:
            assert w.draft_tokens[i, n] not in list(r.fork_tokens[i, n])


# ---------------------------------------------------------------- drafter draw

def test_hand_worked_sample_temp():
    """p = (1/2, 1/4, 1/4) at tau = 1: running sums (1/2, 3/4, 1), so u in
    [0, 1/2) draws 0, [1/2, 3/4) draws 1, [3/4, 1) draws 2."""
    x = np.log([0.5, 0.25, 0.25])
    for u, want in ((0.0, 0), (0.49, 0), (0.51, 1), (0.74, 1), (0.76, 2), (0.999, 2)):
        assert oracle.sample_temp(x, 1.0, u)[0] == want, u
    assert oracle.sample_temp(x, 1.0, 0.5)[1]          # on a breakpoint: flagged
    assert oracle.sample_temp([1.0, 3.0, 3.0, 2.0], 0.0, 0.9) == (1, False)  # greedy, lowest tied id


def test_sample_temp_law_is_the_softmax():
    """Over a lattice of 20000 uniforms the draws follow softmax(x / tau)
    (scipy) to within the lattice resolution."""
    rng = np.random.default_rng(3)
    for tau in (0.5, 1.0, 1.7):
        x = rng.normal(0, 1.5, 7)
        p = scipy.special.softmax(x / tau)
        L = 20000
        counts = np.zeros(7)
        for i in range(L):
            counts[oracle.sample_temp(x, tau, (i + 0.5) / L)[0]] += 1
        np.testing.assert_allclose(counts / L, p, atol=2.0 / L)


def test_sample_temp_scaling_and_errors():
    """Drawing from x at tau equals drawing from x / tau at tau = 1; rows
    without a finite maximum, and invalid temperatures, are errors."""
    rng = np.random.default_rng(8)
    x = rng.normal(0, 2, 50)
    for u in rng.random(40):
        a, fa = oracle.sample_temp(x, 0.4, u)
        b, fb = oracle.sample_temp(x / 0.4, 1.0, u)
        if not (fa or fb):
            assert a == b
    toks, flags = oracle.sample_rows(np.stack([x, np.full(50, -np.inf), x]), "f32",
                                     [1.0, 1.0, -1.0], [0.3, 0.3, 0.3])
    assert toks[1] == -1 and toks[2] == -1 and toks[0] >= 0


# ---------------------------------------------------------------- flags
#
# A draw whose uniform lies within 1e-6 of a decision boundary is flagged
# and its sequence left out of the bit-exact comparison.  The band, and the
# rule that only tests up to the first rejection n count, are pinned here on
# hand-built distributions whose acceptance probabilities are exact binary
# fractions (so |u - a| is known without rounding).

def _one_position(p_d, q_d, u, d=1):
    """k = 1, V = 2: p0 and q0 put p_d / q_d on token d; the bonus row is
    uniform.  Returns the verdict."""
    P0 = [1 - p_d, p_d] if d == 1 else [p_d, 1 - p_d]
    Q0 = [1 - q_d, q_d] if d == 1 else [q_d, 1 - q_d]
    return oracle.verify_from_probs([P0, [0.5, 0.5]], [Q0], [d], [u], [0.3, 0.3])


@pytest.mark.parametrize("delta,flagged", [(5e-7, True), (-5e-7, True), (9.9e-7, True),
                                           (2e-6, False), (-2e-6, False), (1.1e-6, False)])
def test_acceptance_flag_band(delta, flagged):
    """a = p/q = 0.25/0.5 = 1/2 exactly; u = 1/2 + delta."""
    v = _one_position(0.25, 0.5, 0.5 + delta)
    assert v.accept_flags == [flagged]
    assert v.flagged == flagged
    # the decision itself is u < a
    assert v.accept_len == (1 if delta < 0 else 0)


def test_acceptance_flag_band_at_a_equal_one():
    """p > q gives a = 1: only u within 1e-6 of 1 is flagged; u = 0 (the
    other end of [0, 1)) is not, and u = 0 is always accepted."""
    assert _one_position(0.75, 0.5, 1 - 2**-24).accept_flags == [True]
    assert _one_position(0.75, 0.5, 1 - 2**-17).accept_flags == [False]
    v = _one_position(0.75, 0.5, 0.0)
    assert v.accept_flags == [False] and v.accept_len == 1


def test_acceptance_flag_band_q_zero_and_p_zero():
    """q(d) = 0 < p(d): a = 1; p(d) = 0: a = 0, so u = 0 is rejected and
    flagged (|0 - 0| < 1e-6), u = 2^-24 rejected and flagged, u = 2^-19
    rejected and not flagged."""
    v = _one_position(0.5, 0.0, 0.5)
    assert v.accept_len == 1 and not v.flagged
    v = _one_position(0.0, 0.5, 0.0)
    assert v.accept_len == 0 and v.accept_flags == [True] and v.flagged
    assert _one_position(0.0, 0.5, 2**-24).flagged
    v = _one_position(0.0, 0.5, 2**-19)
    assert v.accept_len == 0 and not v.flagged


def _three_positions(u_acc):
    """k = 3, V = 2, drafted token 1 everywhere, a_j = 1/2 at every
    position (p = 1/4, q = 1/2).  Residual at a rejection: (1/4, 0) ->
    token 0; bonus row (1/2, 1/2)."""
    P = [[0.75, 0.25]] * 3 + [[0.5, 0.5]]
    Q = [[0.5, 0.5]] * 3
    return oracle.verify_from_probs(P, Q, [1, 1, 1], u_acc, [0.3] * 4)


def test_flags_after_the_first_rejection_do_not_count():
    """Position 0 rejects clearly (u = 0.9 >= 1/2), so n = 0; positions 1
    and 2 sit inside the band, but a flip there cannot change n: the
    sequence is not flagged, though their per-position flags are set."""
    v = _three_positions([0.9, 0.5 + 5e-7, 0.5 - 5e-7])
    assert v.accept_len == 0
    assert v.accept_flags == [False, True, True]
    assert not v.flagged


def test_flag_at_or_before_the_first_rejection_counts():
    # flag at j < n: accepted inside the band, rejected at position 2
    v = _three_positions([0.5 - 5e-7, 0.1, 0.9])
    assert v.accept_len == 2 and v.accept_flags == [True, False, False] and v.flagged
    # flag exactly at j = n: the rejecting test itself is inside the band
    v = _three_positions([0.1, 0.5 + 5e-7, 0.1])
    assert v.accept_len == 1 and v.accept_flags == [False, True, False] and v.flagged
    # every test accepted, the last inside the band (n = k)
    v = _three_positions([0.1, 0.1, 0.5 - 5e-7])
    assert v.accept_len == 3 and v.flagged
    # nothing inside the band
    v = _three_positions([0.1, 0.5 + 2e-6, 0.5 - 2e-6])
    assert v.accept_len == 1 and not v.flagged


def test_draw_flag_band():
    """Inverse CDF over (1/2, 1/2): the breakpoint C_0/Z = 1/2.  u = 1/2
    -/+ 5e-7 picks token 0 / 1, both flagged; 2e-6 away, neither.  A token of
    weight below 2e-6 Z has both its breakpoints within the band, so drawing
    it is always flagged."""
    w = [0.5, 0.5]
    assert oracle.inverse_cdf(w, 0.5 - 5e-7) == (0, True)
    assert oracle.inverse_cdf(w, 0.5 + 5e-7) == (1, True)
    assert oracle.inverse_cdf(w, 0.5 - 2e-6) == (0, False)
    assert oracle.inverse_cdf(w, 0.5 + 2e-6) == (1, False)
    tiny = [0.5, 1.5e-6, 0.5]
    Z = sum(tiny)
    assert oracle.inverse_cdf(tiny, (0.5 + 0.75e-6) / Z) == (1, True)


def test_draw_flag_flags_the_sequence():
    """A clean acceptance followed by a draw inside the band: the sequence
    is flagged through its draw flag alone."""
    P = [[0.75, 0.25], [0.5, 0.5]]
    Q = [[0.5, 0.5]]
    v = oracle.verify_from_probs(P, Q, [1], [0.1], [0.3, 0.5 + 5e-7])
    assert v.accept_len == 1 and v.accept_flags == [False]
    assert v.draw_flag and v.flagged
    v = oracle.verify_from_probs(P, Q, [1], [0.1], [0.3, 0.5 + 2e-6])
    assert not v.draw_flag and not v.flagged


def test_draw_flag_absolute_band():
    """The verify draw's band adds 2^-23 of the unit probability mass (the
    resolution of a cumulative sum of fp32 probabilities) to 1e-6 Z.  Unit
    mass (1/2, 1/2): 1e-6 + 1.2e-7 around 1/2.  Mass 1/100 (1/200, 1/200):
    the absolute part is 1.2e-5 in units of Z.  The plain inverse CDF (no
    absolute band) keeps 1e-6."""
    band = oracle.DRAW_ABS_BAND
    assert band == 2.0 ** -23
    w = [0.5, 0.5]
    assert oracle.inverse_cdf(w, 0.5 + 1.05e-6, band) == (1, True)
    assert oracle.inverse_cdf(w, 0.5 + 1.05e-6) == (1, False)
    assert oracle.inverse_cdf(w, 0.5 + 1.2e-6, band) == (1, False)
    w = [0.005, 0.005]
    assert oracle.inverse_cdf(w, 0.5 + 1e-5, band) == (1, True)
    assert oracle.inverse_cdf(w, 0.5 + 1.5e-5, band) == (1, False)


def test_residual_below_fp32_resolution_is_flagged():
    """p_0 and q_0 agree on token 0 up to 1e-60: the residual (0, 1e-60, 0)
    is exact and positive, the rejection at 0 draws token 1 from it, and
    the draw is flagged (fp32 weights cannot hold that mass).  With a
    residual mass of 1/4 the same draw is clean."""
    F_ = Fraction
    Q = [[F_(1), F_(0), F_(0)]]
    for mass, flagged in [(F_(1, 10**60), True), (F_(1, 4), False)]:
        P = [[1 - mass, mass, F_(0)], [F_(1, 3)] * 3]
        v = oracle.verify_from_probs(P, Q, [2], [F_(1, 2)], [F_(1, 2), F_(1, 2)])
        assert v.accept_len == 0 and v.token == 1
        assert v.accept_flags == [False]
        assert v.draw_flag == flagged and v.flagged == flagged


def test_batch_flag_counts():
    """The batch driver's counts, worked by hand on four sequences built from
    logits with exact probabilities (V = 2, tau = 1): target rows (0, 0)
    give p = (1/2, 1/2); draft rows (0, ln 3) give q = (1/4, 3/4), so the
    drafted token 1 has a = (1/2)/(3/4) = 2/3 (up to the rounding of ln 3 and
    exp, ~1e-16).  k = 2.
      seq 0: u = (2/3 + 5e-7, 0.1)  rejects at 0 inside the band: flagged, 1 draw
      seq 1: u = (0.95, 2/3 - 5e-7) rejects at 0; position 1 in the band but
             after n: not flagged, 0 draws counted
      seq 2: u = (2/3 - 5e-7, 2/3 + 5e-7) accepted then rejected, both in the
             band: flagged, 2 draws
      seq 3: u = (0.1, 0.2)          both accepted (n = k), nothing flagged
    Every rejection leaves the residual max(0, p - q) = (1/4, 0), whose CDF
    breakpoints are 0 and 1, and the bonus row p_2 = (1/2, 1/2) has its
    breakpoint at 1/2: u_recover = 0.3 is far from all of them and picks
    token 0 in both cases."""
    k, V = 2, 2
    T = np.zeros((4, k + 1, V))
    D = np.zeros((4, k + 1, V))
    D[:, :, 1] = math.log(3.0)
    a = 2.0 / 3.0
    ua = np.array([[a + 5e-7, 0.1], [0.95, a - 5e-7], [a - 5e-7, a + 5e-7], [0.1, 0.2]])
    ur = np.full((4, k + 1), 0.3)
    drafts = np.ones((4, k), dtype=np.int64)
    r = oracle.verify_batch(T, D, "f32", drafts, np.ones(4), ua, ur)
    np.testing.assert_array_equal(r.accept_len, [0, 0, 1, 2])
    np.testing.assert_array_equal(r.flagged, [True, False, True, False])
    assert r.n_flagged_draws == 3
    np.testing.assert_array_equal(r.token, [0, 0, 0, 0])


# ---------------------------------------------------------------- small helpers and batch drivers

def test_acceptance_probability_closed_forms():
    F_ = Fraction
    assert oracle.acceptance_probability(F_(3, 10), F_(6, 10)) == F_(1, 2)   # p / q below one
    assert oracle.acceptance_probability(F_(6, 10), F_(3, 10)) == 1          # capped at one
    assert oracle.acceptance_probability(F_(1, 4), F_(1, 4)) == 1
    assert oracle.acceptance_probability(F_(1, 5), F_(0)) == 1               # q = 0 < p
    assert oracle.acceptance_probability(F_(0), F_(0)) == 0                  # p = q = 0
    assert oracle.acceptance_probability(F_(0), F_(1, 3)) == 0
    assert oracle.acceptance_probability(0.25, 0.5) == 0.5


def test_first_rejection():
    assert oracle.first_rejection([True, True, False, True]) == 2
    assert oracle.first_rejection([False, False]) == 0
    assert oracle.first_rejection([True] * 7) == 7
    assert oracle.first_rejection([]) == 0


def test_argmax_first_is_numpys_first_maximum():
    rng = np.random.default_rng(70)
    for _ in range(50):
        x = rng.integers(0, 5, 40).astype(np.float64)     # many ties
        assert oracle.argmax_first(x) == int(np.argmax(x))
    assert oracle.argmax_first(np.array([1.0, 3.0, 3.0, -np.inf])) == 1


def test_softmax_rows_per_row_temperatures_and_errors():
    rng = np.random.default_rng(71)
    x = (rng.standard_normal((5, 300)) * 2).astype(np.float32)
    x[3, :] = -np.inf                                     # no finite entry
    tau = np.array([0.5, 1.0, -1.0, 0.8, np.nan], dtype=np.float32)
    got = oracle.softmax_rows(x, "f32", tau)
    for r in (0, 1):
        np.testing.assert_allclose(got[r], scipy.special.softmax(x[r].astype(np.float64) / tau[r]),
                                   rtol=1e-13, atol=0)
    for r in (2, 3, 4):                                  # bad temperature or row
        assert np.all(np.isnan(got[r]))


def test_forked_topf_batch_rows_and_errors():
    V, k, f = 40, 2, 3
    rng = np.random.default_rng(72)
    D = rng.integers(-3, 4, (3, k + 1, V)).astype(np.float32)   # many ties
    drafts = np.array([[5, 6], [7, 8], [9, V]], dtype=np.int32)  # sequence 2: id out of range
    tau = np.array([0.7, 0.0, 1.0], dtype=np.float32)
    toks, probs = oracle.forked_topf_batch(D, "f32", drafts, tau, f)
    for b in (0, 1):
        for j in range(k + 1):
            excl = int(drafts[b, j]) if j < k else None
            order = sorted((t for t in range(V) if t != excl), key=lambda t: (-D[b, j, t], t))
            assert list(toks[b, j]) == order[:f], (b, j)
        if tau[b] == 0:
            np.testing.assert_array_equal(probs[b][:, 0], 1.0)
            np.testing.assert_array_equal(probs[b][:, 1:], 0.0)
        else:
            for j in range(k + 1):
                y = D[b, j].astype(np.float64).copy()
                if j < k:
                    y[drafts[b, j]] = -np.inf
                q = scipy.special.softmax(y / tau[b])
                np.testing.assert_allclose(probs[b, j], q[toks[b, j]], rtol=1e-13)
    assert np.all(toks[2] == -1) and np.all(np.isnan(probs[2]))
