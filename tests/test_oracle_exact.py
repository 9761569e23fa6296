"""Exact pins of the oracle's decision code (acceptance, first rejection,
residual, inverse CDF), on rational distributions with fractions.Fraction.

The property pinned is the one the pages lead with: the method is exact, the
emitted tokens follow the target distribution ("What changes in SSD",
hysenlabs.com editorial).  Each emitted token j, given the emitted prefix and
given that at least j+1 tokens are emitted, must have law p_j(. | prefix)
exactly.  Drafts are drawn from q; every uniform ranges over the midpoints of
a lattice of L cells that contains every decision boundary, so the counts
are exact.  All probabilities below are multiples of 1/4, so every
acceptance probability p/q and every CDF breakpoint C_t/Z is a fraction with
denominator at most 4, and L = lcm(1..4) = 12 makes each cell lie inside a
single decision interval.
"""

import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle

L = 12


def quarter_grid(V):
    """All distributions over V tokens with entries in {0, 1/4, ..., 1}."""
    out = []
    for parts in itertools.product(range(5), repeat=V):
        if sum(parts) == 4:
            out.append(tuple(Fraction(c, 4) for c in parts))
    return out


def cells():
    return [Fraction(2 * i + 1, 2 * L) for i in range(L)]


def make_model(V, seed):
    """Prefix-dependent rational target p_j(.|s) and draft q_j(.|s)."""
    grid = quarter_grid(V)
    rng = np.random.default_rng(seed)
    table_p, table_q = {}, {}

    def pick(table, key):
        if key not in table:
            table[key] = grid[int(rng.integers(len(grid)))]
        return table[key]

    def p(j, prefix):
        return pick(table_p, (j, tuple(prefix)))

    def q(j, prefix):
        # Every fourth context the drafter equals the target (p = q case).
        if hash((j, tuple(prefix), seed)) % 4 == 0:
            return p(j, prefix)
        return pick(table_q, (j, tuple(prefix)))

    return p, q


def emitted_law(V, k, p, q):
    """Exact law of emitted sequences: dict tuple -> Fraction."""
    law = {}
    us = cells()
    w_cell = Fraction(1, L)
    for drafts in itertools.product(range(V), repeat=k):
        w_d = Fraction(1)
        for j in range(k):
            w_d *= q(j, drafts[:j])[drafts[j]]
        if w_d == 0:
            continue
        P = [p(j, drafts[:j]) for j in range(k + 1)]
        Q = [q(j, drafts[:j]) for j in range(k)]
        for ua in itertools.product(us, repeat=k):
            for ur in us:
                v = oracle.verify_from_probs(P, Q, list(drafts), list(ua),
                                             [ur] * (k + 1))
                assert not v.flagged
                seq = tuple(drafts[: v.accept_len]) + (v.token,)
                law[seq] = law.get(seq, 0) + w_d * w_cell ** (k + 1)
    return law


def check_law(V, k, p, law):
    assert sum(law.values()) == 1
    for j in range(k + 1):
        # mass of (prefix of length j, token j) among sequences longer than j
        joint, marg = {}, {}
        for s, w in law.items():
            if len(s) > j:
                joint[s[: j + 1]] = joint.get(s[: j + 1], 0) + w
                marg[s[:j]] = marg.get(s[:j], 0) + w
        for pre, m in marg.items():
            target = p(j, pre)
            for t in range(V):
                got = joint.get(pre + (t,), Fraction(0)) / m
                assert got == target[t], (j, pre, t, got, target[t])


@pytest.mark.parametrize("V,k,seed", [(2, 1, 0), (3, 1, 1), (4, 1, 2),
                                      (2, 2, 3), (3, 2, 4), (3, 2, 5)])
def test_emitted_tokens_follow_target_exactly(V, k, seed):
    p, q = make_model(V, seed)
    law = emitted_law(V, k, p, q)
    check_law(V, k, p, law)


def test_emitted_tokens_follow_target_exactly_k3():
    p, q = make_model(2, 7)
    law = emitted_law(2, 3, p, q)
    check_law(2, 3, p, law)


@pytest.mark.parametrize("V,seed", [(2, 10), (3, 11), (4, 12)])
def test_acceptance_rate_closed_form(V, seed):
    """P(first drafted token accepted) = sum_t min(p_t, q_t): the expected
    acceptance of speculative sampling, derived independently of the rule's
    code (Leviathan et al., 2023)."""
    p, q = make_model(V, seed)
    P0, Q0 = p(0, ()), q(0, ())
    acc = Fraction(0)
    for d in range(V):
        if Q0[d] == 0:
            continue
        for ua in cells():
            v = oracle.verify_from_probs([P0, P0], [Q0], [d], [ua], [cells()[0]] * 2)
            if v.accept_len == 1:
                acc += Q0[d] * Fraction(1, L)
    assert acc == sum(min(a, b) for a, b in zip(P0, Q0))


def test_inverse_cdf_law_exact():
    """Over a fine lattice of uniforms the inverse CDF hits each token with
    frequency w_t / Z exactly, and never a zero-weight token."""
    rng = np.random.default_rng(3)
    for _ in range(20):
        V = int(rng.integers(1, 7))
        w = [Fraction(int(rng.integers(0, 4)), 4) for _ in range(V)]
        if sum(w) == 0:
            w[int(rng.integers(V))] = Fraction(1, 4)
        Z = sum(w)
        # breakpoints are multiples of 1/(4 Z') where Z' = 4Z
        Lw = 4 * int(Z * 4) * 2
        counts = [0] * V
        for i in range(Lw):
            tok, flag = oracle.inverse_cdf(w, Fraction(2 * i + 1, 2 * Lw))
            assert not flag
            counts[tok] += 1
        for t in range(V):
            assert Fraction(counts[t], Lw) == w[t] / Z


def test_zero_residual_falls_back_to_target():
    P = [Fraction(1, 4), Fraction(3, 4)]
    assert oracle.residual_weights(P, P) == P
    # rejection is impossible when p = q: a = 1 > u for every u < 1
    for u in cells():
        v = oracle.verify_from_probs([P, P], [P], [1], [u], [u, u])
        assert v.accept_len == 1
