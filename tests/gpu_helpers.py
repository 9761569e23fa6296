"""Shared helpers of the GPU parity tests: device copies of a workload and
the comparison rule against the oracle.

Comparison rule: token ids, accepted lengths and fork tokens bit-exact for
every sequence the oracle does not flag (a flagged sequence has a uniform
within 1e-6 of a decision boundary); probabilities within 1e-5 relative
(|gpu - ref| <= 1e-5 |ref| + 1e-30); residual probabilities within
1e-5 (p_t + q_t) / Z, since a difference of nearly equal probabilities has
no meaningful relative error.
"""

import sys

import numpy as np
import torch

import oracle

RTOL = 1e-5
ATOL = 1e-30
# Flagged sequences (a uniform within the band of a decision boundary) are
# left out of the exact comparison; at most this share of the compared
# sequences may be flagged (one, in a batch of fewer than 20), so that a
# flag rule that over-fires cannot shrink a comparison unnoticed.  The
# inputs are seeded, so the count is fixed for each test.
MAX_FLAG_SHARE = 0.05


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(arr, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def _pad(n, dtype):
    m = 8 if dtype == "bf16" else 4
    return (n + m - 1) // m * m


def padded_dev(arr, dtype):
    """Device copy of [B, K1, V] logits in a row-padded buffer (16-byte
    aligned rows), returned as a [B, K1, V] view."""
    B, K1, V = arr.shape
    Vp = _pad(V, dtype)
    host = np.zeros((B, K1, Vp), dtype=arr.dtype)
    host[:, :, :V] = arr
    return to_dev(host, dtype)[:, :, :V]


def dev_inputs(w):
    return dict(
        T=to_dev(w.target, w.dtype), D=to_dev(w.draft, w.dtype),
        d=torch.from_numpy(np.ascontiguousarray(w.draft_tokens)).cuda(),
        tau=torch.from_numpy(np.ascontiguousarray(w.temperature)).cuda(),
        ua=torch.from_numpy(np.ascontiguousarray(w.u_accept)).cuda(),
        ur=torch.from_numpy(np.ascontiguousarray(w.u_recover)).cuda())


def assert_probs_close(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), f"{what}: NaN pattern differs"
    g, r = got[~nan_ref], ref[~nan_ref]
    bad = np.abs(g - r) > RTOL * np.abs(r) + ATOL
    if bad.any():
        i = np.flatnonzero(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside 1e-5 rel: "
                             f"got {g[i]} ref {r[i]}")


def assert_flag_share(n_flagged, n_compared, what=""):
    assert n_flagged <= max(1.0, MAX_FLAG_SHARE * n_compared), (
        f"{what}: {n_flagged} of {n_compared} flagged (more than {MAX_FLAG_SHARE:.0%})")


def compare_verify(out, ref, seqs, f, k, want_p=True, want_q=True, bound_flags=True):
    """Compares the GPU outputs (full batch) at sequences `seqs` with the
    oracle's BatchResult over the same sequences, and (unless bound_flags is
    False, for batches built to be near-uniform) bounds the share of flagged
    sequences.  Returns (n_flagged, n_compared)."""
    al = out["accept_len"].cpu().numpy()[seqs]
    tok = out["out_token"].cpu().numpy()[seqs]
    n_flag = 0
    for i in range(len(seqs)):
        if ref.error[i]:
            assert al[i] == -1 and tok[i] == -1, (seqs[i], al[i], tok[i])
            continue
        if ref.flagged[i]:
            n_flag += 1
            continue
        assert al[i] == ref.accept_len[i], (int(seqs[i]), int(al[i]), int(ref.accept_len[i]))
        assert tok[i] == ref.token[i], (int(seqs[i]), int(tok[i]), int(ref.token[i]))
    if want_p:
        assert_probs_close(out["p_draft"].cpu().numpy()[seqs], ref.p_draft, "p_draft")
    if want_q:
        assert_probs_close(out["q_draft"].cpu().numpy()[seqs], ref.q_draft, "q_draft")
    if f:
        ft = out["fork_tokens"].cpu().numpy()[seqs]
        np.testing.assert_array_equal(ft, ref.fork_tokens, err_msg="fork tokens")
        assert_probs_close(out["fork_probs"].cpu().numpy()[seqs], ref.fork_probs, "fork probs")
    if f and "cache_hit" in out:
        # the oracle's lookup of its own outcome in its own forks
        ref_hits = oracle.cache_hits_batch(ref.fork_tokens, ref.accept_len, ref.token)
        hits = out["cache_hit"].cpu().numpy()[seqs]
        for i in range(len(seqs)):
            if ref.flagged[i] and not ref.error[i]:
                continue
            assert hits[i] == ref_hits[i], (int(seqs[i]), int(hits[i]), int(ref_hits[i]))
    if bound_flags:
        assert_flag_share(n_flag, int((~np.asarray(ref.error)).sum()), "verify")
    return n_flag, len(seqs)


def residual_tolerance(T, D, dtype, tau, k):
    """Per-element tolerance of the normalised residual rows of one
    sequence: 1e-5 (p + q) / Z for j < k, 1e-5 p at j = k (float64)."""
    V = T.shape[-1]
    tol = np.empty((k + 1, V))
    for j in range(k + 1):
        P = oracle.softmax_temp(oracle.widen(T[j], dtype), tau)
        if j < k:
            Q = oracle.softmax_temp(oracle.widen(D[j], dtype), tau)
            w = np.maximum(P - Q, 0)
            Z = w.sum()
            tol[j] = RTOL * (P + Q) / Z if Z > 0 else RTOL * P
        else:
            tol[j] = RTOL * P
    return tol + ATOL


def assert_residual_close(got, ref, tol, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), f"{what}: NaN pattern differs"
    d = np.abs(got - ref)
    bad = (d > tol) & ~nan_ref
    if bad.any():
        i = np.flatnonzero(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} elements outside tolerance: got "
                             f"{got.ravel()[i]} ref {ref.ravel()[i]} tol {tol.ravel()[i]}")
