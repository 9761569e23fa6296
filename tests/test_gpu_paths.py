"""GPU parity on the kernel paths that ordinary logits do not reach.

- Fork candidates that fill a lane's slots while a long segment streams, so
  that they are ranked inside the streaming loop, and segments with more
  candidate vectors than they may pass on: flat, staircase and tie-block
  draft rows in a 256-sequence fp32 batch and a 64-sequence bf16 batch.
  Flat and tied rows keep every vector a candidate at temperature > 0;
  an ascending staircase keeps beating the running f-th value at
  temperature 0.
- Rows of more than 256 chunks (fp32 V > 262144, bf16 V > 524288), up to
  the largest vocabulary the library accepts, where the chunk totals of the
  draw no longer fit the registers of one wave.
- Residuals of total zero (target and draft rows equal at the drawn
  position), which fall back to the target distribution.
- The largest batches a call accepts (32,768 rows).
- Fork candidates' keys where they are largest (small temperatures, large
  logits) or crowded within their rounding margin (narrow bands of logits
  at large temperatures).

Every comparison is against the oracle on the same inputs; tokens and forks
exactly, probabilities to 1e-5 relative.
"""

import numpy as np
import pytest
import torch

import oracle
from tests import oracle_pool
from tests.gpu_helpers import (assert_flag_share, assert_probs_close,
                               assert_residual_close, compare_verify, log,
                               padded_dev, residual_tolerance)
from workloads import Config, f32_to_bf16_bits, make_workload, uniforms

pytestmark = pytest.mark.gpu

MAX_V = 1048576          # largest vocabulary of verify, residuals and softmax
MAX_V_SAMPLE_BF16 = 2097152


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from verification_sampling_amd import specverify
    specverify.lib()
    return specverify


def _store(x32, dtype):
    x32 = np.asarray(x32, dtype=np.float32)
    return f32_to_bf16_bits(x32) if dtype == "bf16" else x32


def _flat(V, dtype):
    return _store(np.zeros(V, np.float32), dtype)


def _staircase(V, dtype):
    # non-decreasing in id, plateaus of 512 equal values (merged further by
    # bf16 rounding); the top plateau sits at the end of the row
    return _store(np.floor(np.arange(V) / 512.0) * 0.0078125, dtype)


def _tie_block(row, lo, hi, dtype):
    # a block of equal values above everything else in the row
    x = row.copy()
    top = oracle.widen(row, dtype).max() + 1.0
    x[lo:hi] = _store(np.full(hi - lo, top, np.float32), dtype)
    return x


def _verify(sv, w_T, w_D, dtype, drafts, tau, ua, ur, f):
    out = sv.verify(padded_dev(w_T, dtype), padded_dev(w_D, dtype),
                    torch.from_numpy(drafts).cuda(), torch.from_numpy(tau).cuda(),
                    torch.from_numpy(ua).cuda(), torch.from_numpy(ur).cuda(), f=f,
                    want_p=True, want_q=True, want_hits=True)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype,B,f", [("f32", 256, 3), ("bf16", 64, 16)])
def test_fork_candidates_overflow_long_segments(sv, dtype, B, f):
    k, V = 7, 151936
    log(f"[paths] candidate overflow {dtype} B={B} k={k} V={V} f={f}")
    w = make_workload(Config("paths", B=B, k=k, V=V, f=f, dtype=dtype, profile="zipf",
                             seed=7100 + B + f, tau_mixed=(0.5, 1.2), sigma_range=(0.3, 1.2)))
    D = w.draft
    tau = w.temperature.copy()
    drafts = w.draft_tokens.copy()
    stair = _staircase(V, dtype)
    top_ids = np.flatnonzero(oracle.widen(stair, dtype) == oracle.widen(stair, dtype).max())
    top_lo = int(top_ids[0])               # first id of the staircase's top plateau
    assert len(top_ids) > f + 1
    for i in range(24):
        b = i
        kind = ("flat", "stair", "ties")[i // 8]
        tau[b] = 0.0 if i % 2 else 0.7 + 0.05 * (i % 4)
        for j in range(k + 1):
            if kind == "flat":
                D[b, j] = _flat(V, dtype)
            elif kind == "stair":
                D[b, j] = stair
            else:
                lo = 20000 + 9000 * j
                D[b, j] = _tie_block(D[b, j], lo, lo + 5000, dtype)
        # drafted tokens where the masking decides the forks
        if kind == "flat":
            drafts[b, 0] = 0
            drafts[b, 1] = 1
        elif kind == "stair":
            drafts[b, 2] = top_lo
        else:
            drafts[b, 0] = 20000
    out = _verify(sv, w.target, D, dtype, drafts, tau, w.u_accept, w.u_recover, f)
    seqs = np.concatenate([np.arange(24), np.arange(24, B, 8)])
    ref = oracle_pool.verify_batch(w.target, D, dtype, drafts, tau, w.u_accept, w.u_recover,
                                   f=f, seqs=seqs)
    nf, n = compare_verify(out, ref, seqs, f, k)
    # the oracle's forks of these rows, from their construction: the lowest
    # ids of the top tie that are not the drafted token
    ft = ref.fork_tokens
    assert list(ft[0, 0]) == list(range(1, f + 1))                 # flat, id 0 drafted
    assert list(ft[0, 1]) == [0] + list(range(2, f + 1))           # flat, id 1 drafted
    assert list(ft[0, 7]) == list(range(f))                        # bonus row: nothing masked
    assert list(ft[8, 2]) == [int(t) for t in top_ids[1:f + 1]]     # staircase, top_lo drafted
    assert list(ft[16, 0]) == list(range(20001, 20001 + f))
    log(f"[paths] candidate overflow {dtype}: compared {n} sequences, flagged {nf}")


# (scale of the logits, offset, temperature) per sequence: keys largest
# (small temperatures, logits of large magnitude, a large offset that makes
# the reference large), keys crowded within their margin (a narrow band of
# logits at large temperatures), and ordinary rows between them
_KEY_CASES = [(40.0, 0.0, 0.02), (40.0, 0.0, 0.05), (40.0, 0.0, 0.1), (40.0, 0.0, 0.3),
              (1e-3, 0.0, 4.0), (1e-3, 0.0, 20.0), (1e-3, 0.0, 0.7), (1e-3, 0.0, 100.0),
              (1.0, 0.0, 0.7), (1.0, 0.0, 0.0), (1.0, 0.0, 1.5), (1.0, 0.0, 0.05),
              (1.0, 1000.0, 0.05), (1.0, 1000.0, 0.7), (1.0, -1000.0, 0.3), (4.0, 500.0, 0.02)]


@pytest.mark.parametrize("dtype,f", [("bf16", 3), ("f32", 3), ("bf16", 16)])
def test_fork_candidate_keys_at_extreme_scales(sv, dtype, f):
    """Later-chunk fork candidates at temperature > 0 carry a key that bounds
    their maximum from both sides, widened by a rounding margin; a margin
    too tight would skip a vector that holds one of the top f.  Whole
    batches at the scales where the keys are largest or most crowded."""
    B, k, V = len(_KEY_CASES), 3, 151936
    log(f"[paths] fork keys {dtype} B={B} k={k} V={V} f={f}")
    w = make_workload(Config("keys", B=B, k=k, V=V, f=f, dtype=dtype, profile="zipf",
                             seed=7300 + f + (dtype == "f32"), tau=0.7,
                             sigma_range=(0.3, 1.2)))
    T, D = w.target.copy(), w.draft.copy()
    tau = np.empty(B, np.float32)
    for b, (scale, offset, t) in enumerate(_KEY_CASES):
        for X in (T, D):
            x = oracle.widen(X[b], dtype) * scale + offset
            X[b] = _store(x.astype(np.float32), dtype)
        tau[b] = t
    out = _verify(sv, T, D, dtype, w.draft_tokens, tau, w.u_accept, w.u_recover, f)
    ref = oracle.verify_batch(T, D, dtype, w.draft_tokens, tau, w.u_accept, w.u_recover, f=f)
    # Forks and their probabilities are compared for every sequence.  These
    # rows flag many draws on purpose: near-uniform rows put a draw inside
    # the 1e-6 band of a CDF step about a third of the time, and at the
    # smallest temperatures target and draft agree so closely that the
    # residual's mass falls below the fp32 resolution band of the draw.  So
    # the flagged share is bounded at a quarter here, not 5 %.
    nf, n = compare_verify(out, ref, np.arange(B), f, k, bound_flags=False)
    assert nf <= B // 4, np.flatnonzero(ref.flagged)
    log(f"[paths] fork keys {dtype} f={f}: compared {n} sequences, flagged {nf}")


@pytest.mark.parametrize("dtype,V", [("f32", 300000), ("bf16", 600000), ("f32", MAX_V)])
def test_rows_over_256_chunks(sv, dtype, V):
    """Verify with forks (warm and greedy), then every residual row and the
    draw at the outcome position and at position 0."""
    B, k, f = 2, 3, 3
    log(f"[paths] long rows {dtype} V={V}")
    w = make_workload(Config("paths", B=B, k=k, V=V, f=f, dtype=dtype, profile="zipf",
                             seed=7200 + V % 9973, tau=0.8, sigma_range=(0.3, 1.2)))
    tau = w.temperature.copy()
    tau[1] = 0.0
    out = _verify(sv, w.target, w.draft, dtype, w.draft_tokens, tau, w.u_accept, w.u_recover, f)
    ref = oracle.verify_batch(w.target, w.draft, dtype, w.draft_tokens, tau, w.u_accept,
                              w.u_recover, f=f)
    compare_verify(out, ref, np.arange(B), f, k)
    T_d, D_d = padded_dev(w.target, dtype), padded_dev(w.draft, dtype)
    d = torch.from_numpy(w.draft_tokens).cuda()
    n_flag = n_cmp = 0
    for pos in (out["accept_len"].cpu().numpy().astype(np.int32), np.zeros(B, np.int32)):
        rs = sv.residual_sample(T_d, D_d, d, torch.from_numpy(tau).cuda(),
                                torch.from_numpy(pos).cuda(),
                                torch.from_numpy(w.u_recover).cuda(), want_residual=True)
        alone = sv.residual_sample(T_d, D_d, d, torch.from_numpy(tau).cuda(),
                                   torch.from_numpy(pos).cuda(),
                                   torch.from_numpy(w.u_recover).cuda())
        torch.cuda.synchronize()
        assert torch.equal(alone["token"], rs["token"])
        for b in range(B):
            tok, flag, res, err = oracle.sample_at_position(
                w.target[b], w.draft[b], dtype, w.draft_tokens[b], tau[b], int(pos[b]),
                w.u_recover[b], want_residual=True)
            assert not err
            n_cmp += 1
            n_flag += int(flag)
            if not flag:
                assert int(rs["token"][b]) == tok, (b, int(pos[b]), int(rs["token"][b]), tok)
            tol = residual_tolerance(w.target[b], w.draft[b], dtype, float(tau[b]), k)
            assert_residual_close(rs["residual"][b].cpu().numpy(), res, tol,
                                  f"residual b={b} pos={int(pos[b])}")
    assert_flag_share(n_flag, n_cmp, "long-row draws")
    log(f"[paths] long rows {dtype} V={V}: ok")


@pytest.mark.parametrize("dtype,V", [("f32", 151936), ("bf16", 151936), ("f32", 300000)])
def test_zero_residual_falls_back_to_target(sv, dtype, V):
    """Draft rows equal to the target rows: every residual max(p - q, 0) is
    zero, so the draw at a position n < k and the residual rows are those of
    the target distribution p."""
    B, k = 4, 3
    log(f"[paths] zero residual {dtype} V={V}")
    w = make_workload(Config("paths", B=B, k=k, V=V, f=0, dtype=dtype, profile="zipf",
                             seed=7300 + V % 9973, tau=0.9, sigma_range=(0.3, 1.2)))
    T = w.target
    tau = np.array([0.7, 1.0, 0.0, 0.9], dtype=np.float32)
    pos = np.array([0, 2, 1, 1], dtype=np.int32)
    T_d = padded_dev(T, dtype)
    D_d = padded_dev(T.copy(), dtype)
    d = torch.from_numpy(w.draft_tokens).cuda()
    rs = sv.residual_sample(T_d, D_d, d, torch.from_numpy(tau).cuda(),
                            torch.from_numpy(pos).cuda(), torch.from_numpy(w.u_recover).cuda(),
                            want_residual=True)
    alone = sv.residual_sample(T_d, D_d, d, torch.from_numpy(tau).cuda(),
                               torch.from_numpy(pos).cuda(),
                               torch.from_numpy(w.u_recover).cuda())
    torch.cuda.synchronize()
    assert torch.equal(alone["token"], rs["token"])
    n_flag = 0
    for b in range(B):
        tok, flag, res, err = oracle.sample_at_position(
            T[b], T[b], dtype, w.draft_tokens[b], tau[b], int(pos[b]), w.u_recover[b],
            want_residual=True)
        assert not err
        n_flag += int(flag)
        if not flag:
            assert int(rs["token"][b]) == tok, (b, int(rs["token"][b]), tok)
        got = rs["residual"][b].cpu().numpy()
        tol = residual_tolerance(T[b], T[b], dtype, float(tau[b]), k)
        assert_residual_close(got, res, tol, f"residual b={b}")
        if tau[b] > 0:
            # the fallback is p itself at every position
            P = np.stack([oracle.softmax_temp(oracle.widen(T[b, j], dtype), float(tau[b]))
                          for j in range(k + 1)])
            assert_probs_close(got, P, f"fallback rows b={b}")
    assert_flag_share(n_flag, B, "zero-residual draws")
    log(f"[paths] zero residual {dtype} V={V}: ok")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_largest_vocabulary_softmax_and_sampling(sv, dtype):
    """softmax_temp at the largest V it accepts, and the drafter's draw at the
    largest V of its own (twice that for bf16)."""
    rng = np.random.default_rng(7400 if dtype == "f32" else 7401)
    V = MAX_V
    x32 = (rng.standard_normal((3, V)) * 2.0).astype(np.float32)
    host = _store(x32, dtype)
    tau = np.array([0.0, 0.6, 1.3], dtype=np.float32)
    dev = padded_dev(host[None], dtype)[0]
    pr = sv.softmax_temp(dev, torch.from_numpy(tau).cuda())
    torch.cuda.synchronize()
    assert_probs_close(pr.cpu().numpy(), oracle.softmax_rows(host, dtype, tau), "softmax rows")
    Vs = MAX_V_SAMPLE_BF16 if dtype == "bf16" else MAX_V
    x32 = (rng.standard_normal((4, Vs)) * 1.5).astype(np.float32)
    host = _store(x32, dtype)
    tau = np.array([0.0, 0.5, 0.9, 1.4], dtype=np.float32)
    u = uniforms(rng, (4,))
    got = sv.sample_temp(padded_dev(host[None], dtype)[0], torch.from_numpy(tau).cuda(),
                         torch.from_numpy(u).cuda())
    torch.cuda.synchronize()
    ref, flagged = oracle.sample_rows(host, dtype, tau, u)
    assert_flag_share(int(flagged.sum()), 4, "sample_temp")
    g = got.cpu().numpy()
    for r in range(4):
        if not flagged[r]:
            assert g[r] == ref[r], (r, int(g[r]), int(ref[r]))
    log(f"[paths] largest vocabulary softmax / sampling {dtype}: ok")


@pytest.mark.parametrize("B,k", [(4096, 7), (8192, 3)])
def test_largest_batches(sv, B, k):
    """The largest batches a call accepts (32,768 rows), at a small
    vocabulary: every sequence's outputs against the oracle on a sample,
    and the properties on all."""
    V, f = 64, 3
    log(f"[paths] largest batch B={B} k={k} V={V} f={f}")
    w = make_workload(Config("paths", B=B, k=k, V=V, f=f, dtype="bf16", profile="zipf",
                             seed=7500 + B, tau_mixed=(0.5, 1.2), sigma_range=(0.3, 1.2)))
    out = _verify(sv, w.target, w.draft, "bf16", w.draft_tokens, w.temperature, w.u_accept,
                  w.u_recover, f)
    al = out["accept_len"].cpu().numpy()
    assert np.all((al >= 0) & (al <= k))
    ft = out["fork_tokens"].cpu().numpy()
    assert np.all((ft >= 0) & (ft < V))
    seqs = np.arange(0, B, B // 256)
    ref = oracle_pool.verify_batch(w.target, w.draft, "bf16", w.draft_tokens, w.temperature,
                                   w.u_accept, w.u_recover, f=f, seqs=seqs)
    nf, n = compare_verify(out, ref, seqs, f, k)
    log(f"[paths] largest batch B={B}: compared {n} sequences, flagged {nf}")
