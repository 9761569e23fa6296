"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on
the seeded workloads, at their full sizes.  Every sequence of the 64-
sequence batch and 96 of the 256-sequence batch (all 64 of its greedy ones
among them) are compared with the oracle, which runs in worker processes;
properties are checked on every sequence."""

import numpy as np
import pytest
import torch

import oracle
from tests import oracle_pool
from tests.gpu_helpers import (assert_flag_share, assert_probs_close,
                               assert_residual_close, compare_verify,
                               dev_inputs, log, residual_tolerance)
from workloads import CONFIGS, make_workload

pytestmark = pytest.mark.gpu

_cache = {}


def workload(name):
    if name not in _cache:
        _cache.clear()
        _cache[name] = make_workload(CONFIGS[name])
    return _cache[name]


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from verification_sampling_amd import specverify
    specverify.lib()
    return specverify


def run_verify(sv, w, x, f):
    out = sv.verify(x["T"], x["D"], x["d"], x["tau"], x["ua"], x["ur"], f=f,
                    want_p=True, want_q=True, want_hits=f > 0)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", ["tiny_verify", "sync_verify_llama_greedy",
                                  "sync_verify_llama_t1", "ssd_step_llama"])
def test_single_sequence_workloads(sv, name):
    cfg = CONFIGS[name]
    log(f"[parity] {name} B={cfg.B} k={cfg.k} V={cfg.V} f={cfg.f} {cfg.dtype}")
    w = workload(name)
    x = dev_inputs(w)
    out = run_verify(sv, w, x, cfg.f)
    ref = oracle.verify_batch(w.target, w.draft, cfg.dtype, w.draft_tokens,
                              w.temperature, w.u_accept, w.u_recover, f=cfg.f)
    seqs = np.arange(w.B)
    nf, n = compare_verify(out, ref, seqs, cfg.f, cfg.k)
    log(f"[parity] {name}: accept_len={out['accept_len'].tolist()} "
        f"token={out['out_token'].tolist()} flagged={nf}/{n}")


def test_tiny_residual_distributions(sv):
    name = "tiny_verify"
    cfg = CONFIGS[name]
    w = workload(name)
    x = dev_inputs(w)
    n_flag = 0
    for pos in range(cfg.k + 1):
        position = torch.full((w.B,), pos, dtype=torch.int32, device="cuda")
        out = sv.residual_sample(x["T"], x["D"], x["d"], x["tau"], position, x["ur"],
                                 want_residual=True)
        torch.cuda.synchronize()
        tok, flag, res, err = oracle.sample_at_position(
            w.target[0], w.draft[0], cfg.dtype, w.draft_tokens[0], w.temperature[0], pos,
            w.u_recover[0], want_residual=True)
        assert not err
        n_flag += int(flag)
        if not flag:
            assert int(out["token"][0]) == tok, (pos, int(out["token"][0]), tok)
        tol = residual_tolerance(w.target[0], w.draft[0], cfg.dtype, float(w.temperature[0]), cfg.k)
        assert_residual_close(out["residual"][0].cpu().numpy(), res, tol, f"residual pos={pos}")
    assert_flag_share(n_flag, cfg.k + 1, "tiny residual draws")
    log("[parity] tiny_verify residual distributions at every position: ok")


def _properties(out, w, f):
    """Checks that hold for every sequence at any size."""
    al = out["accept_len"].cpu().numpy()
    tok = out["out_token"].cpu().numpy()
    k = w.k
    assert np.all((al >= 0) & (al <= k))
    assert np.all((tok >= 0) & (tok < w.V))
    for b in range(w.B):
        if al[b] < k and w.temperature[b] > 0:
            assert tok[b] != w.draft_tokens[b, al[b]]
    if f:
        ft = out["fork_tokens"].cpu().numpy()
        fp = out["fork_probs"].cpu().numpy()
        assert np.all((ft >= 0) & (ft < w.V))
        for b in range(w.B):
            for j in range(k + 1):
                assert len(set(ft[b, j])) == f
                if j < k:
                    assert w.draft_tokens[b, j] not in ft[b, j]
        assert np.all(np.diff(fp, axis=-1) <= 0)
        # cache hits: the outcome token among the forks of the outcome
        # position; the standalone lookup agrees with the fused one
        hits = out["cache_hit"].cpu().numpy()
        for b in range(w.B):
            row = list(ft[b, al[b]])
            assert hits[b] == (row.index(tok[b]) if tok[b] in row else -1), b
        from verification_sampling_amd import specverify
        alone = specverify.cache_hit(out["fork_tokens"], out["accept_len"], out["out_token"])
        torch.cuda.synchronize()
        assert torch.equal(alone, out["cache_hit"])
        log(f"[parity] cache hits {int((hits >= 0).sum())}/{w.B}")


def test_batched_verify_fork_qwen(sv):
    name = "batched_verify_fork_qwen"
    cfg = CONFIGS[name]
    log(f"[parity] {name} B={cfg.B} k={cfg.k} V={cfg.V} f={cfg.f} {cfg.dtype} (full size)")
    w = workload(name)
    x = dev_inputs(w)
    out = run_verify(sv, w, x, cfg.f)
    _properties(out, w, cfg.f)
    seqs = np.arange(cfg.B)
    ref = oracle_pool.verify_batch(w.target, w.draft, cfg.dtype, w.draft_tokens,
                                   w.temperature, w.u_accept, w.u_recover, f=cfg.f, seqs=seqs)
    nf, n = compare_verify(out, ref, seqs, cfg.f, cfg.k)
    log(f"[parity] {name}: compared all {n} sequences, flagged {nf}; accept_len histogram "
        f"{np.bincount(out['accept_len'].cpu().numpy(), minlength=cfg.k + 1).tolist()}")
    # the same call again: bitwise identical
    out2 = run_verify(sv, w, x, cfg.f)
    for key in out:
        assert torch.equal(out[key], out2[key]), key


def test_stress_mixed_tau_fp32(sv):
    name = "stress_mixed_tau_fp32"
    cfg = CONFIGS[name]
    log(f"[parity] {name} B={cfg.B} k={cfg.k} V={cfg.V} f={cfg.f} {cfg.dtype} (full size)")
    w = workload(name)
    x = dev_inputs(w)
    out = run_verify(sv, w, x, cfg.f)
    _properties(out, w, cfg.f)
    greedy = np.flatnonzero(w.temperature == 0)
    warm = np.flatnonzero(w.temperature > 0)
    # every greedy sequence and every sixth of the others (96 of 256)
    seqs = np.sort(np.concatenate([greedy, warm[::6]]))
    assert len(seqs) >= 64
    ref = oracle_pool.verify_batch(w.target, w.draft, cfg.dtype, w.draft_tokens,
                                   w.temperature, w.u_accept, w.u_recover, f=cfg.f, seqs=seqs)
    nf, n = compare_verify(out, ref, seqs, cfg.f, cfg.k)
    log(f"[parity] {name}: verify compared {n} sequences ({len(greedy)} greedy), flagged {nf}")
    # full residual distributions at the outcome positions
    pos = out["accept_len"].clone()
    rs = sv.residual_sample(x["T"], x["D"], x["d"], x["tau"], pos, x["ur"], want_residual=True)
    torch.cuda.synchronize()
    assert torch.equal(rs["token"], out["out_token"])
    res = rs["residual"]
    rseqs = seqs[np.linspace(0, len(seqs) - 1, 16).astype(int)]
    rref = oracle_pool.verify_batch(w.target, w.draft, cfg.dtype, w.draft_tokens,
                                    w.temperature, w.u_accept, w.u_recover, want_residual=True,
                                    seqs=rseqs)
    for i, b in enumerate(rseqs):
        tol = residual_tolerance(w.target[b], w.draft[b], cfg.dtype, float(w.temperature[b]), cfg.k)
        assert_residual_close(res[b].cpu().numpy(), rref.residual[i], tol, f"residual seq {b}")
    log(f"[parity] {name}: residual distributions of {len(rseqs)} sequences (every row): ok")
