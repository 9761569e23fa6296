"""GPU parity on edge cases: ragged and tiny vocabularies, k = 1 and 63,
f = 1, 16 and V-1, ties, identical and disjoint drafters, error sequences,
empty batches, strided inputs, every draw position, softmax rows and the
standalone fork call."""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import (assert_flag_share, assert_probs_close,
                               assert_residual_close, compare_verify, log,
                               padded_dev, residual_tolerance, to_dev)
from workloads import Config, f32_to_bf16_bits, make_workload, uniforms

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from verification_sampling_amd import specverify
    specverify.lib()
    return specverify


def run_case(sv, T, D, dtype, drafts, tau, ua, ur, f, want_q=True):
    x = dict(T=padded_dev(T, dtype), D=padded_dev(D, dtype))
    out = sv.verify(x["T"], x["D"], torch.from_numpy(drafts).cuda(), torch.from_numpy(tau).cuda(),
                    torch.from_numpy(ua).cuda(), torch.from_numpy(ur).cuda(), f=f,
                    want_p=True, want_q=want_q, want_hits=f > 0)
    torch.cuda.synchronize()
    ref = oracle.verify_batch(T, D, dtype, drafts, tau, ua, ur, f=f, want_q=want_q)
    nf, n = compare_verify(out, ref, np.arange(T.shape[0]), f, drafts.shape[1], want_q=want_q)
    return out, ref, nf


def synth(B, k, V, dtype, tau, seed, f=0):
    return make_workload(Config("edge", B=B, k=k, V=V, f=f, dtype=dtype, profile="zipf",
                                seed=seed, tau=tau, sigma_range=(0.3, 1.2)))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [2, 7, 1000, 2049, 4095, 4097, 8200, 20000])
def test_ragged_vocabularies(sv, dtype, V):
    for tau in (0.0, 0.8):
        for f in sorted({0, 1, min(3, V - 1)}):
            w = synth(3, 3, V, dtype, tau, seed=V * 7 + int(tau * 10) + f, f=f)
            run_case(sv, w.target, w.draft, dtype, w.draft_tokens, w.temperature,
                     w.u_accept, w.u_recover, f)
    log(f"[edges] ragged V={V} {dtype}: ok")


def test_k_limits_and_fan_outs(sv):
    for (k, V, f, dtype) in [(1, 3000, 2, "bf16"), (63, 3000, 3, "bf16"), (63, 1500, 16, "f32"),
                             (4, 5000, 16, "bf16"), (3, 9, 8, "bf16"), (2, 17, 16, "f32"),
                             (5, 33, 5, "bf16")]:
        for tau in (0.0, 1.1):
            w = synth(2, k, V, dtype, tau, seed=k * 100 + V + f, f=f)
            run_case(sv, w.target, w.draft, dtype, w.draft_tokens, w.temperature,
                     w.u_accept, w.u_recover, f)
    log("[edges] k in {1, 63}, f in {2, 3, 5, 8, 16}: ok")


def test_ties_everywhere(sv):
    B, k, V = 3, 4, 3000
    T = np.zeros((B, k + 1, V), dtype=np.float32)
    T[:, :, 100:110] = 1.0  # ten-way tie at the top
    D = T.copy()
    D[1] = 0.0              # flat drafter
    rng = np.random.default_rng(1)
    drafts = rng.integers(100, 110, (B, k)).astype(np.int32)
    drafts[0, 0] = 100
    for tau in (0.0, 0.7):
        taus = np.full(B, tau, dtype=np.float32)
        out, ref, nf = run_case(sv, T, D, "f32", drafts, taus, uniforms(rng, (B, k)),
                                uniforms(rng, (B, k + 1)), 3)
        if tau == 0.0:
            # greedy argmax is the lowest tied id
            assert ref.token[0] in (100, 101)
    log("[edges] ties: ok")


def test_identical_and_disjoint_drafters(sv):
    w = synth(4, 5, 6000, "bf16", 0.9, seed=5, f=3)
    out, ref, _ = run_case(sv, w.target, w.target, "bf16", w.draft_tokens, w.temperature,
                           w.u_accept, w.u_recover, 3)
    assert np.all(out["accept_len"].cpu().numpy() == 5)
    B, k, V = 2, 3, 600
    T = np.full((B, k + 1, V), -np.inf, dtype=np.float32)
    D = np.full((B, k + 1, V), -np.inf, dtype=np.float32)
    T[:, :, :300] = 0.5
    D[:, :, 300:] = 0.25
    drafts = np.array([[301, 302, 303], [400, 500, 599]], dtype=np.int32)
    rng = np.random.default_rng(2)
    out, ref, _ = run_case(sv, T, D, "f32", drafts, np.full(B, 1.0, np.float32),
                           uniforms(rng, (B, k)), uniforms(rng, (B, k + 1)), 2)
    assert np.all(out["accept_len"].cpu().numpy() == 0)
    assert np.all(out["out_token"].cpu().numpy() < 300)
    log("[edges] identical / disjoint drafters: ok")


def test_error_sequences(sv):
    B, k, V = 6, 3, 2500
    w = synth(B, k, V, "bf16", 0.8, seed=9, f=2)
    T, D = w.target.copy(), w.draft.copy()
    drafts = w.draft_tokens.copy()
    tau = w.temperature.copy()
    drafts[0, 1] = V          # drafted id out of range
    drafts[1, 2] = -3
    tau[2] = -0.5             # negative temperature
    tau[3] = np.nan
    ninf = f32_to_bf16_bits(np.array([-np.inf], dtype=np.float32))[0]
    pinf = f32_to_bf16_bits(np.array([np.inf], dtype=np.float32))[0]
    T[4, 2, :] = ninf          # target row with no finite entry
    D[5, 1, 17] = pinf         # draft row with +inf
    out, ref, _ = run_case(sv, T, D, "bf16", drafts, tau, w.u_accept, w.u_recover, 2)
    assert ref.error[:6].all()
    ft = out["fork_tokens"].cpu().numpy()
    assert np.all(ft[:6] == -1)
    assert np.all(np.isnan(out["fork_probs"].cpu().numpy()[:6]))
    assert np.all(np.isnan(out["p_draft"].cpu().numpy()[:6]))
    assert np.all(out["cache_hit"].cpu().numpy()[:6] == -1)
    log("[edges] error sequences: ok")


def test_empty_batch_and_strided_inputs(sv):
    w = synth(3, 2, 3000, "bf16", 0.6, seed=11, f=2)
    e = sv.verify(to_dev(w.target[:0], "bf16"), to_dev(w.draft[:0], "bf16"),
                  torch.zeros(0, 2, dtype=torch.int32, device="cuda"),
                  torch.zeros(0, dtype=torch.float32, device="cuda"),
                  torch.zeros(0, 2, dtype=torch.float32, device="cuda"),
                  torch.zeros(0, 3, dtype=torch.float32, device="cuda"), f=2)
    torch.cuda.synchronize()
    assert e["accept_len"].numel() == 0
    # a draft batch that lives inside a larger buffer, every other sequence
    big = np.zeros((6, 3, 3000), dtype=np.uint16)
    big[::2] = w.draft
    Dv = to_dev(big, "bf16")[::2]
    Tv = to_dev(w.target, "bf16")
    out = sv.verify(Tv, Dv, torch.from_numpy(w.draft_tokens).cuda(),
                    torch.from_numpy(w.temperature).cuda(), torch.from_numpy(w.u_accept).cuda(),
                    torch.from_numpy(w.u_recover).cuda(), f=2, want_p=True, want_q=True)
    torch.cuda.synchronize()
    ref = oracle.verify_batch(w.target, w.draft, "bf16", w.draft_tokens, w.temperature,
                              w.u_accept, w.u_recover, f=2)
    compare_verify(out, ref, np.arange(3), 2, 2)
    log("[edges] empty batch, strided inputs: ok")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_residual_sample_every_position(sv, dtype):
    """Draws and residual rows at every position, an out-of-range position
    once, a greedy sequence; then the token-only call (no output rows), which
    must launch nothing that writes distributions."""
    B, k, V = 4, 3, 5000
    w = synth(B, k, V, dtype, 0.9, seed=13)
    tau = w.temperature.copy()
    tau[1] = 0.0
    x = dict(T=padded_dev(w.target, dtype), D=padded_dev(w.draft, dtype))
    d = torch.from_numpy(w.draft_tokens).cuda()
    n_flag = n_cmp = 0
    for pos_v in range(k + 1):
        pos = np.full(B, pos_v, dtype=np.int32)
        pos[3] = k + 1 if pos_v == 0 else pos_v   # out of range once
        out = sv.residual_sample(x["T"], x["D"], d, torch.from_numpy(tau).cuda(),
                                 torch.from_numpy(pos).cuda(),
                                 torch.from_numpy(w.u_recover).cuda(), want_residual=True)
        torch.cuda.synchronize()
        for b in range(B):
            tok, flag, res, err = oracle.sample_at_position(
                w.target[b], w.draft[b], dtype, w.draft_tokens[b], tau[b], pos[b],
                w.u_recover[b], want_residual=True)
            g = int(out["token"][b])
            if err:
                assert g == -1
                assert np.all(np.isnan(out["residual"][b].cpu().numpy()))
                continue
            n_cmp += 1
            n_flag += int(flag)
            if not flag:
                assert g == tok, (pos_v, b, g, tok)
            tol = residual_tolerance(w.target[b], w.draft[b], dtype, float(tau[b]), k)
            assert_residual_close(out["residual"][b].cpu().numpy(), res, tol,
                                  f"residual b={b} pos={pos_v}")
        # without the residual output only the drawn row is read
        out2 = sv.residual_sample(x["T"], x["D"], d, torch.from_numpy(tau).cuda(),
                                  torch.from_numpy(pos).cuda(),
                                  torch.from_numpy(w.u_recover).cuda())
        torch.cuda.synchronize()
        assert torch.equal(out2["token"], out["token"])
    assert_flag_share(n_flag, n_cmp, "residual draws")
    log(f"[edges] residual_sample every position {dtype}: ok")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_softmax_rows(sv, dtype):
    rows, V = 12, 7000
    rng = np.random.default_rng(17)
    x = (rng.standard_normal((rows, V)) * 3).astype(np.float32)
    x[5, :] = -np.inf
    host = f32_to_bf16_bits(np.where(np.isfinite(x), x, 0)) if dtype == "bf16" else x
    if dtype == "bf16":
        host[5, :] = f32_to_bf16_bits(np.array([-np.inf], np.float32))[0]
    tau = np.array([0.7, 0.0, 1.5, -1.0, 0.3, 2.0], dtype=np.float32)  # two rows per temperature
    dev = padded_dev(host[None], dtype)[0]
    got = sv.softmax_temp(dev, torch.from_numpy(tau).cuda(), rows_per_temp=2)
    torch.cuda.synchronize()
    ref = oracle.softmax_rows(host, dtype, np.repeat(tau, 2))
    assert_probs_close(got.cpu().numpy(), ref, f"softmax {dtype}")
    log(f"[edges] softmax rows {dtype}: ok")


@pytest.mark.parametrize("f", [1, 3, 16])
def test_forked_topf_standalone(sv, f):
    B, k, V = 5, 4, 9000
    w = synth(B, k, V, "bf16", 0.8, seed=19 + f)
    tau = w.temperature.copy()
    tau[2] = 0.0
    drafts = w.draft_tokens.copy()
    drafts[4, 0] = V + 5  # error sequence
    toks, probs = sv.forked_topf(to_dev(w.draft, "bf16"), torch.from_numpy(drafts).cuda(),
                                 torch.from_numpy(tau).cuda(), f)
    torch.cuda.synchronize()
    rt, rp = oracle.forked_topf_batch(w.draft, "bf16", drafts, tau, f)
    np.testing.assert_array_equal(toks.cpu().numpy(), rt)
    assert_probs_close(probs.cpu().numpy(), rp, "fork probs")
    log(f"[edges] forked_topf f={f}: ok")


def test_cache_hit_on_drafter_forks(sv):
    """SSD placement: the drafter ranks its forks with sv_forked_topf, the
    verifier decides without forks, and sv_cache_hit looks the outcome up in
    the drafter's forks.  The hits equal the oracle's lookup of its own
    outcome in its own forks on every unflagged sequence, and the fused
    lookup of a verify call with forks."""
    B, k, V, f = 24, 7, 6000, 3
    w = synth(B, k, V, "bf16", 0.8, seed=77)
    tau = w.temperature.copy()
    tau[::5] = 0.0
    D = padded_dev(w.draft, "bf16")
    T = padded_dev(w.target, "bf16")
    d = torch.from_numpy(w.draft_tokens).cuda()
    tt = torch.from_numpy(tau).cuda()
    ua, ur = torch.from_numpy(w.u_accept).cuda(), torch.from_numpy(w.u_recover).cuda()
    toks, _ = sv.forked_topf(D, d, tt, f)
    out = sv.verify(T, D, d, tt, ua, ur)
    hits = sv.cache_hit(toks, out["accept_len"], out["out_token"])
    fused = sv.verify(T, D, d, tt, ua, ur, f=f, want_hits=True)
    torch.cuda.synchronize()
    assert torch.equal(hits, fused["cache_hit"])
    ref = oracle.verify_batch(w.target, w.draft, "bf16", w.draft_tokens, tau, w.u_accept,
                              w.u_recover, f=f)
    ref_hits = oracle.cache_hits_batch(ref.fork_tokens, ref.accept_len, ref.token)
    h = hits.cpu().numpy()
    for b in range(B):
        if not ref.flagged[b]:
            assert h[b] == ref_hits[b], (b, int(h[b]), int(ref_hits[b]))
    log(f"[edges] cache hits on drafter forks: {int((h >= 0).sum())}/{B}")


def test_workspace_reused_across_shapes(sv):
    """One workspace serves calls of different sizes and entry points in
    turn (grown, and zero-filled, only when a call needs more room)."""
    ws = sv.Workspace(torch.device("cuda", 0))
    shapes = [(2, 5, 33, 5, "bf16"), (6, 7, 3000, 3, "bf16"), (1, 2, 17, 0, "f32"),
              (2, 5, 33, 5, "bf16"), (9, 3, 4097, 2, "f32"), (6, 7, 3000, 3, "bf16")]
    for i, (B, k, V, f, dtype) in enumerate(shapes):
        w = synth(B, k, V, dtype, 0.9, seed=4100 + i, f=f)
        T, D = padded_dev(w.target, dtype), padded_dev(w.draft, dtype)
        d = torch.from_numpy(w.draft_tokens).cuda()
        tau = torch.from_numpy(w.temperature).cuda()
        for _ in range(2):
            out = sv.verify(T, D, d, tau, torch.from_numpy(w.u_accept).cuda(),
                            torch.from_numpy(w.u_recover).cuda(), f=f, want_p=True, want_q=True,
                            workspace=ws)
            torch.cuda.synchronize()
            ref = oracle.verify_batch(w.target, w.draft, dtype, w.draft_tokens, w.temperature,
                                      w.u_accept, w.u_recover, f=f)
            compare_verify(out, ref, np.arange(B), f, k)
        if f > 0:
            toks, _ = sv.forked_topf(D, d, tau, f, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(toks, out["fork_tokens"])
    log("[edges] workspace reused across shapes and entry points: ok")


def test_workspace_zeroed_once_serves_every_call(sv):
    """The workspace contract: zero-filled once, then any sequence of calls
    of any entry point and size, with no re-initialisation in between, gives
    the oracle's results (the arrival counters sit at fixed offsets and every
    call returns them to zero)."""
    shapes = [(2, 5, 33, 5, "bf16"), (6, 7, 3000, 3, "bf16"), (1, 2, 17, 0, "f32"),
              (9, 3, 4097, 2, "f32"), (64, 7, 2048, 3, "bf16")]
    need = max(sv.workspace_size(B, k, V, f) for B, k, V, f, _ in shapes)
    need = max(need, sv.workspace_size(40, 0, 4097, 0))
    ws = sv.Workspace(torch.device("cuda", 0))
    buf = ws.get(need)                        # the one zero fill
    for rnd in range(2):
        for i, (B, k, V, f, dtype) in enumerate(shapes):
            w = synth(B, k, V, dtype, 0.9, seed=5100 + i, f=f)
            T, D = padded_dev(w.target, dtype), padded_dev(w.draft, dtype)
            d = torch.from_numpy(w.draft_tokens).cuda()
            tau = torch.from_numpy(w.temperature).cuda()
            out = sv.verify(T, D, d, tau, torch.from_numpy(w.u_accept).cuda(),
                            torch.from_numpy(w.u_recover).cuda(), f=f, want_p=True, want_q=True,
                            want_hits=f > 0, workspace=ws)
            torch.cuda.synchronize()
            ref = oracle.verify_batch(w.target, w.draft, dtype, w.draft_tokens, w.temperature,
                                      w.u_accept, w.u_recover, f=f)
            compare_verify(out, ref, np.arange(B), f, k)
            if f > 0:
                toks, _ = sv.forked_topf(D, d, tau, f, workspace=ws)
                torch.cuda.synchronize()
                assert torch.equal(toks, out["fork_tokens"])
            host_rows = w.target.reshape(-1, V)[:40]
            rows = padded_dev(host_rows[None], dtype)[0]   # aligned rows, [n, V]
            tr = torch.full((rows.shape[0],), 0.8, dtype=torch.float32, device="cuda")
            pr = sv.softmax_temp(rows, tr, workspace=ws)
            torch.cuda.synchronize()
            refp = oracle.softmax_rows(host_rows, dtype, np.full(rows.shape[0], 0.8))
            assert_probs_close(pr.cpu().numpy(), refp, "softmax rows")
            assert ws.buf is buf, "the workspace was reallocated"
    log("[edges] workspace zeroed once serves every call: ok")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sample_temp_rows(sv, dtype):
    """The drafter's draw on logits rows of several vocabularies (ragged
    tails, one and many slabs), temperatures 0 and above, and error rows,
    against the oracle: tokens equal on every row it does not flag."""
    rng = np.random.default_rng(31 if dtype == "bf16" else 32)
    for V in (2, 7, 1000, 4097, 128256):
        w = synth(2, 7, V, dtype, 0.8, seed=900 + V)
        rows = w.draft.reshape(-1, V)              # 16 rows
        R = rows.shape[0]
        tau = np.where(rng.random(R) < 0.25, 0.0, rng.uniform(0.3, 1.5, R)).astype(np.float32)
        u = uniforms(rng, (R,))
        host = rows.copy()
        if V > 2:
            tau[3] = -1.0                          # invalid temperature
            if dtype == "bf16":
                host[5] = f32_to_bf16_bits(np.full(V, -np.inf, dtype=np.float32))
            else:
                host[5] = -np.inf                  # no finite entry
        x = padded_dev(host[None], dtype)[0]
        got = sv.sample_temp(x, torch.from_numpy(tau).cuda(), torch.from_numpy(u).cuda())
        torch.cuda.synchronize()
        ref, flagged = oracle.sample_rows(host, dtype, tau, u)
        assert_flag_share(int(flagged.sum()), R, "sample_temp")
        g = got.cpu().numpy()
        for r in range(R):
            if not flagged[r]:
                assert g[r] == ref[r], (V, r, int(g[r]), int(ref[r]), float(tau[r]))
        log(f"[edges] sample_temp {dtype} V={V}: {int((~flagged).sum())}/{R} rows compared")
