"""The seeded input generator: determinism, subset consistency, shapes and
the drafted tokens' support (CPU only)."""

import numpy as np

from workloads import CONFIG_ORDER, CONFIGS, Config, make_workload


def test_deterministic_and_subset_consistent():
    cfg = Config("t", B=6, k=3, V=5000, f=2, dtype="bf16", profile="zipf",
                 seed=99, tau=0.7, sigma_range=(0.3, 1.2))
    a = make_workload(cfg)
    b = make_workload(cfg, threads=1)
    for x, y in [(a.target, b.target), (a.draft, b.draft),
                 (a.draft_tokens, b.draft_tokens), (a.u_accept, b.u_accept),
                 (a.u_recover, b.u_recover), (a.temperature, b.temperature)]:
        np.testing.assert_array_equal(x, y)
    s = make_workload(cfg, seqs=[4, 1])
    np.testing.assert_array_equal(s.target, a.target[[4, 1]])
    np.testing.assert_array_equal(s.draft_tokens, a.draft_tokens[[4, 1]])
    np.testing.assert_array_equal(s.u_recover, a.u_recover[[4, 1]])


def test_shapes_and_ranges_small_configs():
    for name in CONFIG_ORDER[:4]:
        cfg = CONFIGS[name]
        w = make_workload(cfg)
        assert w.target.shape == (cfg.B, cfg.k + 1, cfg.V)
        assert w.draft.shape == w.target.shape
        assert w.target.dtype == (np.uint16 if cfg.dtype == "bf16" else np.float32)
        assert w.draft_tokens.shape == (cfg.B, cfg.k)
        assert np.all((w.draft_tokens >= 0) & (w.draft_tokens < cfg.V))
        for u in (w.u_accept, w.u_recover):
            assert u.dtype == np.float32
            assert np.all((u >= 0) & (u < 1))
            assert np.all(u * 2**24 == np.round(u * 2**24))


def test_mixed_temperatures_quarter_greedy():
    cfg = CONFIGS["stress_mixed_tau_fp32"]
    from workloads import batch_temperatures
    t = batch_temperatures(cfg)
    assert (t == 0).sum() == cfg.B // 4
    nz = t[t > 0]
    assert nz.min() >= 0.5 and nz.max() <= 1.2


def test_greedy_drafts_are_draft_argmax():
    cfg = CONFIGS["sync_verify_llama_greedy"]
    w = make_workload(cfg)
    d = (w.draft[0, :cfg.k].astype(np.uint32) << 16).view(np.float32)
    np.testing.assert_array_equal(w.draft_tokens[0], d.argmax(1))
