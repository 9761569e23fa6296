"""The worker-process driver of the oracle returns exactly what the
single-process driver returns."""

import numpy as np

import oracle
from tests import oracle_pool
from workloads import Config, make_workload


def test_pool_matches_single_process():
    w = make_workload(Config("pool", B=9, k=3, V=700, f=2, dtype="bf16", profile="zipf",
                             seed=55, tau_mixed=(0.5, 1.2), sigma_range=(0.3, 1.2)))
    args = (w.target, w.draft, "bf16", w.draft_tokens, w.temperature, w.u_accept, w.u_recover)
    seqs = np.array([0, 2, 3, 5, 6, 8])
    one = oracle.verify_batch(*args, f=2, want_residual=True, seqs=seqs)
    many = oracle_pool.verify_batch(*args, f=2, want_residual=True, seqs=seqs)
    for name in ("seqs", "accept_len", "token", "fork_tokens", "flagged", "error"):
        np.testing.assert_array_equal(getattr(many, name), getattr(one, name), err_msg=name)
    for name in ("p_draft", "q_draft", "fork_probs", "residual"):
        np.testing.assert_array_equal(getattr(many, name), getattr(one, name), err_msg=name)
    assert many.n_flagged_draws == one.n_flagged_draws
