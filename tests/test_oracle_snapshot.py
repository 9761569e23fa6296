"""The oracle still reproduces its committed snapshot (tests/golden)."""

import json
import os

import numpy as np

from tests.golden.make_golden import CASES, snapshot

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_oracle_matches_snapshot():
    with open(os.path.join(HERE, "oracle_snapshot.json")) as fh:
        ref = json.load(fh)
    for name, cfg in CASES.items():
        got = snapshot(cfg)
        for key in ("accept_len", "token", "fork_tokens", "flagged"):
            assert got[key] == ref[name][key], (name, key)
        for key in ("p_draft", "q_draft", "fork_probs"):
            np.testing.assert_allclose(np.array(got[key], dtype=float),
                                       np.array(ref[name][key], dtype=float),
                                       rtol=1e-12, atol=0, equal_nan=True)
