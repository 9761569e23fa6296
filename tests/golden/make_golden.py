"""Writes oracle_snapshot.json: the CPU oracle's outputs on two small seeded
workloads.  Calls only the oracle and the input generator.

The pages print no worked example of the verify step, so nothing here comes
from them; this snapshot guards the oracle against unintended changes (any
change to it must name the passage or reading that justifies it).

    python tests/golden/make_golden.py
"""

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from workloads import CONFIGS, Config, make_workload  # noqa: E402

CASES = {
    "tiny_verify": CONFIGS["tiny_verify"],
    "small_zipf_bf16": Config("small_zipf_bf16", B=4, k=3, V=3000, f=2,
                              dtype="bf16", profile="zipf", seed=424242,
                              tau=0.8, sigma_range=(0.3, 1.2)),
}


def snapshot(cfg):
    w = make_workload(cfg)
    r = oracle.verify_batch(w.target, w.draft, cfg.dtype, w.draft_tokens,
                            w.temperature, w.u_accept, w.u_recover, f=cfg.f)
    return {
        "accept_len": r.accept_len.tolist(),
        "token": r.token.tolist(),
        "p_draft": r.p_draft.tolist(),
        "q_draft": r.q_draft.tolist(),
        "fork_tokens": r.fork_tokens.tolist(),
        "fork_probs": r.fork_probs.tolist(),
        "flagged": r.flagged.tolist(),
    }


def main():
    out = {name: snapshot(cfg) for name, cfg in CASES.items()}
    with open(os.path.join(HERE, "oracle_snapshot.json"), "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")


if __name__ == "__main__":
    main()
