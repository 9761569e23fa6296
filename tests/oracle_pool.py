"""The oracle's batch drivers spread over worker processes, so that whole
full-size batches can be checked in seconds.  Test infrastructure: imports
only numpy and the oracle (never torch); the workers are spawned, never
forked, so a parent that holds a GPU context is not copied.

Each worker runs the oracle's own driver over a contiguous group of the
requested sequences; the groups' results are concatenated in order, so the
result is the one the single-process driver returns.
"""

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

import oracle

MAX_WORKERS = 16


def workers(n_items):
    try:
        cpus = len(os.sched_getaffinity(0))
    except AttributeError:
        cpus = os.cpu_count() or 1
    return max(1, min(MAX_WORKERS, cpus, n_items))


def _verify_group(args):
    T, D, dtype, drafts, tau, ua, ur, f, want_q, want_residual = args
    return oracle.verify_batch(T, D, dtype, drafts, tau, ua, ur, f=f, want_q=want_q,
                               want_residual=want_residual)


def _merge(parts, seqs, want_residual):
    cat = lambda name: np.concatenate([getattr(p, name) for p in parts])
    return oracle.BatchResult(
        seqs=np.asarray(seqs), accept_len=cat("accept_len"), token=cat("token"),
        p_draft=cat("p_draft"), q_draft=cat("q_draft"), fork_tokens=cat("fork_tokens"),
        fork_probs=cat("fork_probs"),
        residual=cat("residual") if want_residual else None,
        flagged=cat("flagged"), n_flagged_draws=int(sum(p.n_flagged_draws for p in parts)),
        error=cat("error"))


def verify_batch(target, draft, dtype, draft_tokens, temperature, u_accept, u_recover,
                 f=0, want_q=True, want_residual=False, seqs=None):
    """oracle.verify_batch over ``seqs`` (default: every sequence), in
    worker processes."""
    B = np.asarray(target).shape[0]
    seqs = np.arange(B) if seqs is None else np.asarray(seqs)
    nw = workers(len(seqs))
    if nw <= 1 or len(seqs) < 4:
        return oracle.verify_batch(target, draft, dtype, draft_tokens, temperature, u_accept,
                                   u_recover, f=f, want_q=want_q, want_residual=want_residual,
                                   seqs=seqs)
    groups = [g for g in np.array_split(seqs, nw) if len(g)]
    args = [(np.ascontiguousarray(target[g]), np.ascontiguousarray(draft[g]), dtype,
             draft_tokens[g], temperature[g], u_accept[g], u_recover[g], f, want_q,
             want_residual) for g in groups]
    with ProcessPoolExecutor(max_workers=len(groups),
                             mp_context=mp.get_context("spawn")) as ex:
        parts = list(ex.map(_verify_group, args))
    return _merge(parts, seqs, want_residual)
