"""Throughput of the verify-and-speculate step on one MI355X.

One step = one sv_verify call with fused forked top-f over one batch of the
batched Qwen3-vocabulary workload: B=64 sequences, k=7 drafted positions
plus the bonus position, f=3, V=151936, bf16 logits, temperature 0.7
(seeded synthetic Zipf-profile logits; the drafted tokens are drawn from the
draft distribution).  Inputs are resident in HBM before timing; three input
sets rotate so that no step finds its 311 MB of logits in the 256 MB
last-level cache.

Prints one JSON line: rows/s (512 verified (sequence, position) rows per
step), the roofline of the streaming statistics kernel (algorithmic bytes
per launch / its average duration, measured with HIP events on the call's
stream), and the CPU oracle's rows/s on a bounded sample of the same
workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""

import argparse
import ctypes
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("verified (seq×position) rows/s and % of HBM roofline, "
          "V=151936 k=7 f=3 B=64")
WORKLOAD = "batched_verify_fork_qwen"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_stats_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "verification_sampling_amd", "csrc", n)
                  for n in ("specverify.hip", "sv_device.h", "sv_stats.h", "sv_stream.h")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (profiling runs)")
    ap.add_argument("--cpu-seqs", type=int, default=64,
                    help="sequences of the workload the oracle is timed on")
    ap.add_argument("--latency-b1", action="store_true",
                    help="instead of the throughput step: the latency of one sv_verify call "
                         "on each single-sequence workload (B=1), one JSON line each")
    ap.add_argument("--stress", action="store_true",
                    help="instead of the throughput step: the fp32 stress workload (B=256, "
                         "mixed temperatures): the verify step with forks, then the full "
                         "residual distributions at the outcome positions")
    ap.add_argument("--sample", action="store_true",
                    help="instead of the throughput step: the drafter's draw (sv_sample_temp) "
                         "on the 512 draft rows of the batched workload")
    ap.add_argument("--softmax", action="store_true",
                    help="time sv_softmax_temp on the batched workload's 512 target rows "
                         "instead of the verify step")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain device copy of the logits' size (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn two rocprofv3 --pmc counter_collection.csv files "
                         "(FETCH_SIZE, WRITE_SIZE; runs made with --copy-calib) into the "
                         "per-launch HBM traffic of the statistics kernel and write it to "
                         + os.path.relpath(TRAFFIC_FILE, ROOT))
    return ap.parse_args()


class Hip:
    """The few HIP runtime calls needed for event timing."""

    def __init__(self):
        self.L = ctypes.CDLL("libamdhip64.so")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                               ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        if self.L.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def elapsed_ms(self, a, b):
        t = ctypes.c_float()
        if self.L.hipEventElapsedTime(ctypes.byref(t), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(t.value)


def kernel_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def alg_bytes(B, k, V, f, elem):
    """Algorithmic bytes of the step (every input byte read once, every
    output byte written once) and of the statistics kernel (the logits, the
    drafted ids and the temperatures it reads; what it writes are partial
    results, not outputs)."""
    logits = 2 * B * (k + 1) * V * elem          # target + draft, rows 0..k
    small_in = B * k * 4 + B * 4 + B * k * 4 + B * (k + 1) * 4   # d, tau, u_acc, u_rec
    out = B * 4 + B * 4 + 2 * B * (k + 1) * f * 4               # len, token, forks
    stats_kernel = logits + B * k * 4 + B * 4
    return logits + small_in + out, stats_kernel


def counter_means(path, counter):
    """Mean value per dispatch of one counter, by kernel-name prefix, from a
    rocprofv3 counter_collection.csv (one row per dispatch and counter)."""
    import csv
    acc = {}
    with open(path, newline="") as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = ("k_stats" if "sv::k_stats" in name else
                   "k_decide" if "sv::k_decide" in name else
                   "copy" if "neg_kernel_cuda" in name else None)
            if key is None:
                continue
            s_, n_ = acc.get(key, (0.0, 0))
            acc[key] = (s_ + float(r["Counter_Value"]), n_ + 1)
    return {k_: v[0] / v[1] for k_, v in acc.items()}


def write_traffic(fetch_csv, write_csv):
    """HBM bytes per launch of the statistics kernel.  Each counter is scaled
    by what it reads for the plain copy kernel (torch.neg over a float32
    tensor of COPY_BYTES, which reads and writes COPY_BYTES once each)."""
    from workloads import CONFIGS
    cfg = CONFIGS[WORKLOAD]
    copy_bytes = (alg_bytes(cfg.B, cfg.k, cfg.V, cfg.f, 2)[0] // 8) * 4
    fe = counter_means(fetch_csv, "FETCH_SIZE")
    wr = counter_means(write_csv, "WRITE_SIZE")
    f_scale = copy_bytes / (fe["copy"] * 1024.0)
    w_scale = copy_bytes / (wr["copy"] * 1024.0)
    fetch_b = fe["k_stats"] * 1024.0 * f_scale
    write_b = wr["k_stats"] * 1024.0 * w_scale
    out = {"kernel": "k_stats", "kernel_hash": kernel_hash(),
           "bytes_per_launch": fetch_b + write_b,
           "fetch_bytes": fetch_b, "write_bytes": write_b,
           "fetch_kib_raw": fe["k_stats"], "write_kib_raw": wr["k_stats"],
           "fetch_scale": f_scale, "write_scale": w_scale,
           "copy_bytes": copy_bytes}
    if "k_decide" in fe and "k_decide" in wr:
        out["k_decide"] = {"fetch_bytes": fe["k_decide"] * 1024.0 * f_scale,
                           "write_bytes": wr["k_decide"] * 1024.0 * w_scale,
                           "fetch_kib_raw": fe["k_decide"], "write_kib_raw": wr["k_decide"]}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out))


def _oracle_chunk(args):
    """Worker of the multi-process oracle leg (runs in a fresh interpreter):
    the oracle on a list of whole sequences."""
    import oracle
    T, D, dtype, d, tau, ua, ur, f = args
    r = oracle.verify_batch(T, D, dtype, d, tau, ua, ur, f=f)
    return r.accept_len, r.token, r.fork_tokens


def cpu_model():
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    return "unknown"


def cpu_baseline(w, nseq):
    """The oracle timed on the first nseq sequences, on the host's cores.

    Leg 1: one process (its result also serves the parity check).  Leg 2:
    N = len(os.sched_getaffinity(0)) worker processes (fresh interpreters,
    no GPU state), each taking a contiguous share of the sequences; the
    workers' start-up is included.  The reported value is leg 2; cores is
    the number of workers it actually used."""
    import oracle
    from concurrent.futures import ProcessPoolExecutor
    import multiprocessing as mp

    seqs = list(range(min(nseq, w.B)))
    t0 = time.perf_counter()
    ref = oracle.verify_batch(w.target, w.draft, w.dtype, w.draft_tokens, w.temperature,
                              w.u_accept, w.u_recover, f=w.f, seqs=seqs)
    dt1 = time.perf_counter() - t0
    rows = len(seqs) * (w.k + 1)

    ncpu = len(os.sched_getaffinity(0))
    nw = max(1, min(ncpu, len(seqs)))
    parts = [seqs[i * len(seqs) // nw:(i + 1) * len(seqs) // nw] for i in range(nw)]
    jobs = [(w.target[p], w.draft[p], w.dtype, w.draft_tokens[p], w.temperature[p],
             w.u_accept[p], w.u_recover[p], w.f) for p in parts if p]
    t0 = time.perf_counter()
    with ProcessPoolExecutor(max_workers=len(jobs), mp_context=mp.get_context("spawn")) as ex:
        res = list(ex.map(_oracle_chunk, jobs))
    dtn = time.perf_counter() - t0
    import numpy as np
    same = (np.array_equal(np.concatenate([r[0] for r in res]), ref.accept_len)
            and np.array_equal(np.concatenate([r[1] for r in res]), ref.token))
    return {"value": rows / dtn, "unit": "rows/s", "cores": len(jobs), "kind": "oracle",
            "cpu_model": cpu_model(), "affinity_cpus": ncpu,
            "sample": f"{len(seqs)} of {w.B} sequences of {WORKLOAD} ({rows} rows): "
                      f"{len(jobs)} worker processes, {dtn:.1f} s including their start-up",
            "one_process": {"value": rows / dt1, "cores": 1, "seconds": dt1},
            "legs_agree": bool(same)}, ref


def parity(out, ref):
    """The timed calls' outputs (input set 0, the workload in its own order)
    against the oracle on the same sequences: token ids, accepted lengths and
    fork tokens bit-exact on every sequence the oracle does not flag (a
    uniform within 1e-6 of a decision boundary), fork probabilities within
    1e-5 relative."""
    import numpy as np

    seqs = np.asarray(ref.seqs)
    al = out["accept_len"].cpu().numpy()[seqs]
    tok = out["out_token"].cpu().numpy()[seqs]
    ft = out["fork_tokens"].cpu().numpy()[seqs]
    fp = out["fork_probs"].cpu().numpy()[seqs].astype(np.float64)
    bad = 0
    for i in range(len(seqs)):
        if ref.flagged[i]:
            continue
        if al[i] != ref.accept_len[i] or tok[i] != ref.token[i]:
            bad += 1
    fork_bad = int(np.sum(np.any(ft != ref.fork_tokens, axis=(1, 2))))
    prob_bad = int(np.sum(np.abs(fp - ref.fork_probs) > 1e-5 * np.abs(ref.fork_probs) + 1e-30))
    return {"sequences": int(len(seqs)), "flagged_sequences": int(np.sum(ref.flagged)),
            "flagged_draws": int(ref.n_flagged_draws), "token_or_length_mismatches": bad,
            "fork_token_mismatches": fork_bad, "fork_probs_outside_1e-5": prob_bad}


def latency_b1(steps, warmup):
    """Microseconds per sv_verify call at B = 1, calls issued back to back
    (device time per call) on the single-sequence workloads."""
    import numpy as np
    import torch

    from verification_sampling_amd import specverify as sv
    from workloads import CONFIGS, make_workload

    dev = torch.device("cuda", 0)
    for name in ("tiny_verify", "sync_verify_llama_greedy", "sync_verify_llama_t1",
                 "ssd_step_llama"):
        cfg = CONFIGS[name]
        w = make_workload(cfg)

        def logits(a_):
            if cfg.dtype == "bf16":
                return torch.from_numpy(np.ascontiguousarray(a_).view(np.int16)).view(
                    torch.bfloat16).to(dev)
            return torch.from_numpy(a_).to(dev)

        x = [logits(w.target), logits(w.draft)] + [
            torch.from_numpy(v).to(dev)
            for v in (w.draft_tokens, w.temperature, w.u_accept, w.u_recover)]
        B, k, f = cfg.B, cfg.k, cfg.f
        out = {"accept_len": torch.empty(B, dtype=torch.int32, device=dev),
               "out_token": torch.empty(B, dtype=torch.int32, device=dev)}
        if f:
            out["fork_tokens"] = torch.empty(B, k + 1, f, dtype=torch.int32, device=dev)
            out["fork_probs"] = torch.empty(B, k + 1, f, dtype=torch.float32, device=dev)
        call = sv.PreparedVerify(*x, f, out, sv.Workspace(dev))
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        print(json.dumps({"workload": name, "B": B, "k": k, "f": f, "V": cfg.V,
                          "logits": cfg.dtype, "us_per_call": e0.elapsed_time(e1) * 1e3 / steps}),
              flush=True)


def stress(steps, warmup):
    """Throughput on the B=256 fp32 stress workload: sv_verify with forks
    (rows/s, algorithmic GB/s of the logits), then sv_residual_sample with
    the full residual distributions at the outcome positions (every row read
    for the statistics, re-read for the residual sums and again for the
    normalised write)."""
    import torch

    from verification_sampling_amd import specverify as sv
    from workloads import CONFIGS, make_workload

    cfg = CONFIGS["stress_mixed_tau_fp32"]
    w = make_workload(cfg)
    dev = torch.device("cuda", 0)
    T, D, d, tau, ua, ur = (torch.from_numpy(v).to(dev) for v in (
        w.target, w.draft, w.draft_tokens, w.temperature, w.u_accept, w.u_recover))
    B, k, f, V = cfg.B, cfg.k, cfg.f, cfg.V
    out = {"accept_len": torch.empty(B, dtype=torch.int32, device=dev),
           "out_token": torch.empty(B, dtype=torch.int32, device=dev),
           "fork_tokens": torch.empty(B, k + 1, f, dtype=torch.int32, device=dev),
           "fork_probs": torch.empty(B, k + 1, f, dtype=torch.float32, device=dev)}
    call = sv.PreparedVerify(T, D, d, tau, ua, ur, f, out, sv.Workspace(dev))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, n):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / n

    rows = B * (k + 1)
    logits = 2 * rows * V * 4
    t = timed(call, steps)
    print(json.dumps({"workload": "stress_mixed_tau_fp32", "call": "sv_verify (f=3)",
                      "us_per_call": t * 1e6, "rows_per_s": rows / t,
                      "logits_GBs": logits / t / 1e9}), flush=True)
    pos = out["accept_len"].clone()
    ws = sv.Workspace(dev)
    t2 = timed(lambda: sv.residual_sample(T, D, d, tau, pos, ur, want_residual=True,
                                          workspace=ws), max(1, steps // 4))
    alg = logits + rows * V * 4
    print(json.dumps({"workload": "stress_mixed_tau_fp32",
                      "call": "sv_residual_sample (full distributions)",
                      "us_per_call": t2 * 1e6, "alg_bytes": alg, "alg_GBs": alg / t2 / 1e9,
                      "moved_bytes": 3 * logits + rows * V * 4,
                      "moved_GBs": (3 * logits + rows * V * 4) / t2 / 1e9}), flush=True)


def softmax_bench(steps, warmup):
    """sv_softmax_temp on the 512 target rows of the batched Qwen3-vocabulary
    workload (the workload's temperatures, one per sequence), into a
    preallocated float32 output: rows/s and algorithmic GB/s (each logit read
    once, each probability written once)."""
    import numpy as np
    import torch

    from verification_sampling_amd import specverify as sv
    from workloads import CONFIGS, make_workload

    cfg = CONFIGS[WORKLOAD]
    w = make_workload(cfg)
    dev = torch.device("cuda", 0)
    B, k, V = cfg.B, cfg.k, cfg.V
    rows = B * (k + 1)
    x = torch.from_numpy(np.ascontiguousarray(w.target).view(np.int16)).view(
        torch.bfloat16).reshape(rows, V).to(dev)
    tau = torch.from_numpy(w.temperature).to(dev)
    out = torch.empty(rows, V, dtype=torch.float32, device=dev)
    ws = sv.Workspace(dev)
    for _ in range(warmup):
        sv.softmax_temp(x, tau, rows_per_temp=k + 1, workspace=ws, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        sv.softmax_temp(x, tau, rows_per_temp=k + 1, workspace=ws, out=out)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / steps
    alg = rows * V * (2 + 4)
    print(json.dumps({"workload": WORKLOAD + " target rows", "call": "sv_softmax_temp",
                      "rows": rows, "us_per_call": t * 1e6, "rows_per_s": rows / t,
                      "alg_bytes": alg, "alg_GBs": alg / t / 1e9,
                      "frac_of_hbm_peak": alg / t / 8e12,
                      "bytes_moved": rows * V * (2 + 2 + 4),
                      "note": "two launches: row statistics (reads the logits), then the "
                              "normalised rows (reads them again, writes fp32)"}), flush=True)


def sample_rows(steps, warmup):
    """sv_sample_temp on the 512 draft rows of the batched Qwen3-vocabulary
    workload (one uniform per row, the workload's temperatures): rows/s and
    algorithmic GB/s (each row read once)."""
    import numpy as np
    import torch

    from verification_sampling_amd import specverify as sv
    from workloads import CONFIGS, make_workload

    cfg = CONFIGS[WORKLOAD]
    w = make_workload(cfg)
    dev = torch.device("cuda", 0)
    B, k, V = cfg.B, cfg.k, cfg.V
    rows = B * (k + 1)
    x = torch.from_numpy(np.ascontiguousarray(w.draft).view(np.int16)).view(
        torch.bfloat16).reshape(rows, V).to(dev)
    tau = torch.from_numpy(w.temperature).to(dev)
    u = torch.from_numpy(np.ascontiguousarray(w.u_recover.reshape(-1))).to(dev)
    for _ in range(warmup):
        sv.sample_temp(x, tau, u, rows_per_temp=k + 1)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        sv.sample_temp(x, tau, u, rows_per_temp=k + 1)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / steps
    print(json.dumps({"workload": WORKLOAD + " draft rows", "call": "sv_sample_temp",
                      "rows": rows, "us_per_call": t * 1e6, "rows_per_s": rows / t,
                      "alg_GBs": rows * V * 2 / t / 1e9}), flush=True)


def main():
    a = parse()
    if a.sample:
        sample_rows(a.steps, a.warmup)
        return
    if a.softmax:
        softmax_bench(a.steps, a.warmup)
        return
    if a.stress:
        stress(a.steps, a.warmup)
        return
    if a.latency_b1:
        latency_b1(a.steps, a.warmup)
        return
    if a.traffic_from:
        write_traffic(*a.traffic_from)
        return
    if a.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; "
                                   "--gpus must be 1 (the step has no multi-GPU path)"}))
        sys.exit(2)

    import numpy as np
    import torch

    from verification_sampling_amd import specverify as sv
    from workloads import CONFIGS, make_workload

    cfg = CONFIGS[WORKLOAD]
    w = make_workload(cfg)
    B, k, V, f = cfg.B, cfg.k, cfg.V, cfg.f
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def bf16(a_):
        return torch.from_numpy(np.ascontiguousarray(a_).view(np.int16)).view(torch.bfloat16)

    base = dict(T=bf16(w.target).to(dev), D=bf16(w.draft).to(dev),
                d=torch.from_numpy(w.draft_tokens).to(dev),
                tau=torch.from_numpy(w.temperature).to(dev),
                ua=torch.from_numpy(w.u_accept).to(dev),
                ur=torch.from_numpy(w.u_recover).to(dev))
    # three input sets (the batch rolled by 0, 21 and 42 sequences)
    sets = []
    for r in (0, 21, 42):
        sets.append({key: torch.roll(v, r, 0).contiguous() for key, v in base.items()})
    del base
    ws = sv.Workspace(dev)
    calls, outs = [], []
    for s in sets:
        out = {"accept_len": torch.empty(B, dtype=torch.int32, device=dev),
               "out_token": torch.empty(B, dtype=torch.int32, device=dev),
               "fork_tokens": torch.empty(B, k + 1, f, dtype=torch.int32, device=dev),
               "fork_probs": torch.empty(B, k + 1, f, dtype=torch.float32, device=dev)}
        calls.append(sv.PreparedVerify(s["T"], s["D"], s["d"], s["tau"], s["ua"], s["ur"],
                                       f, out, ws))
        outs.append(out)
    torch.cuda.synchronize()

    hip = Hip()
    for i in range(a.warmup):
        calls[i % 3]()
    torch.cuda.synchronize()

    # the timed steps: nothing but the calls between the two events
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(a.steps):
        calls[i % 3]()
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)

    # per-step times: the same calls with an event between consecutive steps
    pev = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    torch.cuda.synchronize()
    pev[0].record()
    for i in range(a.steps):
        calls[i % 3]()
        pev[i + 1].record()
    torch.cuda.synchronize()
    step_us = np.array([pev[i].elapsed_time(pev[i + 1]) * 1e3 for i in range(a.steps)])

    # the statistics kernel alone, from events the library records around it
    # on the call's stream (a further pass of as many steps)
    ev = [(hip.event(), hip.event()) for _ in range(a.steps)]
    opts = [sv.SvOpts(e0.value, e1.value) for e0, e1 in ev]
    torch.cuda.synchronize()
    for i in range(a.steps):
        calls[i % 3](opts[i])
    torch.cuda.synchronize()
    stats_ms = [hip.elapsed_ms(e0, e1) for e0, e1 in ev]

    ms_per_step = total_ms / a.steps
    rows = B * (k + 1)
    total_bytes, stats_bytes = alg_bytes(B, k, V, f, 2)
    stats_avg_s = float(np.mean(stats_ms)) * 1e-3
    achieved = stats_bytes / stats_avg_s / 1e9

    traffic = None
    decide_traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            tr = json.load(fh)
        if tr.get("kernel_hash") == kernel_hash():
            traffic = tr.get("bytes_per_launch")
            if "k_decide" in tr:
                decide_traffic = tr["k_decide"]["fetch_bytes"] + tr["k_decide"]["write_bytes"]

    if a.copy_calib:
        # counter calibration: a plain copy kernel of known size (reads and
        # writes total_bytes // 2 bytes once each)
        x = torch.empty(total_bytes // 8, dtype=torch.float32, device=dev).normal_()
        y = torch.empty_like(x)
        for _ in range(3):
            torch.neg(x, out=y)
        torch.cuda.synchronize()
        del x, y

    # what this GPU reaches on plain HBM traffic of the logits' size: a
    # device-to-device copy (reads and writes every byte), three buffer sets
    # rotated like the step
    nbytes = stats_bytes // 16 * 16
    srcs = [torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1) for _ in range(3)]
    dsts = [torch.empty_like(srcs[0]) for _ in range(3)]
    for i in range(3):
        dsts[i].copy_(srcs[i])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(30):
        dsts[i % 3].copy_(srcs[i % 3])
    e1.record()
    torch.cuda.synchronize()
    copy_s = e0.elapsed_time(e1) * 1e-3 / 30
    del srcs, dsts
    copy_gbs = 2 * nbytes / copy_s / 1e9

    res = {
        "metric": METRIC,
        "value": rows / (ms_per_step * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "B": B, "k": k, "f": f, "V": V,
                   "logits": "bf16", "temperature": 0.7, "rows_per_step": rows,
                   "input_sets": 3},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "k_stats", "alg_bytes_per_launch": stats_bytes,
                     "avg_launch_us": stats_avg_s * 1e6},
        "step": {"alg_bytes": total_bytes,
                 "alg_GBs": total_bytes / (ms_per_step * 1e-3) / 1e9,
                 "frac_of_hbm_peak": total_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                 "frac_of_measured_copy": total_bytes / (ms_per_step * 1e-3) / 1e9 / copy_gbs,
                 "us_median": float(np.median(step_us)),
                 "us_p10": float(np.percentile(step_us, 10)),
                 "us_p90": float(np.percentile(step_us, 90)),
                 "steps_with_events": int(a.steps),
                 "decide_traffic_bytes": decide_traffic,
                 "decide_draw_rows_bytes": B * 2 * V * 2},
        "measured_peak": {"d2d_copy_GBs": copy_gbs, "bytes": int(nbytes),
                          "how": "device-to-device copy of a buffer of the step's logits "
                                 "size (bytes read + bytes written per second), three sets "
                                 "rotated"},
    }
    if not a.no_cpu_baseline:
        res["cpu_baseline"], ref = cpu_baseline(w, a.cpu_seqs)
        res["parity"] = parity(outs[0], ref)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
