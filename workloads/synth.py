"""Seeded synthetic inputs for the verify-and-speculate step.

This module only *draws inputs*: logits, drafted tokens, temperatures and the
uniform random numbers that the verifier consumes.  It holds none of the
verifier's arithmetic (no softmax, no acceptance test, no residual, no
inverse CDF, no top-f); both the CPU oracle and the GPU path read the bytes it
produces.

Workload shapes come from the pages' own benchmark commands: k=6 for the
synchronous speculative decode and k=7, f=3 for the asynchronous (SSD) run
("Async spec decode (SSD) ... k=7, f=3" in the benchmark section of the SSD
README translation, m.111cn.net page, section 基准测试), and the Llama-3 /
Qwen3 model families the SSD project page lists under "Highlighted Details"
(vocabularies of 128256 and 151936 tokens).  The pages run on real datasets
(four of them, "--all"); those are replaced here by seeded synthetic logits.

Draw recipe (fixed; every sequence b has its own stream so that any subset of
sequences can be regenerated bit-identically):

* stream of sequence b: ``PCG64(SeedSequence([seed, b]))``.
* "zipf" profile: ``perm = permutation(V)``; ``lr = -1.1*log(perm+1)``;
  ``sigma_b`` (fixed, or ``uniform(lo, hi)``); then for j = 0..k:
  ``base = lr + 0.3*N(0,1)`` (float32 draws), ``T[b,j] = base``,
  ``D[b,j] = base + sigma_b*N(0,1)``; both rounded to the storage dtype
  (bf16: round-to-nearest-even of the float32 value).
* "tiny" profile: for j = 0..k: ``x = 2*N(0,1)`` (float64 draws),
  five distinct "hot" ids ``choice(V, 5, replace=False)`` get ``+6``,
  ``T[b,j] = x``, ``D[b,j] = x + 0.5*N(0,1)``; stored as float32.
* temperatures: fixed per workload, or (mixed) a batch stream
  ``PCG64(SeedSequence([seed, 2**31-1]))`` picks ``B//4`` sequences at 0 and
  draws the others from ``uniform(lo, hi)``.
* drafted tokens: the drafter's own choice, emulated with the Gumbel-max
  device on the *stored* draft logits: stream ``SeedSequence([seed, b, 1])``,
  ``d = argmax_t (D[b,j,t]/tau_b - log E_t)`` with ``E_t ~ Exp(1)``, which
  draws ``d`` from softmax(D[b,j]/tau_b); at tau_b = 0 the drafter is greedy,
  ``d = argmax_t D[b,j,t]`` (first maximum).
* uniforms: stream ``SeedSequence([seed, b, 2])``; ``u_accept[b] =
  integers(0, 2**24, k) * 2**-24`` and ``u_recover[b] = integers(0, 2**24,
  k+1) * 2**-24``, exact float32 values in [0, 1 - 2**-24].
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

F32 = "f32"
BF16 = "bf16"

_TAU_STREAM = 2**31 - 1


@dataclasses.dataclass(frozen=True)
class Config:
    """One synthetic workload shape."""

    name: str
    B: int
    k: int
    V: int
    f: int  # fork fan-out; 0 = no forks asked for
    dtype: str  # F32 or BF16
    profile: str  # "zipf" or "tiny"
    seed: int
    tau: Optional[float] = None  # fixed temperature for every sequence
    tau_mixed: Optional[tuple] = None  # (lo, hi): B//4 greedy, rest uniform(lo, hi)
    sigma: Optional[float] = None  # fixed draft noise std
    sigma_range: Optional[tuple] = None  # (lo, hi): per-sequence draft noise std
    residual_out: bool = False  # whether full residual distributions are asked for


CONFIGS = {
    # Tiny fp32 verify: B=1, k=4, V=1000, temperature 1.
    "tiny_verify": Config("tiny_verify", B=1, k=4, V=1000, f=0, dtype=F32,
                          profile="tiny", seed=20261, tau=1.0,
                          residual_out=True),
    # Synchronous speculative decode at the Llama-3 vocabulary, k=6,
    # greedy and stochastic.
    "sync_verify_llama_greedy": Config("sync_verify_llama_greedy", B=1, k=6,
                                       V=128256, f=0, dtype=BF16,
                                       profile="zipf", seed=20262, tau=0.0,
                                       sigma=0.7),
    "sync_verify_llama_t1": Config("sync_verify_llama_t1", B=1, k=6,
                                   V=128256, f=0, dtype=BF16, profile="zipf",
                                   seed=20262, tau=1.0, sigma=0.7),
    # One SSD step at the Llama-3 vocabulary: k=7, f=3, temperature 0.7.
    "ssd_step_llama": Config("ssd_step_llama", B=1, k=7, f=3, V=128256,
                             dtype=BF16, profile="zipf", seed=20263, tau=0.7,
                             sigma=0.7),
    # Batched verify + forked top-3 at the Qwen3 vocabulary (the measured
    # workload): B=64, k=7, f=3, V=151936, bf16, temperature 0.7.
    "batched_verify_fork_qwen": Config("batched_verify_fork_qwen", B=64, k=7,
                                       f=3, V=151936, dtype=BF16,
                                       profile="zipf", seed=20264, tau=0.7,
                                       sigma_range=(0.3, 1.2)),
    # Large-batch fp32 stress with mixed temperatures and full residuals.
    "stress_mixed_tau_fp32": Config("stress_mixed_tau_fp32", B=256, k=7, f=3,
                                    V=151936, dtype=F32, profile="zipf",
                                    seed=20265, tau_mixed=(0.5, 1.2),
                                    sigma_range=(0.3, 1.2),
                                    residual_out=True),
}

# The order the configurations are listed in (smallest first).
CONFIG_ORDER = ["tiny_verify", "sync_verify_llama_greedy",
                "sync_verify_llama_t1", "ssd_step_llama",
                "batched_verify_fork_qwen", "stress_mixed_tau_fp32"]


@dataclasses.dataclass
class Workload:
    """Host arrays of one call.  Logits are ``[B, k+1, V]`` row-major; bf16
    logits are held as their uint16 bit patterns."""

    config: Config
    seqs: np.ndarray  # int64 [B]: which sequences of the full batch these are
    target: np.ndarray  # [B, k+1, V] float32 or uint16 (bf16 bits)
    draft: np.ndarray  # [B, k+1, V] float32 or uint16 (bf16 bits)
    draft_tokens: np.ndarray  # int32 [B, k]
    temperature: np.ndarray  # float32 [B]
    u_accept: np.ndarray  # float32 [B, k]
    u_recover: np.ndarray  # float32 [B, k+1]
    sigma: np.ndarray  # float32 [B] draft noise std (informational)

    @property
    def B(self):
        return int(self.target.shape[0])

    @property
    def k(self):
        return self.config.k

    @property
    def V(self):
        return self.config.V

    @property
    def f(self):
        return self.config.f

    @property
    def dtype(self):
        return self.config.dtype


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns.  Inputs must be finite."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def _bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    # Exact widening of the stored values; used only to emulate the drafter.
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return f32_to_bf16_bits(x32)
    return np.asarray(x32, dtype=np.float32)


def _stored_as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return _bf16_bits_to_f64(a)
    return a.astype(np.float64)


def batch_temperatures(cfg: Config) -> np.ndarray:
    """Per-sequence temperatures of the whole batch (float32 [B])."""
    if cfg.tau is not None:
        return np.full(cfg.B, cfg.tau, dtype=np.float32)
    lo, hi = cfg.tau_mixed
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, _TAU_STREAM])))
    greedy = rng.choice(cfg.B, cfg.B // 4, replace=False)
    tau = rng.uniform(lo, hi, cfg.B).astype(np.float32)
    tau[greedy] = 0.0
    return tau


def _gen_sequence(cfg: Config, b: int, tau_b: float):
    V, k = cfg.V, cfg.k
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, b])))
    T = np.empty((k + 1, V), dtype=np.uint16 if cfg.dtype == BF16 else np.float32)
    D = np.empty_like(T)
    if cfg.profile == "zipf":
        perm = rng.permutation(V)
        lr = (-1.1 * np.log(perm.astype(np.float64) + 1.0)).astype(np.float32)
        if cfg.sigma is not None:
            sigma = float(cfg.sigma)
        else:
            sigma = float(rng.uniform(*cfg.sigma_range))
        s32 = np.float32(sigma)
        for j in range(k + 1):
            base = lr + np.float32(0.3) * rng.standard_normal(V, dtype=np.float32)
            T[j] = _store(base, cfg.dtype)
            D[j] = _store(base + s32 * rng.standard_normal(V, dtype=np.float32), cfg.dtype)
    elif cfg.profile == "tiny":
        sigma = 0.5
        for j in range(k + 1):
            x = 2.0 * rng.standard_normal(V)
            hot = rng.choice(V, 5, replace=False)
            x[hot] += 6.0
            T[j] = x.astype(np.float32)
            D[j] = (x + 0.5 * rng.standard_normal(V)).astype(np.float32)
    else:
        raise ValueError(cfg.profile)

    # Drafted tokens: the drafter samples from its own softmax (Gumbel-max)
    # or, at temperature 0, takes its argmax.
    rng_d = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, b, 1])))
    drafts = np.empty(k, dtype=np.int32)
    for j in range(k):
        dv = _stored_as_f64(D[j], cfg.dtype)
        if tau_b == 0.0:
            drafts[j] = int(np.argmax(dv))
        else:
            e = rng_d.standard_exponential(V)
            drafts[j] = int(np.argmax(dv / float(tau_b) - np.log(e)))

    rng_u = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, b, 2])))
    scale = np.float32(2.0 ** -24)
    u_acc = rng_u.integers(0, 2**24, k).astype(np.float32) * scale
    u_rec = rng_u.integers(0, 2**24, k + 1).astype(np.float32) * scale
    return T, D, drafts, u_acc, u_rec, sigma


def make_workload(cfg, seqs: Optional[Sequence[int]] = None,
                  threads: Optional[int] = None) -> Workload:
    """Draw the inputs of ``cfg`` (a Config or a name in CONFIGS).

    ``seqs`` selects a subset of the batch's sequences; each sequence's bytes
    are identical to those it has in the full batch.
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if seqs is None:
        seqs = np.arange(cfg.B, dtype=np.int64)
    else:
        seqs = np.asarray(seqs, dtype=np.int64)
        if seqs.size and (seqs.min() < 0 or seqs.max() >= cfg.B):
            raise ValueError("sequence index outside the batch")
    tau_all = batch_temperatures(cfg)
    tau = tau_all[seqs]
    Bsel = int(seqs.size)
    store_dt = np.uint16 if cfg.dtype == BF16 else np.float32
    T = np.empty((Bsel, cfg.k + 1, cfg.V), dtype=store_dt)
    D = np.empty_like(T)
    drafts = np.empty((Bsel, cfg.k), dtype=np.int32)
    u_acc = np.empty((Bsel, cfg.k), dtype=np.float32)
    u_rec = np.empty((Bsel, cfg.k + 1), dtype=np.float32)
    sig = np.empty(Bsel, dtype=np.float32)

    def one(i):
        t, d, dr, ua, ur, s = _gen_sequence(cfg, int(seqs[i]), float(tau[i]))
        T[i] = t
        D[i] = d
        drafts[i] = dr
        u_acc[i] = ua
        u_rec[i] = ur
        sig[i] = s

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if Bsel > 1 and threads > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(Bsel)))
    else:
        for i in range(Bsel):
            one(i)
    return Workload(config=cfg, seqs=seqs, target=T, draft=D,
                    draft_tokens=drafts, temperature=tau.astype(np.float32),
                    u_accept=u_acc, u_recover=u_rec, sigma=sig)


def uniforms(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniforms on the 2**-24 grid in [0, 1 - 2**-24], as float32."""
    return rng.integers(0, 2**24, shape).astype(np.float32) * np.float32(2.0 ** -24)
