"""GPU checks of the call paths around the verify step (through the C ABI):
repeated calls are bitwise identical for verify, the full residual
distributions and softmax rows; the prepared call and the call with timing
events give the plain call's outputs."""

import numpy as np
import pytest
import torch

from tests.gpu_helpers import dev_inputs, log
from workloads import CONFIGS, Config, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from verification_sampling_amd import specverify
    specverify.lib()
    return specverify


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def _same(a, b, what):
    assert set(a) == set(b), what
    for key in a:
        assert torch.equal(_bits(a[key]), _bits(b[key])), (what, key)


def test_repeated_calls_are_bitwise_identical(sv):
    cfg = CONFIGS["stress_mixed_tau_fp32"]
    log(f"[calls] repeat: B={cfg.B} k={cfg.k} V={cfg.V} f={cfg.f} {cfg.dtype}")
    w = make_workload(cfg)
    x = dev_inputs(w)
    outs = []
    for _ in range(2):
        outs.append(sv.verify(x["T"], x["D"], x["d"], x["tau"], x["ua"], x["ur"], f=cfg.f,
                              want_p=True, want_q=True, want_hits=True))
    torch.cuda.synchronize()
    _same(outs[0], outs[1], "verify")
    pos = outs[0]["accept_len"].clone()
    res = [sv.residual_sample(x["T"], x["D"], x["d"], x["tau"], pos, x["ur"], want_residual=True)
           for _ in range(2)]
    torch.cuda.synchronize()
    _same(res[0], res[1], "residual_sample")
    assert torch.equal(res[0]["token"], outs[0]["out_token"])
    rows = x["T"][:32].reshape(-1, cfg.V)
    sm = [sv.softmax_temp(rows, x["tau"][:32].contiguous(), rows_per_temp=cfg.k + 1)
          for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(_bits(sm[0]), _bits(sm[1]))
    log("[calls] repeated calls identical")


def test_prepared_and_timed_calls_match_the_plain_call(sv):
    w = make_workload(Config("calls", B=6, k=5, V=20000, f=3, dtype="bf16", profile="zipf",
                             seed=8080, tau_mixed=(0.5, 1.2), sigma_range=(0.3, 1.2)))
    x = dev_inputs(w)
    B, k, f = w.B, w.k, 3
    ref = sv.verify(x["T"], x["D"], x["d"], x["tau"], x["ua"], x["ur"], f=f)
    out = {"accept_len": torch.full((B,), -9, dtype=torch.int32, device="cuda"),
           "out_token": torch.full((B,), -9, dtype=torch.int32, device="cuda"),
           "fork_tokens": torch.full((B, k + 1, f), -9, dtype=torch.int32, device="cuda"),
           "fork_probs": torch.full((B, k + 1, f), 9.0, dtype=torch.float32, device="cuda")}
    call = sv.PreparedVerify(x["T"], x["D"], x["d"], x["tau"], x["ua"], x["ur"], f, out,
                             sv.Workspace(torch.device("cuda", 0)))
    call()
    torch.cuda.synchronize()
    _same({k_: out[k_] for k_ in ref}, ref, "prepared")
    # the same call with the library's timing events around the statistics kernel
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    ev = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in ev:
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
    for t in out.values():
        t.fill_(-9)
    call(sv.SvOpts(ev[0].value, ev[1].value))
    torch.cuda.synchronize()
    _same({k_: out[k_] for k_ in ref}, ref, "timed")
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
    assert 0.0 < ms.value < 1000.0
    log(f"[calls] prepared and timed calls match; statistics kernel {ms.value * 1e3:.1f} us")
