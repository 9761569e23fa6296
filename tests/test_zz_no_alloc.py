"""sv_verify_noalloc (the call for callers that cannot allocate) against
sv_verify: two calls in a row, the second on a smaller batch of another
dtype and fan-out, every output bitwise equal to sv_verify's on the same
inputs."""

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


def _outputs(B, k, f, like):
    """Output tensors pre-filled with values no call writes, so that an
    output the call leaves unwritten cannot match."""
    dev = like.device
    out = {
        "accept_len": torch.full((B,), -77, dtype=torch.int32, device=dev),
        "out_token": torch.full((B,), -77, dtype=torch.int32, device=dev),
        "p_draft": torch.full((B, k), 7.0, dtype=torch.float32, device=dev),
        "q_draft": torch.full((B, k), 7.0, dtype=torch.float32, device=dev),
    }
    if f > 0:
        out["fork_tokens"] = torch.full((B, k + 1, f), -77, dtype=torch.int32, device=dev)
        out["fork_probs"] = torch.full((B, k + 1, f), 7.0, dtype=torch.float32, device=dev)
        out["cache_hit"] = torch.full((B,), -77, dtype=torch.int32, device=dev)
    return out


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def _case(sv, w, f):
    x = dev_inputs(w)
    B, k = w.B, w.k
    ref = sv.verify(x["T"], x["D"], x["d"], x["tau"], x["ua"], x["ur"], f=f,
                    want_p=True, want_q=True, want_hits=f > 0)
    out = _outputs(B, k, f, x["T"])
    got = sv.verify_noalloc(x["T"], x["D"], x["d"], x["tau"], x["ua"], x["ur"], out, f=f)
    torch.cuda.synchronize()
    assert got is out
    assert set(out) == set(ref)
    for key in ref:
        assert torch.equal(_bits(out[key]), _bits(ref[key])), key
    return out


def test_noalloc_matches_verify_on_two_calls(sv):
    cfg = CONFIGS["batched_verify_fork_qwen"]
    log(f"[noalloc] call 1: B={cfg.B} k={cfg.k} V={cfg.V} f={cfg.f} {cfg.dtype}")
    assert sv.workspace_size(cfg.B, cfg.k, cfg.V, cfg.f) <= sv.NOALLOC_SCRATCH_BYTES
    big = _case(sv, make_workload(cfg), cfg.f)
    assert (big["accept_len"] >= 0).all()
    small = make_workload(Config("noalloc_small", B=5, k=3, V=5000, f=2, dtype="f32",
                                 profile="zipf", seed=4242, tau_mixed=(0.5, 1.2),
                                 sigma_range=(0.3, 1.2)))
    small.temperature[1] = 0.0
    log("[noalloc] call 2: B=5 k=3 V=5000 f=2 f32")
    _case(sv, small, 2)
    log("[noalloc] two calls in a row match sv_verify bitwise")


def test_noalloc_refuses_a_shape_beyond_its_scratch(sv):
    B, k, V, f = 256, 7, 151936, 3
    assert sv.workspace_size(B, k, V, f) > sv.NOALLOC_SCRATCH_BYTES
    T = torch.zeros(B, k + 1, V, dtype=torch.bfloat16, device="cuda")
    d = torch.zeros(B, k, dtype=torch.int32, device="cuda")
    tau = torch.ones(B, dtype=torch.float32, device="cuda")
    ua = torch.zeros(B, k, dtype=torch.float32, device="cuda")
    ur = torch.zeros(B, k + 1, dtype=torch.float32, device="cuda")
    out = _outputs(B, k, f, T)
    with pytest.raises(sv.SpecVerifyError, match="scratch"):
        sv.verify_noalloc(T, T, d, tau, ua, ur, out, f=f)
    torch.cuda.synchronize()
    assert (out["accept_len"] == -77).all()
