"""The Python binding rejects every mismatched shape, count, dtype or device
with ValueError before it touches the library (CPU only: the library entry
is replaced by a function that fails the test if it is reached)."""

import pytest
import torch

from verification_sampling_amd import specverify as sv


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def forbidden():
        raise AssertionError("the library was called before the arguments were checked")
    monkeypatch.setattr(sv, "lib", forbidden)


B, K, V, F = 3, 4, 1000, 3


def good(dtype=torch.bfloat16):
    return dict(
        target=torch.zeros(B, K + 1, V, dtype=dtype),
        draft=torch.zeros(B, K + 1, V, dtype=dtype),
        draft_tokens=torch.zeros(B, K, dtype=torch.int32),
        temperature=torch.ones(B, dtype=torch.float32),
        u_accept=torch.zeros(B, K, dtype=torch.float32),
        u_recover=torch.zeros(B, K + 1, dtype=torch.float32))


def call_verify(a, **kw):
    return sv.verify(a["target"], a["draft"], a["draft_tokens"], a["temperature"],
                     a["u_accept"], a["u_recover"], **kw)


def test_consistent_cpu_arguments_fail_only_on_the_device():
    with pytest.raises(ValueError, match="ROCm device"):
        call_verify(good(), f=F)


@pytest.mark.parametrize("key,bad", [
    ("target", torch.zeros(B, K + 1, V, dtype=torch.float16)),       # dtype
    ("draft", torch.zeros(B, K + 1, V, dtype=torch.float32)),        # dtype differs from target
    ("draft", torch.zeros(B + 1, K + 1, V, dtype=torch.bfloat16)),   # B
    ("draft", torch.zeros(B, K + 1, V + 8, dtype=torch.bfloat16)),   # V
    ("draft", torch.zeros(B, K + 2, V, dtype=torch.bfloat16)),       # k
    ("draft", torch.zeros(B, K + 1, 2 * V, dtype=torch.bfloat16)[:, :, ::2]),  # V not contiguous
    ("draft_tokens", torch.zeros(B, K + 1, dtype=torch.int32)),      # k + 1 drafted tokens
    ("draft_tokens", torch.zeros(B - 1, K, dtype=torch.int32)),      # B - 1 sequences
    ("draft_tokens", torch.zeros(B, K, dtype=torch.int64)),          # dtype
    ("draft_tokens", torch.zeros(K, B, dtype=torch.int32).t()),      # not contiguous
    ("temperature", torch.ones(B - 1, dtype=torch.float32)),         # too few
    ("temperature", torch.ones(B + 1, dtype=torch.float32)),         # too many
    ("temperature", torch.ones(B, dtype=torch.float64)),             # dtype
    ("u_accept", torch.zeros(B, K + 1, dtype=torch.float32)),
    ("u_recover", torch.zeros(B, K, dtype=torch.float32)),
    ("target", torch.zeros(B, K + 1, dtype=torch.bfloat16)),         # 2-D
])
def test_verify_rejects_mismatch(key, bad):
    a = good()
    a[key] = bad
    with pytest.raises((ValueError, TypeError)) as e:
        call_verify(a, f=F)
    assert "ROCm device" not in str(e.value)


def test_draft_without_bonus_row_only_without_forks():
    a = good()
    a["draft"] = torch.zeros(B, K, V, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="draft logits"):
        call_verify(a, f=F)
    with pytest.raises(ValueError, match="ROCm device"):
        call_verify(a, f=0)


@pytest.mark.parametrize("f", [-1, 17, V])
def test_verify_rejects_fan_out(f):
    with pytest.raises(ValueError):
        call_verify(good(), f=f)


def test_verify_rejects_mismatched_out():
    a = good()
    out = {"accept_len": torch.zeros(B, dtype=torch.int32),
           "out_token": torch.zeros(B + 1, dtype=torch.int32)}
    with pytest.raises(ValueError, match="out_token"):
        call_verify(a, out=out)
    out["out_token"] = torch.zeros(B, dtype=torch.int32)
    out["fork_tokens"] = torch.zeros(B, K, F, dtype=torch.int32)
    out["fork_probs"] = torch.zeros(B, K + 1, F, dtype=torch.float32)
    with pytest.raises(ValueError, match="fork_tokens"):
        call_verify(a, f=F, out=out)


def test_mixed_devices_rejected():
    a = good()
    a["u_accept"] = torch.zeros(B, K, dtype=torch.float32, device="meta")
    with pytest.raises(ValueError, match="one device"):
        call_verify(a, f=F)


def test_residual_sample_checks_position():
    a = good()
    for bad in (torch.zeros(B + 1, dtype=torch.int32), torch.zeros(B, dtype=torch.int64),
                torch.zeros(B, 1, dtype=torch.int32)):
        with pytest.raises(ValueError, match="position"):
            sv.residual_sample(a["target"], a["draft"], a["draft_tokens"], a["temperature"],
                               bad, a["u_recover"])
    with pytest.raises(ValueError, match="ROCm device"):
        sv.residual_sample(a["target"], a["draft"], a["draft_tokens"], a["temperature"],
                           torch.zeros(B, dtype=torch.int32), a["u_recover"])


def test_forked_topf_checks():
    a = good()
    with pytest.raises(ValueError):
        sv.forked_topf(a["draft"], a["draft_tokens"][:, :-1].contiguous(), a["temperature"], F)
    with pytest.raises(ValueError):
        sv.forked_topf(a["draft"], a["draft_tokens"], a["temperature"], 0)
    with pytest.raises(ValueError, match="ROCm device"):
        sv.forked_topf(a["draft"], a["draft_tokens"], a["temperature"], F)


def test_softmax_and_sample_check_temperature_count():
    x = torch.zeros(10, V, dtype=torch.float32)
    with pytest.raises(ValueError, match="temperature"):
        sv.softmax_temp(x, torch.ones(2, dtype=torch.float32), rows_per_temp=4)
    with pytest.raises(ValueError, match="ROCm device"):
        sv.softmax_temp(x, torch.ones(3, dtype=torch.float32), rows_per_temp=4)
    u = torch.zeros(10, dtype=torch.float32)
    with pytest.raises(ValueError, match="temperature"):
        sv.sample_temp(x, torch.ones(9, dtype=torch.float32), u)
    with pytest.raises(ValueError, match="uniforms"):
        sv.sample_temp(x, torch.ones(10, dtype=torch.float32), u[:9].contiguous())


def test_cache_hit_checks():
    ft = torch.zeros(B, K + 1, F, dtype=torch.int32)
    with pytest.raises(ValueError):
        sv.cache_hit(ft, torch.zeros(B + 1, dtype=torch.int32), torch.zeros(B, dtype=torch.int32))
    with pytest.raises(ValueError, match="ROCm device"):
        sv.cache_hit(ft, torch.zeros(B, dtype=torch.int32), torch.zeros(B, dtype=torch.int32))


def test_softmax_checks_its_output():
    x = torch.zeros(8, 500, dtype=torch.bfloat16)
    t = torch.ones(8, dtype=torch.float32)
    with pytest.raises(ValueError, match="out must be"):
        sv.softmax_temp(x, t, out=torch.zeros(8, 499, dtype=torch.float32))
    with pytest.raises(ValueError, match="out must be"):
        sv.softmax_temp(x, t, out=torch.zeros(8, 500, dtype=torch.float16))
    with pytest.raises(ValueError, match="ROCm device"):
        sv.softmax_temp(x, t, out=torch.zeros(8, 500, dtype=torch.float32))


def test_noalloc_needs_its_outputs():
    a = good()
    with pytest.raises(ValueError, match="out"):
        sv.verify_noalloc(a["target"], a["draft"], a["draft_tokens"], a["temperature"],
                          a["u_accept"], a["u_recover"], None, f=F)
    outs = {"accept_len": torch.zeros(B, dtype=torch.int32),
            "out_token": torch.zeros(B, dtype=torch.int32)}
    with pytest.raises(ValueError, match="fork_tokens"):
        sv.verify_noalloc(a["target"], a["draft"], a["draft_tokens"], a["temperature"],
                          a["u_accept"], a["u_recover"], outs, f=F)
    with pytest.raises(ValueError, match="ROCm device"):
        sv.verify_noalloc(a["target"], a["draft"], a["draft_tokens"], a["temperature"],
                          a["u_accept"], a["u_recover"], outs, f=0)
