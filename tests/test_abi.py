"""The C ABI library loads, exports every function include/specverify.h
declares, and its host-side validation returns the documented status codes
before touching the GPU (CPU only: no call here reaches a kernel launch)."""

import ctypes
import os
import re

import pytest

from verification_sampling_amd import specverify as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")

OK, INVALID, MISALIGNED, WORKSPACE = 0, 1, 2, 3


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(sv.LIB_PATH):
        pytest.skip("library not built")
    return sv.lib()


def test_every_declared_function_is_exported(L):
    names = header_functions()
    assert "sv_verify" in names and "sv_forked_topf" in names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    assert sv.status_string(OK) == "SV_OK"
    assert sv.status_string(MISALIGNED) == "SV_ERR_MISALIGNED"
    assert sv.status_string(99) == "SV_UNKNOWN_STATUS"
    assert L.sv_version().decode().startswith("libspecverify")


def test_workspace_size_ranges(L):
    assert L.sv_workspace_size(64, 7, 151936, 3) > 0
    assert L.sv_workspace_size(64, 7, 151936, 3) >= L.sv_workspace_size(64, 7, 151936, 0)
    assert L.sv_workspace_size(64, 64, 151936, 3) == 0   # k > 63
    assert L.sv_workspace_size(64, 7, 1, 0) == 0         # V < 2
    assert L.sv_workspace_size(64, 7, 1000, 17) == 0     # f > 16
    assert L.sv_workspace_size(-1, 7, 1000, 0) == 0


FAKE = 0x10000  # 16-byte aligned; never dereferenced by host validation


def batch(B=2, k=3, V=1024, dtype=1, target=FAKE, draft=FAKE, t_row=1024, d_row=1024):
    b = sv.SvBatch()
    b.B, b.k, b.V, b.dtype = B, k, V, dtype
    b.target, b.draft = target, draft
    b.t_seq_stride, b.t_row_stride = (k + 1) * t_row, t_row
    b.d_seq_stride, b.d_row_stride = (k + 1) * d_row, d_row
    b.draft_tokens = FAKE
    b.temperature = FAKE
    return b


def call_verify(L, b, ws_bytes=0, forks=None, outs=True):
    p = ctypes.c_void_p(FAKE) if outs else None
    return L.sv_verify(ctypes.byref(b), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), p, p,
                       None, None, ctypes.byref(forks) if forks else None,
                       ctypes.c_void_p(FAKE), ws_bytes, None)


def test_verify_validation(L):
    assert L.sv_verify(None, None, None, None, None, None, None, None, None, 0, None) == INVALID
    assert call_verify(L, batch(k=0)) == INVALID
    assert call_verify(L, batch(k=64)) == INVALID
    assert call_verify(L, batch(V=1)) == INVALID
    assert call_verify(L, batch(dtype=7)) == INVALID
    assert call_verify(L, batch(B=0)) == OK            # empty batch: nothing to do
    assert call_verify(L, batch(target=FAKE + 2)) == MISALIGNED
    assert call_verify(L, batch(t_row=1025)) == MISALIGNED   # bf16 row of 2050 bytes
    assert call_verify(L, batch(dtype=0, V=1002, t_row=1002, d_row=1002)) == MISALIGNED
    assert call_verify(L, batch(), outs=False) == INVALID
    assert call_verify(L, batch(), ws_bytes=16) == WORKSPACE
    assert call_verify(L, batch(), forks=sv.SvForks(0, FAKE, FAKE)) == INVALID
    assert call_verify(L, batch(), forks=sv.SvForks(17, FAKE, FAKE)) == INVALID
    assert call_verify(L, batch(V=4, t_row=8, d_row=8), forks=sv.SvForks(4, FAKE, FAKE)) == INVALID
    assert call_verify(L, batch(), forks=sv.SvForks(3, None, FAKE)) == INVALID
    assert call_verify(L, batch(), ws_bytes=16, forks=sv.SvForks(3, FAKE, None)) == WORKSPACE


def test_residual_and_forks_validation(L):
    b = batch()
    p = ctypes.c_void_p(FAKE)
    assert L.sv_residual_sample(ctypes.byref(b), None, p, p, None, 0, 0, p, 1 << 30, None) == INVALID
    assert L.sv_residual_sample(ctypes.byref(b), p, p, p, ctypes.c_void_p(FAKE + 4), 0, 0, p,
                                1 << 30, None) == MISALIGNED
    assert L.sv_residual_sample(ctypes.byref(b), p, p, p, p, 4 * 1025, 1025, p, 1 << 30,
                                None) == MISALIGNED
    assert L.sv_residual_sample(ctypes.byref(b), p, p, p, None, 0, 0, p, 8, None) == WORKSPACE
    f = sv.SvForks(3, FAKE, FAKE)
    assert L.sv_forked_topf(ctypes.byref(b), None, p, 1 << 30, None) == INVALID
    bt = batch(target=0)
    assert L.sv_forked_topf(ctypes.byref(bt), ctypes.byref(f), p, 8, None) == WORKSPACE
    bd = batch(draft=FAKE + 8)
    assert L.sv_forked_topf(ctypes.byref(bd), ctypes.byref(f), p, 1 << 30, None) == MISALIGNED


def test_softmax_validation(L):
    p = ctypes.c_void_p(FAKE)
    args = dict(logits=p, dtype=1, rows=4, V=1000, row_stride=1000, temp=p, rpt=1, probs=p,
                ostride=1000, ws=p, wsb=1 << 30)

    def call(**kw):
        a = dict(args, **kw)
        return L.sv_softmax_temp(a["logits"], a["dtype"], a["rows"], a["V"], a["row_stride"],
                                 a["temp"], a["rpt"], a["probs"], a["ostride"], a["ws"], a["wsb"],
                                 None)

    assert call(rows=0) == OK
    assert call(rpt=0) == INVALID
    assert call(dtype=3) == INVALID
    assert call(V=1) == INVALID
    assert call(ostride=996) == INVALID
    assert call(row_stride=1004) == MISALIGNED   # bf16 rows of 2008 bytes
    assert call(ostride=1001) == MISALIGNED
    assert call(wsb=64) == WORKSPACE
    assert call(logits=None) == INVALID


def test_cache_hit_validation(L):
    p = ctypes.c_void_p(FAKE)
    assert L.sv_cache_hit(0, 7, 3, None, None, None, None, None) == OK   # empty batch
    assert L.sv_cache_hit(-1, 7, 3, p, p, p, p, None) == INVALID
    assert L.sv_cache_hit(4, 0, 3, p, p, p, p, None) == INVALID
    assert L.sv_cache_hit(4, 64, 3, p, p, p, p, None) == INVALID
    assert L.sv_cache_hit(4, 7, 0, p, p, p, p, None) == INVALID
    assert L.sv_cache_hit(4, 7, 17, p, p, p, p, None) == INVALID
    for i in range(4):
        args = [p, p, p, p]
        args[i] = None
        assert L.sv_cache_hit(4, 7, 3, *args, None) == INVALID


def test_sample_temp_validation(L):
    p = ctypes.c_void_p(FAKE)

    def call(logits=p, dtype=1, rows=4, V=1000, stride=1000, temp=p, rpt=1, u=p, out=p):
        return L.sv_sample_temp(logits, dtype, rows, V, stride, temp, rpt, u, out, None)

    assert call(rows=0, logits=None, temp=None, u=None, out=None) == OK
    assert call(rows=-1) == INVALID
    assert call(V=1) == INVALID
    assert call(dtype=2) == INVALID
    assert call(rpt=0) == INVALID
    assert call(stride=999) == INVALID
    assert call(dtype=0, V=1048577, stride=1048580) == INVALID    # more than 4096 fp32 slabs
    assert call(V=2097153, stride=2097160) == INVALID             # more than 4096 bf16 slabs
    assert call(stride=1004) == MISALIGNED                         # bf16 rows of 2008 bytes
    assert call(logits=ctypes.c_void_p(FAKE + 8)) == MISALIGNED
    for name in ("logits", "temp", "u", "out"):
        assert call(**{name: None}) == INVALID


def test_noalloc_scratch_limit_and_validation(L):
    """sv_verify_noalloc refuses shapes whose workspace exceeds its static
    array, and bad arguments, before any GPU call; the binding's copy of the
    array's size is the header's."""
    text = open(HEADER).read()
    m = re.search(r"#define\s+SV_NOALLOC_SCRATCH_BYTES\s+\(\(size_t\)(\d+)\s*<<\s*(\d+)\)", text)
    assert m, "SV_NOALLOC_SCRATCH_BYTES not found in the header"
    assert sv.NOALLOC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))
    p = ctypes.c_void_p(FAKE)

    def call(b, forks=None):
        return L.sv_verify_noalloc(ctypes.byref(b) if b is not None else None, p, p, p, p, None,
                                   None, ctypes.byref(forks) if forks else None, None)

    assert call(None) == INVALID
    assert call(batch(k=64)) == INVALID
    assert call(batch(V=1)) == INVALID
    assert call(batch(), forks=sv.SvForks(17, FAKE, FAKE)) == INVALID
    assert call(batch(), forks=sv.SvForks(0, FAKE, FAKE)) == INVALID
    big = batch(B=256, k=7, V=151936, t_row=151936, d_row=151936)
    assert L.sv_workspace_size(256, 7, 151936, 3) > sv.NOALLOC_SCRATCH_BYTES
    assert call(big, forks=sv.SvForks(3, FAKE, FAKE)) == WORKSPACE
    # the headline batch fits
    assert L.sv_workspace_size(64, 7, 151936, 16) <= sv.NOALLOC_SCRATCH_BYTES


def test_batch_limits(L):
    """B <= 8192 and B * (k + 1) <= 32768 rows per call; at the limits the
    shape is accepted (the call then fails only on the short workspace)."""
    V = 64
    assert call_verify(L, batch(B=8193, k=3, V=V, t_row=V, d_row=V)) == INVALID
    assert call_verify(L, batch(B=4097, k=7, V=V, t_row=V, d_row=V)) == INVALID   # 32,776 rows
    assert call_verify(L, batch(B=8192, k=3, V=V, t_row=V, d_row=V), ws_bytes=16) == WORKSPACE
    assert call_verify(L, batch(B=4096, k=7, V=V, t_row=V, d_row=V), ws_bytes=16) == WORKSPACE
