"""Python binding of libspecverify (ctypes).

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream; tensors must live on
a ROCm device.  The library must have been built (``build_lib.py``); nothing
falls back to the CPU.
"""

from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SV_OK = 0
SV_F32 = 0
SV_BF16 = 1

_lib = None
_lock = threading.Lock()


class SvBatch(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("k", ctypes.c_int32), ("V", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("target", ctypes.c_void_p),
        ("t_seq_stride", ctypes.c_int64), ("t_row_stride", ctypes.c_int64),
        ("draft", ctypes.c_void_p),
        ("d_seq_stride", ctypes.c_int64), ("d_row_stride", ctypes.c_int64),
        ("draft_tokens", ctypes.c_void_p),
        ("temperature", ctypes.c_void_p),
    ]


class SvForks(ctypes.Structure):
    _fields_ = [("f", ctypes.c_int32), ("tokens", ctypes.c_void_p),
                ("probs", ctypes.c_void_p), ("hits", ctypes.c_void_p)]


class SvOpts(ctypes.Structure):
    _fields_ = [("ev_stats_begin", ctypes.c_void_p),
                ("ev_stats_end", ctypes.c_void_p)]


class SpecVerifyError(RuntimeError):
    pass


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise SpecVerifyError(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -m verification_sampling_amd.build_lib`")
            L = ctypes.CDLL(LIB_PATH)
            vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
            L.sv_workspace_size.argtypes = [i32, i32, i32, i32]
            L.sv_workspace_size.restype = sz
            L.sv_workspace_init.argtypes = [vp, sz, vp]
            L.sv_workspace_init.restype = i32
            L.sv_status_string.argtypes = [i32]
            L.sv_status_string.restype = ctypes.c_char_p
            L.sv_version.argtypes = []
            L.sv_version.restype = ctypes.c_char_p
            L.sv_softmax_temp.argtypes = [vp, i32, i64, i32, i64, vp, i64, vp, i64, vp, sz, vp]
            L.sv_softmax_temp.restype = i32
            pb = ctypes.POINTER(SvBatch)
            pf = ctypes.POINTER(SvForks)
            po = ctypes.POINTER(SvOpts)
            L.sv_verify.argtypes = [pb, vp, vp, vp, vp, vp, vp, pf, vp, sz, vp]
            L.sv_verify.restype = i32
            L.sv_verify_ex.argtypes = [pb, vp, vp, vp, vp, vp, vp, pf, vp, sz, vp, po]
            L.sv_verify_ex.restype = i32
            L.sv_verify_noalloc.argtypes = [pb, vp, vp, vp, vp, vp, vp, pf, vp]
            L.sv_verify_noalloc.restype = i32
            L.sv_residual_sample.argtypes = [pb, vp, vp, vp, vp, i64, i64, vp, sz, vp]
            L.sv_residual_sample.restype = i32
            L.sv_forked_topf.argtypes = [pb, pf, vp, sz, vp]
            L.sv_forked_topf.restype = i32
            L.sv_cache_hit.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
            L.sv_cache_hit.restype = i32
            L.sv_sample_temp.argtypes = [vp, i32, i64, i32, i64, vp, i64, vp, vp, vp]
            L.sv_sample_temp.restype = i32
            _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().sv_status_string(int(code)).decode()


def _check(code: int, what: str) -> None:
    if code != SV_OK:
        raise SpecVerifyError(f"{what} failed: {status_string(code)}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _stream_handle(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ------------------------------------------------------------------ workspace

class Workspace:
    """A device buffer for the library's scratch data, zero-filled once when
    it is allocated (or grown); every call leaves its counters at zero, so
    the buffer then serves calls of any entry point and size.  Calls sharing
    it must not overlap (one workspace per stream)."""

    def __init__(self, device=None):
        self.device = torch.device("cuda") if device is None else torch.device(device)
        self.buf = None

    def get(self, nbytes: int, kind=None, stream=None) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(max(int(nbytes), 256), dtype=torch.uint8,
                                   device=self.device)
            _check(lib().sv_workspace_init(_ptr(self.buf), self.buf.numel(),
                                           _stream_handle(stream)), "sv_workspace_init")
        return self.buf


_ws_cache = {}


def default_workspace(device=None, stream=None) -> Workspace:
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    s = torch.cuda.current_stream(dev) if stream is None else stream
    key = (dev.index, s.cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None:
        ws = _ws_cache[key] = Workspace(dev)
    return ws


def workspace_size(B: int, k: int, V: int, f: int = 0) -> int:
    n = lib().sv_workspace_size(int(B), int(k), int(V), int(f))
    if n == 0:
        raise SpecVerifyError("sizes out of range for the workspace")
    return int(n)


# ------------------------------------------------------------------ helpers

def _same_device(tensors, what):
    """Every tensor on one ROCm device (checked after the shapes, so that a
    shape mistake is reported as such whatever the device)."""
    devs = {t.device for t in tensors if t is not None}
    if len(devs) != 1:
        raise ValueError(f"{what}: all tensors must be on one device, got {sorted(map(str, devs))}")
    dev = devs.pop()
    if dev.type != "cuda":
        raise ValueError(f"{what}: tensors must be on a ROCm device, got {dev}")
    return dev


def _batch(target, draft, draft_tokens, temperature, forks: bool = False):
    """The sv_batch of a call, after checking every shape, dtype and count
    against the others (a mismatch would make the kernels read outside an
    allocation).  target: [B, k+1, V] (None for the drafter-side forks);
    draft: [B, k+1, V], or [B, k, V] when no forks are asked for and a
    target is given; draft_tokens: [B, k] int32; temperature: [B] float32."""
    for t, name in ((draft, "draft"), (target, "target")):
        if t is None:
            continue
        if not isinstance(t, torch.Tensor) or t.dim() != 3:
            raise ValueError(f"{name} logits must be a 3-D tensor [B, k+1, V]")
        if t.stride(2) != 1:
            raise ValueError(f"{name} logits must have V contiguous")
        _dtype_code(t)
    ref = draft if target is None else target
    B, K1, V = ref.shape
    if K1 < 2:
        raise ValueError("logits need k+1 >= 2 positions")
    k = K1 - 1
    if target is not None and target.dtype != draft.dtype:
        raise ValueError("target and draft logits must share a dtype")
    dk = draft.shape[1]
    if draft.shape[0] != B or draft.shape[2] != V or not (
            dk == K1 or (dk == k and target is not None and not forks)):
        raise ValueError(f"draft logits {tuple(draft.shape)} do not match [B, k+1, V] = "
                         f"{(B, K1, V)} (or [B, k, V] without forks)")
    if (not isinstance(draft_tokens, torch.Tensor) or draft_tokens.dtype != torch.int32
            or not draft_tokens.is_contiguous() or tuple(draft_tokens.shape) != (B, k)):
        raise ValueError(f"draft_tokens must be contiguous int32 {(B, k)}")
    if (not isinstance(temperature, torch.Tensor) or temperature.dtype != torch.float32
            or not temperature.is_contiguous() or tuple(temperature.shape) != (B,)):
        raise ValueError(f"temperature must be contiguous float32 {(B,)}")
    b = SvBatch()
    b.B, b.k, b.V = int(B), int(k), int(V)
    b.dtype = _dtype_code(ref)
    if target is not None:
        b.target = target.data_ptr()
        b.t_seq_stride, b.t_row_stride = target.stride(0), target.stride(1)
    b.draft = draft.data_ptr()
    b.d_seq_stride, b.d_row_stride = draft.stride(0), draft.stride(1)
    b.draft_tokens = draft_tokens.data_ptr()
    b.temperature = temperature.data_ptr()
    return b


def _f32(t, shape, name):
    if (not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_contiguous()
            or tuple(t.shape) != tuple(shape)):
        raise ValueError(f"{name} must be contiguous float32 {tuple(shape)}")
    return t


def _out(t, shape, dtype, name):
    if (not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_contiguous()
            or tuple(t.shape) != tuple(shape)):
        raise ValueError(f"out[{name!r}] must be contiguous {dtype} {tuple(shape)}")
    return t


# ------------------------------------------------------------------ API

def _verify_outputs(out, B, k, f):
    _out(out.get("accept_len"), (B,), torch.int32, "accept_len")
    _out(out.get("out_token"), (B,), torch.int32, "out_token")
    for name in ("p_draft", "q_draft"):
        if out.get(name) is not None:
            _out(out[name], (B, k), torch.float32, name)
    if f > 0:
        _out(out.get("fork_tokens"), (B, k + 1, f), torch.int32, "fork_tokens")
        _out(out.get("fork_probs"), (B, k + 1, f), torch.float32, "fork_probs")
        if out.get("cache_hit") is not None:
            _out(out["cache_hit"], (B,), torch.int32, "cache_hit")


def _forks_of(out, f):
    if f <= 0:
        return None
    hits = out.get("cache_hit")
    return SvForks(int(f), out["fork_tokens"].data_ptr(), out["fork_probs"].data_ptr(),
                   hits.data_ptr() if hits is not None else None)


def verify(target, draft, draft_tokens, temperature, u_accept, u_recover, f: int = 0,
           want_p: bool = False, want_q: bool = False, want_hits: bool = False,
           workspace: Optional[Workspace] = None, stream=None, out=None, timing_events=None):
    """sv_verify: returns dict with accept_len [B] int32, out_token [B]
    int32, and optionally p_draft/q_draft [B,k] float32, fork_tokens
    [B,k+1,f] int32 / fork_probs [B,k+1,f] float32 and (f > 0, want_hits)
    cache_hit [B] int32."""
    if target is None:
        raise ValueError("verify needs the target logits")
    f = int(f)
    if f < 0:
        raise ValueError("f must be >= 0")
    b = _batch(target, draft, draft_tokens, temperature, forks=f > 0)
    B, k = b.B, b.k
    if f > min(16, b.V - 1):
        raise ValueError("f must be at most min(16, V - 1)")
    _f32(u_accept, (B, k), "u_accept")
    _f32(u_recover, (B, k + 1), "u_recover")
    if out is not None:
        _verify_outputs(out, B, k, f)
    dev = _same_device([target, draft, draft_tokens, temperature, u_accept, u_recover]
                       + ([t for t in out.values() if t is not None] if out else []), "verify")
    if out is None:
        out = {
            "accept_len": torch.empty(B, dtype=torch.int32, device=dev),
            "out_token": torch.empty(B, dtype=torch.int32, device=dev),
        }
        if want_p:
            out["p_draft"] = torch.empty(B, k, dtype=torch.float32, device=dev)
        if want_q:
            out["q_draft"] = torch.empty(B, k, dtype=torch.float32, device=dev)
        if f > 0:
            out["fork_tokens"] = torch.empty(B, k + 1, f, dtype=torch.int32, device=dev)
            out["fork_probs"] = torch.empty(B, k + 1, f, dtype=torch.float32, device=dev)
            if want_hits:
                out["cache_hit"] = torch.empty(B, dtype=torch.int32, device=dev)
    forks = _forks_of(out, f)
    ws = workspace or default_workspace(dev, stream)
    buf = ws.get(workspace_size(B, k, b.V, f), ("verify", B, k, b.V, f), stream)
    opts = None
    if timing_events is not None:
        opts = SvOpts(timing_events[0], timing_events[1])
    code = lib().sv_verify_ex(
        ctypes.byref(b), _ptr(u_accept), _ptr(u_recover), _ptr(out["accept_len"]),
        _ptr(out["out_token"]), _ptr(out.get("p_draft")), _ptr(out.get("q_draft")),
        ctypes.byref(forks) if forks is not None else None,
        _ptr(buf), buf.numel(), _stream_handle(stream),
        ctypes.byref(opts) if opts is not None else None)
    _check(code, "sv_verify")
    return out


# Bytes of sv_verify_noalloc's static scratch array (the header's
# SV_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20


def verify_noalloc(target, draft, draft_tokens, temperature, u_accept, u_recover, out,
                   f: int = 0, stream=None):
    """sv_verify_noalloc: sv_verify into the caller's output tensors (the
    dict keys of verify(); accept_len and out_token required, p_draft,
    q_draft optional, fork_tokens and fork_probs required when f > 0,
    cache_hit optional), with the library's static scratch array as the
    workspace.  Allocates nothing.  Calls on one device share that array:
    issue them on one stream."""
    if target is None:
        raise ValueError("verify_noalloc needs the target logits")
    if out is None:
        raise ValueError("verify_noalloc writes into `out`, which must hold the output tensors")
    f = int(f)
    if f < 0:
        raise ValueError("f must be >= 0")
    b = _batch(target, draft, draft_tokens, temperature, forks=f > 0)
    B, k = b.B, b.k
    if f > min(16, b.V - 1):
        raise ValueError("f must be at most min(16, V - 1)")
    _f32(u_accept, (B, k), "u_accept")
    _f32(u_recover, (B, k + 1), "u_recover")
    _verify_outputs(out, B, k, f)
    _same_device([target, draft, draft_tokens, temperature, u_accept, u_recover]
                 + [t for t in out.values() if t is not None], "verify_noalloc")
    need = workspace_size(B, k, b.V, f)
    if need > NOALLOC_SCRATCH_BYTES:
        raise SpecVerifyError(
            f"sv_verify_noalloc: B={B}, k={k}, V={b.V}, f={f} needs {need} bytes of workspace, "
            f"more than its scratch array of {NOALLOC_SCRATCH_BYTES} bytes; use verify()")
    forks = _forks_of(out, f)
    code = lib().sv_verify_noalloc(
        ctypes.byref(b), _ptr(u_accept), _ptr(u_recover), _ptr(out["accept_len"]),
        _ptr(out["out_token"]), _ptr(out.get("p_draft")), _ptr(out.get("q_draft")),
        ctypes.byref(forks) if forks is not None else None, _stream_handle(stream))
    _check(code, "sv_verify_noalloc")
    return out


def residual_sample(target, draft, draft_tokens, temperature, position, u_recover,
                    want_residual: bool = False, workspace: Optional[Workspace] = None,
                    stream=None):
    """sv_residual_sample: returns dict with token [B] int32 and optionally
    residual [B,k+1,V] float32."""
    if target is None:
        raise ValueError("residual_sample needs the target logits")
    b = _batch(target, draft, draft_tokens, temperature)
    B, k, V = b.B, b.k, b.V
    if (not isinstance(position, torch.Tensor) or position.dtype != torch.int32
            or not position.is_contiguous() or tuple(position.shape) != (B,)):
        raise ValueError(f"position must be contiguous int32 {(B,)}")
    _f32(u_recover, (B, k + 1), "u_recover")
    dev = _same_device([target, draft, draft_tokens, temperature, position, u_recover],
                       "residual_sample")
    out = {"token": torch.empty(B, dtype=torch.int32, device=dev)}
    res = None
    rs0 = rs1 = 0
    if want_residual:
        Vp = (V + 3) // 4 * 4
        res = torch.empty(B, k + 1, Vp, dtype=torch.float32, device=dev)[:, :, :V]
        rs0, rs1 = res.stride(0), res.stride(1)
        out["residual"] = res
    ws = workspace or default_workspace(dev, stream)
    buf = ws.get(workspace_size(B, k, V, 0), ("residual", B, k, V), stream)
    code = lib().sv_residual_sample(
        ctypes.byref(b), _ptr(position), _ptr(u_recover), _ptr(out["token"]),
        ctypes.c_void_p(res.data_ptr()) if res is not None else None, rs0, rs1,
        _ptr(buf), buf.numel(), _stream_handle(stream))
    _check(code, "sv_residual_sample")
    return out


def forked_topf(draft, draft_tokens, temperature, f: int,
                workspace: Optional[Workspace] = None, stream=None):
    """sv_forked_topf: returns (tokens [B,k+1,f] int32, probs [B,k+1,f]
    float32)."""
    f = int(f)
    b = _batch(None, draft, draft_tokens, temperature, forks=True)
    B, k = b.B, b.k
    if not 1 <= f <= min(16, b.V - 1):
        raise ValueError("f must be in [1, min(16, V - 1)]")
    dev = _same_device([draft, draft_tokens, temperature], "forked_topf")
    toks = torch.empty(B, k + 1, f, dtype=torch.int32, device=dev)
    probs = torch.empty(B, k + 1, f, dtype=torch.float32, device=dev)
    forks = SvForks(int(f), toks.data_ptr(), probs.data_ptr())
    ws = workspace or default_workspace(dev, stream)
    buf = ws.get(workspace_size(B, k, b.V, f), ("forks", B, k, b.V, f), stream)
    code = lib().sv_forked_topf(ctypes.byref(b), ctypes.byref(forks), _ptr(buf),
                                buf.numel(), _stream_handle(stream))
    _check(code, "sv_forked_topf")
    return toks, probs


def cache_hit(fork_tokens, accept_len, out_token, stream=None):
    """sv_cache_hit: the index of each outcome token among the forks of its
    outcome position ([B] int32, -1 on a miss).  fork_tokens [B,k+1,f],
    accept_len [B] and out_token [B]: contiguous int32 on the device."""
    for t, name in ((fork_tokens, "fork_tokens"), (accept_len, "accept_len"),
                    (out_token, "out_token")):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous int32")
    if fork_tokens.dim() != 3:
        raise ValueError("fork_tokens must be [B, k+1, f]")
    B, K1, f = fork_tokens.shape
    if tuple(accept_len.shape) != (B,) or tuple(out_token.shape) != (B,):
        raise ValueError("accept_len and out_token must be [B]")
    _same_device([fork_tokens, accept_len, out_token], "cache_hit")
    hits = torch.empty(B, dtype=torch.int32, device=fork_tokens.device)
    code = lib().sv_cache_hit(int(B), int(K1 - 1), int(f), _ptr(fork_tokens), _ptr(accept_len),
                              _ptr(out_token), _ptr(hits), _stream_handle(stream))
    _check(code, "sv_cache_hit")
    return hits


def sample_temp(logits, temperature, uniforms, rows_per_temp: int = 1, stream=None):
    """sv_sample_temp: one token per row of a [rows, V] tensor (V
    contiguous): greedy at temperature 0, else the inverse-CDF draw from
    softmax(row / tau) with that row's uniform.  Returns int32 [rows] (-1
    for an error row)."""
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be [rows, V] with V contiguous")
    rows, V = logits.shape
    _dtype_code(logits)
    if rows_per_temp < 1:
        raise ValueError("rows_per_temp must be >= 1")
    if temperature.dtype != torch.float32 or not temperature.is_contiguous():
        raise ValueError("temperature must be contiguous float32")
    if temperature.numel() * rows_per_temp < rows:
        raise ValueError("one temperature per rows_per_temp rows is needed")
    _f32(uniforms, (rows,), "uniforms")
    _same_device([logits, temperature, uniforms], "sample_temp")
    toks = torch.empty(rows, dtype=torch.int32, device=logits.device)
    code = lib().sv_sample_temp(_ptr(logits), _dtype_code(logits), int(rows), int(V),
                                logits.stride(0), _ptr(temperature), int(rows_per_temp),
                                _ptr(uniforms), _ptr(toks), _stream_handle(stream))
    _check(code, "sv_sample_temp")
    return toks


def softmax_temp(logits, temperature, rows_per_temp: int = 1,
                 workspace: Optional[Workspace] = None, stream=None, out=None):
    """sv_softmax_temp over the rows of a [rows, V] tensor (V contiguous);
    returns float32 [rows, V] (written into `out` when given: float32
    [rows, V], V contiguous, rows 16-byte aligned)."""
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise ValueError("logits must be [rows, V] with V contiguous")
    rows, V = logits.shape
    _dtype_code(logits)
    if rows_per_temp < 1:
        raise ValueError("rows_per_temp must be >= 1")
    if temperature.dtype != torch.float32 or not temperature.is_contiguous():
        raise ValueError("temperature must be contiguous float32")
    if temperature.numel() * rows_per_temp < rows:
        raise ValueError("one temperature per rows_per_temp rows is needed")
    if out is not None and (out.dtype != torch.float32 or tuple(out.shape) != (rows, V)
                            or out.stride(1) != 1):
        raise ValueError(f"out must be float32 [{rows}, {V}] with V contiguous")
    dev = _same_device([logits, temperature] + ([out] if out is not None else []),
                       "softmax_temp")
    if out is None:
        Vp = (V + 3) // 4 * 4
        out = torch.empty(rows, Vp, dtype=torch.float32, device=dev)[:, :V]
    ws = workspace or default_workspace(dev, stream)
    buf = ws.get(workspace_size(rows, 0, V, 0), ("softmax", rows, V), stream)
    code = lib().sv_softmax_temp(
        _ptr(logits), _dtype_code(logits), int(rows), int(V), logits.stride(0),
        _ptr(temperature), int(rows_per_temp), ctypes.c_void_p(out.data_ptr()), out.stride(0),
        _ptr(buf), buf.numel(), _stream_handle(stream))
    _check(code, "sv_softmax_temp")
    return out


class PreparedVerify:
    """sv_verify with every argument marshalled once, for issuing the same
    call repeatedly (benchmark loops): calling it only forwards the prepared
    pointers to the library."""

    def __init__(self, target, draft, draft_tokens, temperature, u_accept, u_recover,
                 f: int, out: dict, workspace: Workspace, stream=None):
        self._keep = (target, draft, draft_tokens, temperature, u_accept, u_recover, out)
        self.batch = _batch(target, draft, draft_tokens, temperature, forks=f > 0)
        B, k = self.batch.B, self.batch.k
        _f32(u_accept, (B, k), "u_accept")
        _f32(u_recover, (B, k + 1), "u_recover")
        _out(out.get("accept_len"), (B,), torch.int32, "accept_len")
        _out(out.get("out_token"), (B,), torch.int32, "out_token")
        if f > 0:
            _out(out.get("fork_tokens"), (B, k + 1, f), torch.int32, "fork_tokens")
            _out(out.get("fork_probs"), (B, k + 1, f), torch.float32, "fork_probs")
        _same_device([target, draft, draft_tokens, temperature, u_accept, u_recover]
                     + [t for t in out.values() if t is not None], "PreparedVerify")
        hits = out.get("cache_hit")
        self.forks = SvForks(int(f), out["fork_tokens"].data_ptr(),
                             out["fork_probs"].data_ptr(),
                             hits.data_ptr() if hits is not None else None) if f > 0 else None
        buf = workspace.get(workspace_size(B, k, self.batch.V, f),
                            ("verify", B, k, self.batch.V, f), stream)
        self._buf = buf
        self.args = [
            ctypes.byref(self.batch), _ptr(u_accept), _ptr(u_recover), _ptr(out["accept_len"]),
            _ptr(out["out_token"]), _ptr(out.get("p_draft")), _ptr(out.get("q_draft")),
            ctypes.byref(self.forks) if self.forks is not None else None,
            _ptr(buf), ctypes.c_size_t(buf.numel()), _stream_handle(stream)]
        self.fn = lib().sv_verify_ex

    def __call__(self, opts: Optional[SvOpts] = None) -> None:
        code = self.fn(*self.args, ctypes.byref(opts) if opts is not None else None)
        if code != SV_OK:
            _check(code, "sv_verify")
