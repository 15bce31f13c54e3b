"""ctypes binding of libattn.so; names follow the C ABI in include/attn.h."""
from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libattn.so")

ATTN_OK, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP, ATTN_ERR_SCRATCH = 0, 1, 2, 3, 4
ATTN_F32, ATTN_BF16 = 0, 1

_lib = None
_lock = threading.Lock()

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_S = ctypes.c_size_t
_U64 = ctypes.c_uint64

_SIGNATURES = {
    "attn_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_bwd_workspace_bytes": (_S, [_I, _I, _I, _I]),
    "attn_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_bwd_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_bwd_noalloc_max_rows": (_S, []),
    "attn_bwd_preprocess": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "attn_bwd_dkdv": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_bwd_dq": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_bwd_dq_fused": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_fwd_block_sparse": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_bwd_block_sparse": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _S, _I, _I, _I, _I, _I, _F,
                                   _I, _P]),
    "attn_fwd_dropout": (_I, [_P, _P, _P, _P, _P, _F, _U64, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_bwd_dropout": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _F, _U64, _P, _S, _I, _I, _I, _I, _I, _F, _I,
                              _P]),
    "attn_decode_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "attn_decode": (_I, [_P, _P, _P, _P, _P, _P, _S, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "attn_fwd_fp8": (_I, [_P, _P, _P, _F, _F, _F, _P, _P, _I, _I, _I, _I, _F, _I, _P]),
    "attn_status_string": (ctypes.c_char_p, [_I]),
    "attn_abi_version": (_I, []),
    # hardware probes (include/attn_probe.h)
    "attn_probe_lds_rate": (_I, [_I, _I, _P, _P, _P]),
    "attn_probe_issue": (_I, [_P, _I, _I, _P, _P, _P]),
    "attn_probe_wave_simd": (_I, [_I, _P, _P]),
    "attn_probe_atomic": (_I, [_P, _S, _I, _P]),
    "attn_probe_exp2": (_I, [_P, _P, _S, _P]),
    "attn_probe_read_rate": (_I, [_P, _S, _I, _I, _P, _P]),
}


class AttnError(RuntimeError):
    """A non-OK status from the C ABI."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")


def load_library(path: str | None = None):
    """Load libattn.so (built in-tree by exact_io_aware_23_amd.build) once."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is missing: build it with `python -m exact_io_aware_23_amd.build`")
        lib = ctypes.CDLL(p)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if path is None:
            _lib = lib
        return lib


def status_string(status: int) -> str:
    return load_library().attn_status_string(status).decode()


def abi_version() -> int:
    return load_library().attn_abi_version()


def bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return load_library().attn_bwd_workspace_bytes(B, H, N, d)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(name: str, t: torch.Tensor, shape, dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _call(name: str, *args):
    st = getattr(load_library(), name)(*args)
    if st != ATTN_OK:
        raise AttnError(name, st)


def _default_scale(d: int, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None, causal: bool = False,
        out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """attn_fwd on [B, H, N, d] tensors; returns (O, L) with L fp32 [B, H, N]."""
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(name, t, (B, H, N, d), q.dtype)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check("out", out, (B, H, N, d), q.dtype)
    _check("lse", lse, (B, H, N), torch.float32)
    _call("attn_fwd", q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
          _dtype_code(q), _default_scale(d, scale), int(bool(causal)), _stream(q.device))
    return out, lse


def fwd_fp8(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, descale_q: float, descale_k: float,
            descale_v: float, scale: float | None = None, causal: bool = False, out=None, lse=None):
    """attn_fwd_fp8: q8, k8, v8 are e4m3 codes [B, H, N, d] (torch.uint8 or
    torch.float8_e4m3fn) with one scale per tensor; returns (O bf16, L fp32)."""
    B, H, N, d = q8.shape
    for name, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        if not isinstance(t, torch.Tensor) or t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError(f"{name} must be a uint8 or float8_e4m3fn tensor")
        _check(name, t, (B, H, N, d), t.dtype)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    _check("out", out, (B, H, N, d), torch.bfloat16)
    _check("lse", lse, (B, H, N), torch.float32)
    _call("attn_fwd_fp8", q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), float(descale_q), float(descale_k),
          float(descale_v), out.data_ptr(), lse.data_ptr(), B, H, N, d, _default_scale(d, scale),
          int(bool(causal)), _stream(q8.device))
    return out, lse


def bwd(q, k, v, o, lse, do, scale: float | None = None, causal: bool = False, workspace=None,
        dq=None, dk=None, dv=None):
    """attn_bwd; returns (dQ, dK, dV)."""
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(name, t, (B, H, N, d), q.dtype)
    _check("lse", lse, (B, H, N), torch.float32)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check(name, t, (B, H, N, d), q.dtype)
    ws_bytes = bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    _call("attn_bwd", q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
          dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), workspace.numel(), B, H, N, d,
          _dtype_code(q), _default_scale(d, scale), int(bool(causal)), _stream(q.device))
    return dq, dk, dv


def bwd_noalloc_max_rows() -> int:
    return int(load_library().attn_bwd_noalloc_max_rows())


def bwd_noalloc(q, k, v, o, lse, do, scale: float | None = None, causal: bool = False, dq=None, dk=None, dv=None):
    """attn_bwd_noalloc (no workspace: the library's static scratch array); returns (dQ, dK, dV).
    dq, dk, dv are allocated here when not given; the library call itself allocates nothing."""
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(name, t, (B, H, N, d), q.dtype)
    _check("lse", lse, (B, H, N), torch.float32)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check(name, t, (B, H, N, d), q.dtype)
    _call("attn_bwd_noalloc", q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
          dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, _dtype_code(q), _default_scale(d, scale),
          int(bool(causal)), _stream(q.device))
    return dq, dk, dv


def _block_mask(block_mask: torch.Tensor, B: int, H: int, N: int) -> torch.Tensor:
    """Check a block mask: uint8 on the GPU, [nb, nb] or [1 or B*H, nb, nb], nb = ceil(N/128)."""
    nb = (N + 127) // 128
    if not isinstance(block_mask, torch.Tensor):
        raise TypeError("block_mask must be a torch.Tensor")
    m = block_mask[None] if block_mask.dim() == 2 else block_mask
    if m.dim() != 3 or m.shape[1:] != (nb, nb) or m.shape[0] not in (1, B * H):
        raise ValueError(f"block_mask has shape {tuple(block_mask.shape)}, expected ({nb}, {nb}) or "
                         f"(1 or {B * H}, {nb}, {nb})")
    _check("block_mask", m, tuple(m.shape), torch.uint8)
    return m


def fwd_block_sparse(q, k, v, block_mask, scale: float | None = None, causal: bool = False, out=None, lse=None):
    """attn_fwd_block_sparse; returns (O, L).  A row with no allowed key gets O = 0, L = -inf."""
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(name, t, (B, H, N, d), q.dtype)
    m = _block_mask(block_mask, B, H, N)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check("out", out, (B, H, N, d), q.dtype)
    _check("lse", lse, (B, H, N), torch.float32)
    _call("attn_fwd_block_sparse", q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
          m.data_ptr(), m.shape[0], B, H, N, d, _dtype_code(q), _default_scale(d, scale), int(bool(causal)),
          _stream(q.device))
    return out, lse


def bwd_block_sparse(q, k, v, o, lse, do, block_mask, scale: float | None = None, causal: bool = False,
                     workspace=None, dq=None, dk=None, dv=None):
    """attn_bwd_block_sparse; returns (dQ, dK, dV)."""
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(name, t, (B, H, N, d), q.dtype)
    _check("lse", lse, (B, H, N), torch.float32)
    m = _block_mask(block_mask, B, H, N)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check(name, t, (B, H, N, d), q.dtype)
    ws_bytes = bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    _call("attn_bwd_block_sparse", q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
          do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), m.data_ptr(), m.shape[0],
          workspace.data_ptr(), workspace.numel(), B, H, N, d, _dtype_code(q), _default_scale(d, scale),
          int(bool(causal)), _stream(q.device))
    return dq, dk, dv


def fwd_dropout(q, k, v, p_drop: float, seed: int, scale: float | None = None, causal: bool = False, out=None,
                lse=None):
    """attn_fwd_dropout; returns (O, L).  The rate applied is round(256 p_drop) / 256."""
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(name, t, (B, H, N, d), q.dtype)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check("out", out, (B, H, N, d), q.dtype)
    _check("lse", lse, (B, H, N), torch.float32)
    _call("attn_fwd_dropout", q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
          float(p_drop), int(seed) & 0xFFFFFFFFFFFFFFFF, B, H, N, d, _dtype_code(q), _default_scale(d, scale),
          int(bool(causal)), _stream(q.device))
    return out, lse


def bwd_dropout(q, k, v, o, lse, do, p_drop: float, seed: int, scale: float | None = None, causal: bool = False,
                workspace=None, dq=None, dk=None, dv=None):
    """attn_bwd_dropout with the forward's p_drop and seed; returns (dQ, dK, dV)."""
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(name, t, (B, H, N, d), q.dtype)
    _check("lse", lse, (B, H, N), torch.float32)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check(name, t, (B, H, N, d), q.dtype)
    ws_bytes = bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    _call("attn_bwd_dropout", q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
          do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), float(p_drop),
          int(seed) & 0xFFFFFFFFFFFFFFFF, workspace.data_ptr(), workspace.numel(), B, H, N, d, _dtype_code(q),
          _default_scale(d, scale), int(bool(causal)), _stream(q.device))
    return dq, dk, dv


def decode_workspace_bytes(B: int, H: int, Nq: int, Nk: int, d: int) -> int:
    return int(load_library().attn_decode_workspace_bytes(B, H, Nq, Nk, d))


def decode(q, k_cache, v_cache, scale: float | None = None, causal: bool = False, out=None, lse=None,
           workspace=None):
    """attn_decode: q [B, H, Nq, d] against the cache [B, H, Nk, d]; returns (O [B, H, Nq, d], L [B, H, Nq])."""
    B, H, Nq, d = q.shape
    Nk = k_cache.shape[2]
    _check("q", q, (B, H, Nq, d), q.dtype)
    _check("k_cache", k_cache, (B, H, Nk, d), q.dtype)
    _check("v_cache", v_cache, (B, H, Nk, d), q.dtype)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    _check("out", out, (B, H, Nq, d), q.dtype)
    _check("lse", lse, (B, H, Nq), torch.float32)
    ws_bytes = decode_workspace_bytes(B, H, Nq, Nk, d)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    _call("attn_decode", q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(), lse.data_ptr(),
          workspace.data_ptr(), workspace.numel(), B, H, Nq, Nk, d, _dtype_code(q), _default_scale(d, scale),
          int(bool(causal)), _stream(q.device))
    return out, lse


def bwd_preprocess(o, do, delta=None):
    """attn_bwd_preprocess; returns delta fp32 [B, H, N]."""
    B, H, N, d = o.shape
    for name, t in (("o", o), ("do", do)):
        _check(name, t, (B, H, N, d), o.dtype)
    delta = torch.empty((B, H, N), dtype=torch.float32, device=o.device) if delta is None else delta
    _check("delta", delta, (B, H, N), torch.float32)
    _call("attn_bwd_preprocess", o.data_ptr(), do.data_ptr(), delta.data_ptr(), B, H, N, d, _dtype_code(o),
          _stream(o.device))
    return delta


def bwd_dkdv(q, k, v, lse, do, delta, scale: float | None = None, causal: bool = False, dk=None, dv=None):
    """attn_bwd_dkdv; returns (dK, dV)."""
    B, H, N, d = q.shape
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t in (("q", q), ("k", k), ("v", v), ("do", do), ("dk", dk), ("dv", dv)):
        _check(name, t, (B, H, N, d), q.dtype)
    _check("lse", lse, (B, H, N), torch.float32)
    _check("delta", delta, (B, H, N), torch.float32)
    _call("attn_bwd_dkdv", q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(), do.data_ptr(),
          delta.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, _dtype_code(q), _default_scale(d, scale),
          int(bool(causal)), _stream(q.device))
    return dk, dv


def bwd_dq(q, k, v, lse, do, delta, scale: float | None = None, causal: bool = False, dq=None,
           delta_out=None):
    """attn_bwd_dq; returns (dQ, exact delta)."""
    B, H, N, d = q.shape
    dq = torch.empty_like(q) if dq is None else dq
    delta_out = torch.empty_like(delta) if delta_out is None else delta_out
    for name, t in (("q", q), ("k", k), ("v", v), ("do", do), ("dq", dq)):
        _check(name, t, (B, H, N, d), q.dtype)
    _check("lse", lse, (B, H, N), torch.float32)
    _check("delta", delta, (B, H, N), torch.float32)
    _check("delta_out", delta_out, (B, H, N), torch.float32)
    _call("attn_bwd_dq", q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(), do.data_ptr(),
          delta.data_ptr(), dq.data_ptr(), delta_out.data_ptr(), B, H, N, d, _dtype_code(q),
          _default_scale(d, scale), int(bool(causal)), _stream(q.device))
    return dq, delta_out


def bwd_dq_fused(q, k, v, o, lse, do, scale: float | None = None, causal: bool = False, dq=None, delta_out=None):
    """attn_bwd_dq_fused (preprocess and dq in one launch); returns (dQ, exact delta)."""
    B, H, N, d = q.shape
    dq = torch.empty_like(q) if dq is None else dq
    delta_out = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if delta_out is None else delta_out
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq)):
        _check(name, t, (B, H, N, d), q.dtype)
    _check("lse", lse, (B, H, N), torch.float32)
    _check("delta_out", delta_out, (B, H, N), torch.float32)
    _call("attn_bwd_dq_fused", q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
          dq.data_ptr(), delta_out.data_ptr(), B, H, N, d, _dtype_code(q), _default_scale(d, scale),
          int(bool(causal)), _stream(q.device))
    return dq, delta_out


class _Attention(torch.autograd.Function):
    """attn_fwd in the forward (saving O and L), attn_bwd in the backward."""

    @staticmethod
    def forward(ctx, q, k, v, scale, causal):
        o, lse = fwd(q, k, v, scale=scale, causal=causal)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.scale, ctx.causal = scale, causal
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = bwd(q, k, v, o, lse, do.to(q.dtype).contiguous(), scale=ctx.scale, causal=ctx.causal)
        return dq, dk, dv, None, None


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None, causal: bool = False):
    """O = softmax(scale Q K^T + mask) V on [B, H, N, d] tensors, differentiable
    with respect to q, k and v through attn_bwd (bf16 only; the fp32 forward
    has no backward and raises there)."""
    return _Attention.apply(q, k, v, _default_scale(q.shape[-1], scale), bool(causal))
