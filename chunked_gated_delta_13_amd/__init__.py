"""Kimi Delta Attention (KDA) on MI355X: Python binding of libkda.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libkda.so``; PyTorch supplies device memory and the current stream.

    o, S_T = chunk_prefill(q, k, v, log_alpha, beta, S0=None, chunk=64)
    o      = decode_step(q, k, v, log_alpha, beta, S)      # S updated in place

Layouts: q, k, log_alpha [B, T, H, dk]; v [B, T, H, dv]; beta [B, T, H];
S0 / S_T [B, H, dk, dv] (fp32).  q, k, v, o share one dtype (bf16 or fp32);
log_alpha and beta are fp32.
"""
from __future__ import annotations

import ctypes

from . import _lib
from ._lib import KDAError

__all__ = ["chunk_prefill", "chunk_prefill_ckpt", "chunk_prefill_gate", "chunk_prefill_noalloc",
           "decode_step", "spec_verify", "spec_commit", "prefill_plan", "prefill_workspace_bytes",
           "abi_version", "KDAError", "load_library"]


def load_library():
    return _lib.load()


def abi_version() -> int:
    return _lib.load().kda_abi_version()


def _torch():
    import torch
    return torch


def _dtype_code(dt):
    torch = _torch()
    if dt == torch.bfloat16:
        return _lib.KDA_BF16
    if dt == torch.float32:
        return _lib.KDA_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {dt}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_tensor(name, t, dtype, shape, device):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def prefill_plan(B, T, H, dk, dv, chunk=64, dtype=None):
    """(seg_len, n_vs) that the library's scheduler picks for this shape."""
    torch = _torch()
    code = _dtype_code(dtype or torch.bfloat16)
    seg = ctypes.c_int(0)
    nvs = ctypes.c_int(0)
    _lib.check(_lib.load().kda_chunk_prefill_plan(B, T, H, dk, dv, chunk, code,
                                                  ctypes.byref(seg), ctypes.byref(nvs)),
               "kda_chunk_prefill_plan")
    return seg.value, nvs.value


def prefill_workspace_bytes(B, T, H, dk, dv, chunk=64, dtype=None, seg_len=0):
    """Device workspace bytes of a prefill on the automatic plan (seg_len 0) or with explicit
    segments of seg_len tokens."""
    torch = _torch()
    code = _dtype_code(dtype or torch.bfloat16)
    lib = _lib.load()
    if seg_len == 0:
        return int(lib.kda_chunk_prefill_workspace_bytes(B, T, H, dk, dv, chunk, code))
    return int(lib.kda_chunk_prefill_workspace_bytes_ex(B, T, H, dk, dv, chunk, code, seg_len))


def chunk_prefill(q, k, v, log_alpha, beta, S0=None, chunk=64, *, seg_len=0, n_vs=0,
                  o=None, S_T=None, return_state=True, workspace=None):
    """Chunked KDA prefill.  Returns (o, S_T); S_T is None when return_state is False.

    ``S_T`` may be passed as ``S0`` itself to update the state in place.
    ``seg_len`` / ``n_vs`` force a sequence-split plan (0 = the library's choice).
    """
    o, S_T, _ = _prefill(q, k, v, log_alpha, beta, S0, chunk, seg_len, n_vs, o, S_T,
                         return_state, workspace, 0, None)
    return o, S_T


def chunk_prefill_ckpt(q, k, v, log_alpha, beta, S0=None, chunk=64, *, ckpt_every, seg_len=0,
                       n_vs=0, o=None, S_T=None, S_ckpt=None, return_state=True, workspace=None):
    """chunk_prefill that also returns state checkpoints for prefix reuse.

    Returns (o, S_T, S_ckpt) with S_ckpt [B, T // ckpt_every, H, dk, dv]: the state after the
    first (i + 1) * ckpt_every tokens of each sequence.  ``ckpt_every`` is a positive multiple
    of ``chunk``.
    """
    return _prefill(q, k, v, log_alpha, beta, S0, chunk, seg_len, n_vs, o, S_T, return_state,
                    workspace, ckpt_every, S_ckpt)


def _prefill(q, k, v, log_alpha, beta, S0, chunk, seg_len, n_vs, o, S_T, return_state,
             workspace, ckpt_every, S_ckpt):
    torch = _torch()
    lib = _lib.load()
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("chunk_prefill runs on a HIP device; got a tensor on " + str(dev))
    code = _dtype_code(q.dtype)
    _check_tensor("q", q, q.dtype, (B, T, H, dk), dev)
    _check_tensor("k", k, q.dtype, (B, T, H, dk), dev)
    _check_tensor("v", v, q.dtype, (B, T, H, dv), dev)
    _check_tensor("log_alpha", log_alpha, torch.float32, (B, T, H, dk), dev)
    _check_tensor("beta", beta, torch.float32, (B, T, H), dev)
    if S0 is not None:
        _check_tensor("S0", S0, torch.float32, (B, H, dk, dv), dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    else:
        _check_tensor("o", o, q.dtype, (B, T, H, dv), dev)
    if S_T is None and return_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif S_T is not None:
        _check_tensor("S_T", S_T, torch.float32, (B, H, dk, dv), dev)
    need = prefill_workspace_bytes(B, T, H, dk, dv, chunk, q.dtype, seg_len)
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if ckpt_every:
        n_ckpt = T // ckpt_every if ckpt_every > 0 else 0
        if S_ckpt is None:
            S_ckpt = torch.empty((B, n_ckpt, H, dk, dv), dtype=torch.float32, device=dev)
        else:
            _check_tensor("S_ckpt", S_ckpt, torch.float32, (B, n_ckpt, H, dk, dv), dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.kda_chunk_prefill_ckpt(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                    _ptr(S0), _ptr(o), _ptr(S_T), B, T, H, dk, dv, chunk, code,
                                    int(ckpt_every), _ptr(S_ckpt), seg_len, n_vs,
                                    _ptr(workspace), ws_bytes, ctypes.c_void_p(stream))
    _lib.check(st, "kda_chunk_prefill")
    return o, S_T, S_ckpt


def decode_step(q, k, v, log_alpha, beta, S, *, o=None):
    """One KDA decode step for [N, H, ...] inputs; updates S in place and returns o."""
    torch = _torch()
    lib = _lib.load()
    if q.dim() != 3:
        raise ValueError("q must be [N, H, dk]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("decode_step runs on a HIP device; got a tensor on " + str(dev))
    code = _dtype_code(q.dtype)
    _check_tensor("q", q, q.dtype, (N, H, dk), dev)
    _check_tensor("k", k, q.dtype, (N, H, dk), dev)
    _check_tensor("v", v, q.dtype, (N, H, dv), dev)
    _check_tensor("log_alpha", log_alpha, torch.float32, (N, H, dk), dev)
    _check_tensor("beta", beta, torch.float32, (N, H), dev)
    _check_tensor("S", S, torch.float32, (N, H, dk, dv), dev)
    if o is None:
        o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    else:
        _check_tensor("o", o, q.dtype, (N, H, dv), dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S),
                             _ptr(o), N, H, dk, dv, code, ctypes.c_void_p(stream))
    _lib.check(st, "kda_decode_step")
    return o


def chunk_prefill_gate(q, k, v, gate, beta, S0=None, chunk=64, *, seg_len=0, n_vs=0, o=None,
                       S_T=None, return_state=True, workspace=None):
    """chunk_prefill with the bounded gate fused: ``gate`` [B, T, H, dk] (bf16) is the raw gate
    pre-activation x, and log alpha = -5 * sigmoid(x) is formed in the kernel.  bf16 inputs with
    dk == dv == 128 only.  Returns (o, S_T)."""
    torch = _torch()
    lib = _lib.load()
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("chunk_prefill_gate runs on a HIP device; got a tensor on " + str(dev))
    code = _dtype_code(q.dtype)
    for name, t, shape in (("q", q, (B, T, H, dk)), ("k", k, (B, T, H, dk)), ("v", v, (B, T, H, dv)),
                           ("gate", gate, (B, T, H, dk))):
        _check_tensor(name, t, q.dtype, shape, dev)
    _check_tensor("beta", beta, torch.float32, (B, T, H), dev)
    if S0 is not None:
        _check_tensor("S0", S0, torch.float32, (B, H, dk, dv), dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=dev)
    else:
        _check_tensor("o", o, q.dtype, (B, T, H, dv), dev)
    if S_T is None and return_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif S_T is not None:
        _check_tensor("S_T", S_T, torch.float32, (B, H, dk, dv), dev)
    need = prefill_workspace_bytes(B, T, H, dk, dv, chunk, q.dtype, seg_len)
    if need > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.kda_chunk_prefill_gate(_ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(S0),
                                    _ptr(o), _ptr(S_T), B, T, H, dk, dv, chunk, code, seg_len, n_vs,
                                    _ptr(workspace), ws_bytes, ctypes.c_void_p(stream))
    _lib.check(st, "kda_chunk_prefill_gate")
    return o, S_T


def chunk_prefill_noalloc(q, k, v, log_alpha, beta, S0=None, chunk=64, *, seg_len=0, n_vs=0, o,
                          S_T=None):
    """chunk_prefill through the allocation-free entry point: the caller passes the output
    tensors (o, and S_T or None), and a sequence split takes its scratch from the library's
    fixed device array instead of a workspace.  Allocates nothing.  Returns (o, S_T)."""
    torch = _torch()
    lib = _lib.load()
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("chunk_prefill_noalloc runs on a HIP device; got a tensor on " + str(dev))
    code = _dtype_code(q.dtype)
    _check_tensor("q", q, q.dtype, (B, T, H, dk), dev)
    _check_tensor("k", k, q.dtype, (B, T, H, dk), dev)
    _check_tensor("v", v, q.dtype, (B, T, H, dv), dev)
    _check_tensor("log_alpha", log_alpha, torch.float32, (B, T, H, dk), dev)
    _check_tensor("beta", beta, torch.float32, (B, T, H), dev)
    _check_tensor("o", o, q.dtype, (B, T, H, dv), dev)
    if S0 is not None:
        _check_tensor("S0", S0, torch.float32, (B, H, dk, dv), dev)
    if S_T is not None:
        _check_tensor("S_T", S_T, torch.float32, (B, H, dk, dv), dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.kda_chunk_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                       _ptr(S0), _ptr(o), _ptr(S_T), B, T, H, dk, dv, chunk, code,
                                       seg_len, n_vs, ctypes.c_void_p(stream))
    _lib.check(st, "kda_chunk_prefill_noalloc")
    return o, S_T


def _spec_inputs(q, k, v, log_alpha, beta, S, where):
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [N, m, H, dk]")
    N, m, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError(where + " runs on a HIP device; got a tensor on " + str(dev))
    _check_tensor("q", q, q.dtype, (N, m, H, dk), dev)
    _check_tensor("k", k, q.dtype, (N, m, H, dk), dev)
    _check_tensor("v", v, q.dtype, (N, m, H, dv), dev)
    _check_tensor("log_alpha", log_alpha, torch.float32, (N, m, H, dk), dev)
    _check_tensor("beta", beta, torch.float32, (N, m, H), dev)
    _check_tensor("S", S, torch.float32, (N, H, dk, dv), dev)
    return N, m, H, dk, dv, dev


def spec_verify(q, k, v, log_alpha, beta, S, *, o=None):
    """Outputs of m drafted tokens per sequence ([N, m, H, ...] inputs) from state S.

    S is not modified.  Returns o [N, m, H, dv]."""
    torch = _torch()
    lib = _lib.load()
    N, m, H, dk, dv, dev = _spec_inputs(q, k, v, log_alpha, beta, S, "spec_verify")
    if o is None:
        o = torch.empty((N, m, H, dv), dtype=q.dtype, device=dev)
    else:
        _check_tensor("o", o, q.dtype, (N, m, H, dv), dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.kda_spec_verify(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S),
                             _ptr(o), N, m, H, dk, dv, _dtype_code(q.dtype),
                             ctypes.c_void_p(stream))
    _lib.check(st, "kda_spec_verify")
    return o


def spec_commit(q, k, v, log_alpha, beta, S, accepted):
    """Advance S in place over the first accepted[n] of the m cached drafted tokens of each
    sequence (the inputs given to spec_verify).  ``accepted`` is an int32 device tensor [N]."""
    torch = _torch()
    lib = _lib.load()
    N, m, H, dk, dv, dev = _spec_inputs(q, k, v, log_alpha, beta, S, "spec_commit")
    _check_tensor("accepted", accepted, torch.int32, (N,), dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib.kda_spec_commit(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S),
                             _ptr(accepted), N, m, H, dk, dv, _dtype_code(q.dtype),
                             ctypes.c_void_p(stream))
    _lib.check(st, "kda_spec_commit")
