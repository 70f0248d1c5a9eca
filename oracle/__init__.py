"""KDA oracle: float64 CPU token-by-token recurrence (ctypes wrapper over kda_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP library and never imports it.

The recurrence (see the header of ``kda_oracle.c`` for the page citations):

    S' = Diag(exp(clamp(log_alpha_t, -5, 0))) S
    e  = v_t - S'^T k_t
    S  = S' + beta_t k_t e^T
    o_t = S^T q_t

Inputs are widened to float64 before the call, so the oracle sees exactly the
values (bf16 or fp32) that a device path receives.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = True, sanitized_out: str | None = None) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math).  With sanitized_out, build a copy
    at that path under AddressSanitizer and UndefinedBehaviorSanitizer instead."""
    if sanitized_out:
        cmd = ["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
               "-Wall", "-Wextra", "-o", sanitized_out, _SRC, "-lm"]
        subprocess.check_call(cmd)
        return sanitized_out
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.kda_oracle_prefill.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp,
                                           ctypes.c_long, ctypes.c_long, ctypes.c_long,
                                           ctypes.c_long, ctypes.c_long, ctypes.c_long,
                                           ctypes.c_int]
        lib.kda_oracle_prefill.restype = ctypes.c_int
        lib.kda_oracle_version.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    if hasattr(x, "detach"):  # a torch tensor: widen on the host
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def prefill(q, k, v, log_alpha, beta, S0=None, nthreads: int | None = None,
            col_block: int = 32):
    """Run the recurrence over a whole batch.

    q, k, log_alpha: [B, T, H, dk]; v: [B, T, H, dv]; beta: [B, T, H];
    S0: [B, H, dk, dv] or None.  Returns (o [B, T, H, dv], S_T [B, H, dk, dv]),
    both float64 numpy arrays.
    """
    q, k, v, la, bt = (_f64(x) for x in (q, k, v, log_alpha, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or la.shape != q.shape:
        raise ValueError("q, k and log_alpha must share the shape [B, T, H, dk]")
    if v.shape[:3] != (B, T, H) or bt.shape != (B, T, H):
        raise ValueError("v must be [B, T, H, dv] and beta [B, T, H]")
    s0 = None
    if S0 is not None:
        s0 = _f64(S0)
        if s0.shape != (B, H, dk, dv):
            raise ValueError("S0 must be [B, H, dk, dv]")
    o = np.empty((B, T, H, dv), dtype=np.float64)
    st = np.empty((B, H, dk, dv), dtype=np.float64)
    rc = _load().kda_oracle_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(bt), _ptr(s0),
                                    _ptr(o), _ptr(st), B, T, H, dk, dv, col_block,
                                    nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"kda_oracle_prefill failed with code {rc}")
    return o, st


def decode_step(q, k, v, log_alpha, beta, S, nthreads: int | None = None):
    """One decode step: exactly one token of the recurrence with S in and out.

    q, k, log_alpha: [N, H, dk]; v: [N, H, dv]; beta: [N, H]; S: [N, H, dk, dv].
    Returns (o [N, H, dv], S_new [N, H, dk, dv]) as float64 numpy arrays.
    """
    q, k, v, la, bt, s = (_f64(x) for x in (q, k, v, log_alpha, beta, S))
    o, st = prefill(q[:, None], k[:, None], v[:, None], la[:, None], bt[:, None], s,
                    nthreads=nthreads)
    return o[:, 0], st


def spec_verify(q, k, v, log_alpha, beta, S, nthreads: int | None = None):
    """Speculative decoding, verify step: the outputs of m drafted tokens per sequence, run
    from the state S, with S itself left as it was.

    Source: "Kimi K3's architecture" (orkas.ai), section "The bill comes due in the serving
    stack": the state is updated in place, so a rejected draft cannot be undone; the projected
    inputs are kept and the state is rebuilt from them.  Verifying is therefore the recurrence
    over the m drafted tokens from S, with its final state discarded.

    q, k, log_alpha: [N, m, H, dk]; v: [N, m, H, dv]; beta: [N, m, H]; S: [N, H, dk, dv].
    Returns o [N, m, H, dv] (float64).
    """
    o, _ = prefill(q, k, v, log_alpha, beta, S, nthreads=nthreads)
    return o


def spec_commit(q, k, v, log_alpha, beta, S, accepted, nthreads: int | None = None):
    """Speculative decoding, commit step: the state after the first accepted[n] drafted tokens
    of sequence n, rebuilt from the kept inputs (same source as spec_verify).  Counts outside
    [0, m] are clamped.  Returns S_new [N, H, dk, dv] (float64); S is not modified."""
    q, k, v, la, bt, s = (_f64(x) for x in (q, k, v, log_alpha, beta, S))
    acc = np.asarray(accepted.detach().cpu() if hasattr(accepted, "detach") else accepted)
    N, m = q.shape[:2]
    out = np.empty_like(s)
    for n in range(N):
        a = int(min(max(int(acc[n]), 0), m))
        _, st = prefill(q[n:n + 1, :a], k[n:n + 1, :a], v[n:n + 1, :a], la[n:n + 1, :a],
                        bt[n:n + 1, :a], s[n:n + 1], nthreads=nthreads)
        out[n] = st[0]
    return out


def prefill_ckpt(q, k, v, log_alpha, beta, S0, ckpt_every, nthreads: int | None = None):
    """The recurrence with state checkpoints for prefix reuse: returns (o, S_T, S_ckpt) where
    S_ckpt[b, i] is the state after the first (i + 1) * ckpt_every tokens (i < T // ckpt_every),
    shaped [B, T // ckpt_every, H, dk, dv].

    Source: "Kimi K3's architecture" (orkas.ai), section "The bill comes due in the serving
    stack": a prefix-cache hit needs the recurrent state restorable at the same boundary as the
    cached token pages, so the state is checkpointed at a sparse subset of the 512-token hash
    endpoints.  The run is taken piece by piece between consecutive checkpoint positions, each
    piece starting from the state the previous one ended in.
    """
    q, k, v, la, bt = (_f64(x) for x in (q, k, v, log_alpha, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    s = np.zeros((B, H, dk, dv)) if S0 is None else _f64(S0)
    n = T // ckpt_every
    o = np.empty((B, T, H, dv))
    ck = np.empty((B, n, H, dk, dv))
    bounds = [i * ckpt_every for i in range(n + 1)] + ([T] if n * ckpt_every < T else [])
    for i in range(len(bounds) - 1):
        a, e = bounds[i], bounds[i + 1]
        o[:, a:e], s = prefill(q[:, a:e], k[:, a:e], v[:, a:e], la[:, a:e], bt[:, a:e], s,
                               nthreads=nthreads)
        if i < n:
            ck[:, i] = s
    return o, s, ck


def gate_log_alpha(gate):
    """The bounded decay curve log alpha = -5 * sigmoid(x) of a raw gate pre-activation x, in
    float64 (written as -5 / (1 + exp(-x)), stable for large |x|).

    Sources: "Inside Kimi K3" (academa.ai lecture), sequence paragraph: the decay curve itself is
    changed so that the log-decay is bounded below at -5; "Kimi K3's architecture" (orkas.ai),
    section "A lower bound that deleted a GPU code path": the activation has to be bounded
    below.  The pages do not print the curve; -5 * sigmoid is the reading used, the one the
    benchmark workloads draw log alpha from.
    """
    x = _f64(gate)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = -5.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = -5.0 * e / (1.0 + e)
    return out


def prefill_gate(q, k, v, gate, beta, S0=None, nthreads: int | None = None):
    """The recurrence with the fused bounded gate: log alpha = gate_log_alpha(gate)."""
    return prefill(q, k, v, gate_log_alpha(gate), beta, S0, nthreads=nthreads)
