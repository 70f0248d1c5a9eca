"""Shared helpers for the device-vs-oracle parity tests.

Tolerances (stated for KDA in the benchmark definition): bf16 inputs with fp32
accumulation: rel-L2 <= 1e-2 and max-abs <= 3e-2 on o and S_T; fp32 inputs:
rel-L2 <= 1e-4.  For fp32 a max-abs bound is not stated; 1e-3 is used, about
ten times the rel-L2 bound scaled to the O(1) magnitudes of o and S here.
rel-L2 = ||x - y||_2 / ||y||_2 over the whole tensor, in float64.
"""
from __future__ import annotations

import numpy as np
import torch

TOL = {"bf16": (1e-2, 3e-2), "f32": (1e-4, 1e-3)}


def to_f64(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().float().cpu().double().numpy()


def rel_l2(x, y) -> float:
    x, y = to_f64(x), to_f64(y)
    den = np.linalg.norm(y)
    return float(np.linalg.norm(x - y) / (den if den > 0 else 1.0))


def max_abs(x, y) -> float:
    x, y = to_f64(x), to_f64(y)
    return float(np.max(np.abs(x - y))) if x.size else 0.0


def assert_close(name, got, ref, dtype):
    rl, ma = TOL[dtype]
    g = to_f64(got)
    assert np.isfinite(g).all(), f"{name}: non-finite values"
    r = rel_l2(g, ref)
    m = max_abs(g, ref)
    print(f"    {name}: rel-L2 {r:.3e} max-abs {m:.3e} ({dtype})", flush=True)
    assert r <= rl and m <= ma, f"{name}: rel-L2 {r:.3e} (<= {rl}) max-abs {m:.3e} (<= {ma})"
    return r, m


def to_device(d, device="cuda"):
    return {k: (None if v is None else v.to(device)) for k, v in d.items()}
