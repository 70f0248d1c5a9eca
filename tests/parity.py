"""Shared helpers for the device-vs-oracle parity tests.

Tolerances (stated for KDA in the benchmark definition): bf16 inputs with fp32
accumulation: rel-L2 <= 1e-2 and max-abs <= 3e-2 on o and S_T; fp32 inputs:
rel-L2 <= 1e-4.  For fp32 a max-abs bound is not stated; 1e-3 is used, about
ten times the rel-L2 bound scaled to the O(1) magnitudes of o and S here.
rel-L2 = ||x - y||_2 / ||y||_2 over the whole tensor, in float64.

For bf16 outputs the rounding floor is printed beside each comparison: the error
of the oracle's own output rounded to bf16 (the closest any bf16 result can be).
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


def bf16_round(y: np.ndarray) -> np.ndarray:
    """y rounded to bf16 (round to nearest even), back in float64."""
    return torch.from_numpy(np.ascontiguousarray(y, dtype=np.float64)).to(torch.bfloat16).double().numpy()


def bf16_floor(ref) -> tuple[float, float]:
    """(rel-L2, max-abs) of the bf16-rounded reference against the reference itself."""
    y = to_f64(ref)
    r = bf16_round(y)
    return rel_l2(r, y), max_abs(r, y)


def _is_bf16(t) -> bool:
    return isinstance(t, torch.Tensor) and t.dtype == torch.bfloat16


def assert_close(name, got, ref, dtype):
    rl, ma = TOL[dtype]
    g = to_f64(got)
    assert np.isfinite(g).all(), f"{name}: non-finite values"
    r = rel_l2(g, ref)
    m = max_abs(g, ref)
    floor = ""
    if _is_bf16(got):
        fr, fm = bf16_floor(ref)
        floor = f"; bf16 rounding floor {fr:.3e} / {fm:.3e}"
    print(f"    {name}: rel-L2 {r:.3e} max-abs {m:.3e} ({dtype}){floor}", flush=True)
    assert r <= rl and m <= ma, f"{name}: rel-L2 {r:.3e} (<= {rl}) max-abs {m:.3e} (<= {ma})"
    return r, m


class Accum:
    """rel-L2 and max-abs over a whole tensor compared piece by piece (float64 sums), with the
    worst rel-L2 of any single piece and, for bf16 outputs, the bf16 rounding floor."""

    def __init__(self, name, dtype):
        self.name, self.dtype = name, dtype
        self.num = self.den = self.fnum = 0.0
        self.max_abs = self.fmax = 0.0
        self.worst = 0.0
        self.worst_at = None
        self.pieces = 0
        self.bf16 = False

    def add(self, got, ref, where=None):
        """Compare one piece: got (a tensor, any device) against ref (float64 array or tensor).
        The sums are taken with torch on the host in float64 (multi-threaded)."""
        bf = _is_bf16(got)
        g = (got.detach().cpu() if isinstance(got, torch.Tensor) else torch.from_numpy(np.asarray(got))).double()
        y = ref if isinstance(ref, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(ref, dtype=np.float64))
        y = y.detach().cpu().double()
        assert g.shape == y.shape, (g.shape, y.shape)
        assert bool(torch.isfinite(g).all()), f"{self.name} {where}: non-finite values"
        d = g - y
        n = float((d * d).sum())
        den = float((y * y).sum())
        self.num += n
        self.den += den
        self.max_abs = max(self.max_abs, float(d.abs().max()) if d.numel() else 0.0)
        r = (n / den) ** 0.5 if den > 0 else n ** 0.5
        if r > self.worst:
            self.worst, self.worst_at = r, where
        if bf:
            self.bf16 = True
            fd = y.to(torch.bfloat16).double() - y
            self.fnum += float((fd * fd).sum())
            self.fmax = max(self.fmax, float(fd.abs().max()) if fd.numel() else 0.0)
        self.pieces += 1

    def rel_l2(self) -> float:
        return (self.num / self.den) ** 0.5 if self.den > 0 else self.num ** 0.5

    def check(self):
        rl, ma = TOL[self.dtype]
        r = self.rel_l2()
        floor = ""
        if self.bf16:
            fr = (self.fnum / self.den) ** 0.5 if self.den > 0 else 0.0
            floor = f"; bf16 rounding floor {fr:.3e} / {self.fmax:.3e}"
        print(f"    {self.name}: rel-L2 {r:.3e} max-abs {self.max_abs:.3e} over {self.pieces} pieces "
              f"(worst piece {self.worst:.3e} at {self.worst_at}) ({self.dtype}){floor}", flush=True)
        assert r <= rl and self.max_abs <= ma, \
            f"{self.name}: rel-L2 {r:.3e} (<= {rl}) max-abs {self.max_abs:.3e} (<= {ma})"
        assert self.worst <= rl, f"{self.name}: piece {self.worst_at} rel-L2 {self.worst:.3e} (<= {rl})"
        return r, self.max_abs


def nan_like(t):
    """A tensor of t's shape, dtype and device filled with NaN (an output buffer whose every
    element must be written for a comparison to pass)."""
    return torch.full_like(t, float("nan"))


def to_device(d, device="cuda"):
    return {k: (None if v is None else v.to(device)) for k, v in d.items()}
