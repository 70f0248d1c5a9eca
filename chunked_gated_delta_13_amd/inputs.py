"""Seeded synthetic inputs for KDA prefill and decode.

This module only draws random numbers and casts them; it holds none of the KDA
arithmetic.  Both the device path and the float64 oracle are fed from it, so
that they see bit-identical values.

Recipe (q, k, v, beta, log_alpha, S0 are drawn in that fixed order from one
``torch.Generator`` seeded per workload):

* q, k ~ N(0, 1), L2-normalised per token in fp32, then cast to the input dtype;
* v ~ N(0, 1), cast to the input dtype;
* beta = sigmoid(N(0, 1)), fp32, one scalar per token and head;
* log_alpha, fp32, one value per token, head and key channel:
    - ``"sig1"``: -5 * sigmoid(N(0, 1));
    - ``"sig2"``: -5 * sigmoid(N(0, 2))  (N(0, 2) read as standard deviation 2);
    - ``"slow"``: -0.05 * sigmoid(N(0, 1))  (long memory; exercises hand-off);
  optionally a fraction ``bound_frac`` of tokens (Bernoulli per (b, t, h)) get
  log_alpha ~ U[-5, -4.95] on every channel, and 1% of those exactly -5;
* S0 ~ N(0, s0_std^2) in fp32, or zeros when ``s0_std`` is 0.

The decay bound log alpha in [-5, 0] and the 1M-token context come from the
pages ("Inside Kimi K3", sequence paragraph; "Kimi K3's architecture", section
"A lower bound that deleted a GPU code path").
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    chunk: int
    dtype: str            # "bf16" or "f32": dtype of q, k, v and o
    decay: str            # "sig1" | "sig2" | "slow"
    s0_std: float
    seed: int
    bound_frac: float = 0.0
    segment: int = 0      # sequence-split segment length (0: library's own plan)
    note: str = ""


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    N: int
    H: int
    dk: int
    dv: int
    dtype: str
    decay: str
    s0_std: float
    seed: int
    steps: int = 1
    note: str = field(default="")


# The five workloads of the benchmark definition plus correctness-only sets.
WORKLOADS = {
    "tiny_f32": PrefillWorkload("tiny_f32", 1, 256, 1, 64, 64, 16, "f32", "sig1", 0.0, 0,
                                note="B1 H1 T256 d64 chunk16 fp32"),
    "small_bf16": PrefillWorkload("small_bf16", 1, 4096, 8, 128, 128, 64, "bf16", "sig2",
                                  0.02, 1, note="B1 H8 T4096 d128 chunk64 bf16"),
    "model_width": PrefillWorkload("model_width", 4, 32768, 56, 128, 128, 64, "bf16", "sig2",
                                   0.02, 2, note="B4 H56 T32768 d128 chunk64 bf16 (7168 hidden)"),
    "long_1m": PrefillWorkload("long_1m", 1, 1 << 20, 16, 128, 128, 64, "bf16", "sig2", 0.02, 3,
                               bound_frac=0.1, segment=1 << 16,
                               note="B1 H16 T1048576 d128 bf16, 64K-token segments"),
    "slow_bf16": PrefillWorkload("slow_bf16", 1, 4096, 2, 128, 128, 64, "bf16", "slow", 1.0, 5,
                                 note="correctness only: long memory"),
    "mixed_bf16": PrefillWorkload("mixed_bf16", 1, 8192, 2, 128, 128, 64, "bf16", "slow", 1.0, 6,
                                  bound_frac=0.1, segment=1024,
                                  note="correctness only: long memory + 10% tokens at the bound"),
}

DECODE_WORKLOADS = {
    "decode_n256": DecodeWorkload("decode_n256", 256, 56, 128, 128, "bf16", "sig2", 0.02, 4,
                                  steps=1000, note="256 sequences x 56 heads, 1000 steps"),
}

@dataclass(frozen=True)
class SpecWorkload:
    """Speculative decoding: m drafted tokens per sequence, verified then partly committed."""
    name: str
    N: int
    m: int
    H: int
    dk: int
    dv: int
    dtype: str
    decay: str
    s0_std: float
    seed: int
    note: str = ""


# Decode-shaped batch (256 sequences x 56 heads) with 4 drafted tokens per step; the accepted
# count of each sequence is uniform on {0, ..., m}.  The pages give no draft length; 4 is a
# common setting for one drafted block.
SPEC_WORKLOADS = {
    "spec_n256_m4": SpecWorkload("spec_n256_m4", 256, 4, 56, 128, 128, "bf16", "sig2", 0.02, 7,
                                 note="256 sequences x 56 heads, 4 drafted tokens per step"),
}

_TORCH_DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPES[name]


def _normal(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _log_alpha(shape_tok, dk, decay, bound_frac, gen, device):
    z = _normal(shape_tok + (dk,), gen, device)
    if decay == "sig1":
        la = -5.0 * torch.sigmoid(z)
    elif decay == "sig2":
        la = -5.0 * torch.sigmoid(2.0 * z)
    elif decay == "slow":
        la = -0.05 * torch.sigmoid(z)
    else:
        raise ValueError(f"unknown decay recipe {decay!r}")
    if bound_frac > 0.0:
        pick = torch.rand(shape_tok, generator=gen, device=device) < bound_frac
        near = -5.0 + 0.05 * torch.rand(shape_tok + (dk,), generator=gen, device=device)
        exact = torch.rand(shape_tok, generator=gen, device=device) < 0.01
        near = torch.where(exact[..., None], torch.full_like(near, -5.0), near)
        la = torch.where(pick[..., None], near, la)
    return la.contiguous()


def _unit_rows(x):
    return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-30)


def make_prefill_inputs(B, T, H, dk, dv, dtype="bf16", decay="sig2", s0_std=0.02, seed=0,
                        bound_frac=0.0, device="cpu"):
    """Return a dict with q, k, v, log_alpha, beta, S0 (S0 is None when s0_std == 0)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    dt = torch_dtype(dtype)
    q = _unit_rows(_normal((B, T, H, dk), gen, device)).to(dt).contiguous()
    k = _unit_rows(_normal((B, T, H, dk), gen, device)).to(dt).contiguous()
    v = _normal((B, T, H, dv), gen, device).to(dt).contiguous()
    beta = torch.sigmoid(_normal((B, T, H), gen, device)).contiguous()
    la = _log_alpha((B, T, H), dk, decay, bound_frac, gen, device)
    S0 = None
    if s0_std > 0.0:
        S0 = (s0_std * _normal((B, H, dk, dv), gen, device)).contiguous()
    return {"q": q, "k": k, "v": v, "log_alpha": la, "beta": beta, "S0": S0}


def make_stress_inputs(B, T, H, d, dtype="bf16", seed=0, beta_lo=0.0, beta_hi=2.0, group=16,
                       noise=0.05, decay="slow", s0_std=1.0, device="cpu"):
    """Inputs that stress the intra-chunk triangular solve: the keys of every `group`
    consecutive tokens (per sequence and head) are near-parallel, each the unit vector of
    u + noise * z with one shared u ~ N(0, I) per group and z ~ N(0, I / d) per token (cosine of
    two keys of a group about 1 - noise^2), and beta ~ U[beta_lo, beta_hi].  With unit keys and
    beta in [0, 2] every token's transition is still a contraction, but the unit lower-triangular
    system of a chunk then has off-diagonal entries near beta, far from the identity.
    Drawn in the order q, u, z, v, beta, log_alpha, S0; the rest as make_prefill_inputs."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    dt = torch_dtype(dtype)
    q = _unit_rows(_normal((B, T, H, d), gen, device)).to(dt).contiguous()
    ng = (T + group - 1) // group
    u = _normal((B, ng, H, d), gen, device)
    u = u / torch.linalg.vector_norm(u, dim=-1, keepdim=True).clamp_min(1e-30)
    z = _normal((B, T, H, d), gen, device) / (d ** 0.5)
    base = u.repeat_interleave(group, dim=1)[:, :T]
    k = _unit_rows(base + noise * z).to(dt).contiguous()
    v = _normal((B, T, H, d), gen, device).to(dt).contiguous()
    beta = (beta_lo + (beta_hi - beta_lo) * torch.rand((B, T, H), generator=gen, device=device)).contiguous()
    la = _log_alpha((B, T, H), d, decay, 0.0, gen, device)
    S0 = None
    if s0_std > 0.0:
        S0 = (s0_std * _normal((B, H, d, d), gen, device)).contiguous()
    return {"q": q, "k": k, "v": v, "log_alpha": la, "beta": beta, "S0": S0}


def workload_inputs(w: PrefillWorkload, device="cpu", T: int | None = None,
                    B: int | None = None, H: int | None = None):
    """Inputs of a named workload, optionally with a smaller B, T or H (same recipe)."""
    return make_prefill_inputs(B or w.B, T or w.T, H or w.H, w.dk, w.dv, w.dtype, w.decay,
                               w.s0_std, w.seed, w.bound_frac, device)


def make_decode_inputs(N, H, dk, dv, dtype="bf16", decay="sig2", seed=0, device="cpu"):
    """One decode step's token inputs: q, k [N, H, dk], v [N, H, dv], log_alpha, beta."""
    d = make_prefill_inputs(N, 1, H, dk, dv, dtype, decay, 0.0, seed, 0.0, device)
    return {"q": d["q"][:, 0].contiguous(), "k": d["k"][:, 0].contiguous(),
            "v": d["v"][:, 0].contiguous(), "log_alpha": d["log_alpha"][:, 0].contiguous(),
            "beta": d["beta"][:, 0].contiguous()}


def make_state(N, H, dk, dv, s0_std=0.02, seed=0, device="cpu"):
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return (s0_std * _normal((N, H, dk, dv), gen, device)).contiguous()


def make_spec_inputs(N, m, H, dk, dv, dtype="bf16", decay="sig2", seed=0, device="cpu"):
    """One drafted block: q, k [N, m, H, dk], v [N, m, H, dv], log_alpha, beta [N, m, H], and
    accepted [N] (int32, uniform on {0, ..., m}), drawn after the token inputs."""
    d = make_prefill_inputs(N, m, H, dk, dv, dtype, decay, 0.0, seed, 0.0, device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) + 7919)
    acc = torch.randint(0, m + 1, (N,), generator=gen, device=device, dtype=torch.int64)
    return {"q": d["q"], "k": d["k"], "v": d["v"], "log_alpha": d["log_alpha"], "beta": d["beta"],
            "accepted": acc.to(torch.int32).contiguous()}


def make_gate(B, T, H, dk, dtype="bf16", seed=0, device="cpu"):
    """Raw gate pre-activation x ~ N(0, 2) (standard deviation 2), cast to the input dtype, so
    that -5 * sigmoid(x) has the distribution of the "sig2" log-decay recipe."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) + 104729)
    return (2.0 * _normal((B, T, H, dk), gen, device)).to(torch_dtype(dtype)).contiguous()
