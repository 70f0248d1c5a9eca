"""Device path vs the float64 oracle, element by element, on seeded inputs.

Sizes are small enough for the oracle to finish in seconds while spanning
several chunks, several 16-token tiles and a ragged tail.  Every call goes
through the C ABI of libkda.so (via the ctypes binding).
"""
import os

import numpy as np
import pytest
import torch

import oracle
from chunked_gated_delta_13_amd import inputs as gen
from tests.parity import TOL, assert_close, nan_like, to_device, to_f64

pytestmark = pytest.mark.gpu


def _kda():
    import chunked_gated_delta_13_amd as kda
    kda.load_library()
    return kda


def _run_prefill(inp, chunk, seg_len=0, n_vs=0, inplace=False):
    """Prefill through the C ABI into output buffers that start as NaN (S_T = S0 when in place)."""
    kda = _kda()
    d = to_device(inp)
    S0 = d["S0"]
    B, T, H, _ = d["q"].shape
    dk, dv = d["q"].shape[-1], d["v"].shape[-1]
    o = nan_like(d["v"])
    if inplace:
        assert S0 is not None
        st = S0
    else:
        st = torch.full((B, H, dk, dv), float("nan"), dtype=torch.float32, device="cuda")
    kda.chunk_prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], S0, chunk=chunk,
                      seg_len=seg_len, n_vs=n_vs, o=o, S_T=st)
    torch.cuda.synchronize()
    return o, st


def _oracle(inp):
    return oracle.prefill(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["S0"])


def _case(B, T, H, d, dtype, decay="sig2", s0=0.02, seed=0, bound_frac=0.0):
    return gen.make_prefill_inputs(B, T, H, d, d, dtype, decay, s0, seed, bound_frac, "cpu")


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_step_matches_oracle(dtype, d):
    kda = _kda()
    print(f"decode dtype={dtype} d={d}", flush=True)
    N, H = 5, 3
    tok = gen.make_decode_inputs(N, H, d, d, dtype, "sig2", seed=11, device="cpu")
    S = gen.make_state(N, H, d, d, 1.0, seed=12, device="cpu")
    dv = to_device(tok)
    Sd = S.cuda()
    o = kda.decode_step(dv["q"], dv["k"], dv["v"], dv["log_alpha"], dv["beta"], Sd, o=nan_like(dv["v"]))
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.decode_step(tok["q"], tok["k"], tok["v"], tok["log_alpha"], tok["beta"], S)
    assert_close("o", o, o_ref, dtype)
    assert_close("S", Sd, s_ref, dtype)


def test_decode_many_steps_matches_oracle():
    kda = _kda()
    N, H, d, steps = 4, 3, 128, 40
    S = gen.make_state(N, H, d, d, 0.02, seed=13, device="cpu")
    Sd = S.cuda()
    S_ref = to_f64(S)
    for step in range(steps):
        tok = gen.make_decode_inputs(N, H, d, d, "bf16", "sig2", seed=1000 + step, device="cpu")
        dv = to_device(tok)
        o = kda.decode_step(dv["q"], dv["k"], dv["v"], dv["log_alpha"], dv["beta"], Sd, o=nan_like(dv["v"]))
        o_ref, S_ref = oracle.decode_step(tok["q"], tok["k"], tok["v"], tok["log_alpha"],
                                          tok["beta"], S_ref)
        torch.cuda.synchronize()
        assert_close(f"o step {step}", o, o_ref, "bf16")
    assert_close("S after steps", Sd, S_ref, "bf16")


def test_decode_equals_prefill_of_one_token():
    kda = _kda()
    N, H, d = 3, 2, 128
    inp = _case(N, 1, H, d, "bf16", s0=0.5, seed=14)
    dv = to_device(inp)
    S = dv["S0"].clone()
    o_dec = kda.decode_step(dv["q"][:, 0].contiguous(), dv["k"][:, 0].contiguous(),
                            dv["v"][:, 0].contiguous(), dv["log_alpha"][:, 0].contiguous(),
                            dv["beta"][:, 0].contiguous(), S)
    o_pf, st = kda.chunk_prefill(dv["q"], dv["k"], dv["v"], dv["log_alpha"], dv["beta"], dv["S0"],
                                 chunk=16)
    torch.cuda.synchronize()
    assert_close("o", o_dec, o_pf[:, 0], "bf16")
    assert_close("S", S, st, "bf16")


# ----------------------------------------------------------------- prefill
def test_prefill_tiny_fp32_workload():
    """B1 H1 T256 d64, chunk 16, fp32 everywhere, S0 = 0, seed 0."""
    w = gen.WORKLOADS["tiny_f32"]
    inp = gen.workload_inputs(w)
    o, st = _run_prefill(inp, w.chunk)
    o_ref, s_ref = _oracle(inp)
    assert_close("o", o, o_ref, "f32")
    assert_close("S_T", st, s_ref, "f32")


CASES = [
    # (B, T, H, d, dtype, chunk)
    (1, 200, 2, 64, "f32", 16),
    (1, 200, 2, 64, "f32", 32),
    (2, 77, 3, 128, "f32", 32),
    (1, 300, 2, 128, "bf16", 64),
    (2, 130, 3, 128, "bf16", 32),
    (1, 250, 2, 128, "bf16", 16),
    (2, 129, 2, 64, "bf16", 64),
    (1, 1, 2, 128, "bf16", 64),
    (1, 15, 1, 128, "bf16", 64),
    (1, 33, 1, 64, "f32", 16),
    (1, 200, 2, 64, "f32", 64),     # fp32 with 64-token chunks (run as 32-token chunks)
    (2, 77, 3, 128, "f32", 64),
    (1, 1, 1, 128, "f32", 64),
]


@pytest.mark.parametrize("B,T,H,d,dtype,chunk", CASES)
def test_prefill_matches_oracle(B, T, H, d, dtype, chunk):
    print(f"prefill B={B} T={T} H={H} d={d} {dtype} chunk={chunk}", flush=True)
    inp = _case(B, T, H, d, dtype, seed=T + d + chunk)
    o, st = _run_prefill(inp, chunk)
    o_ref, s_ref = _oracle(inp)
    assert_close("o", o, o_ref, dtype)
    assert_close("S_T", st, s_ref, dtype)


@pytest.mark.parametrize("dtype,chunk", [("bf16", 64), ("f32", 32)])
def test_prefill_slow_decay_long_memory(dtype, chunk):
    """log alpha ~ -0.05 sigmoid, S0 ~ N(0, 1): S0 and early chunks matter at the end."""
    inp = _case(1, 1000, 2, 128, dtype, decay="slow", s0=1.0, seed=21)
    o, st = _run_prefill(inp, chunk)
    o_ref, s_ref = _oracle(inp)
    assert_close("o", o, o_ref, dtype)
    assert_close("S_T", st, s_ref, dtype)


@pytest.mark.parametrize("fill", [-5.0, 0.0, -100.0])
def test_prefill_decay_extremes(fill):
    """All log alpha at the bound (tile reciprocal exactly e^80), at 0, or clamped from -100."""
    inp = _case(1, 160, 2, 128, "bf16", s0=1.0, seed=22)
    inp["log_alpha"] = torch.full_like(inp["log_alpha"], fill)
    o, st = _run_prefill(inp, 64)
    o_ref, s_ref = _oracle(inp)
    assert_close("o", o, o_ref, "bf16")
    assert_close("S_T", st, s_ref, "bf16")


def test_prefill_mixed_bound_tokens():
    inp = _case(1, 700, 2, 128, "bf16", decay="slow", s0=1.0, seed=23, bound_frac=0.1)
    o, st = _run_prefill(inp, 64)
    o_ref, s_ref = _oracle(inp)
    assert_close("o", o, o_ref, "bf16")
    assert_close("S_T", st, s_ref, "bf16")


@pytest.mark.parametrize("dtype,chunk,seg", [("bf16", 64, 256), ("bf16", 32, 192), ("f32", 16, 128),
                                             ("bf16", 64, 512), ("bf16", 64, 384), ("f32", 32, 512),
                                             ("f32", 64, 256)])
def test_prefill_sequence_split_matches_oracle(dtype, chunk, seg):
    """Segment 0 from S0 beside the transition pass and the zero-start runs of the later
    segments, prefix scan, rerun from entry states.  T = 1000 gives 2 to 8 segments (2: no
    scan); slow decay keeps every transition alive, so this is the full two-pass split."""
    inp = _case(2, 1000, 2, 128 if dtype == "bf16" else 64, dtype, decay="slow", s0=1.0, seed=24)
    o, st = _run_prefill(inp, chunk, seg_len=seg)
    o_ref, s_ref = _oracle(inp)
    assert_close("o", o, o_ref, dtype)
    assert_close("S_T", st, s_ref, dtype)


@pytest.mark.parametrize("T,H", [(12288, 1), (13000, 1), (4096, 8)])
def test_prefill_automatic_split(T, H):
    """The automatic plan splits a sequence of a few thousand tokens over few heads into segments
    of equal length, the last one possibly shorter (13000 tokens: ragged)."""
    kda = _kda()
    seg, nvs = kda.prefill_plan(1, T, H, 128, 128, 64)
    assert nvs == 1 and seg < T and seg % 64 == 0
    n_seg = -(-T // seg)
    assert n_seg >= 3 and 0 < T - (n_seg - 1) * seg <= seg
    inp = _case(1, T, H, 128, "bf16", decay="slow", s0=1.0, seed=31)
    o, st = _run_prefill(inp, 64)
    o_ref, s_ref = _oracle(inp)
    assert_close("o", o, o_ref, "bf16")
    assert_close("S_T", st, s_ref, "bf16")


def test_prefill_split_from_two_host_threads():
    """Split prefills enqueued from two host threads at once, each on its own stream, share the
    library's side stream and fork/join events; each result equals the same call made alone."""
    import threading
    kda = _kda()
    cases = [to_device(_case(1, 4096, 2, 128, "bf16", decay="slow", s0=1.0, seed=s)) for s in (61, 62)]
    assert kda.prefill_plan(1, 4096, 2, 128, 128, 64)[0] < 4096   # the automatic plan splits
    refs = []
    for d in cases:
        o, st = kda.chunk_prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], chunk=64)
        refs.append((o, st))
    torch.cuda.synchronize()
    outs = [[], []]
    errors = []

    def run(i):
        try:
            stream = torch.cuda.Stream()
            d = cases[i]
            with torch.cuda.stream(stream):
                for _ in range(6):
                    outs[i].append(kda.chunk_prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                                                     d["S0"], chunk=64))
            stream.synchronize()
        except Exception as e:   # reported below, in the test's own thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in (0, 1)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in (0, 1):
        assert len(outs[i]) == 6
        for o, st in outs[i]:
            assert torch.equal(o, refs[i][0]) and torch.equal(st, refs[i][1])


def test_prefill_column_split_matches_unsplit():
    inp = _case(1, 300, 3, 128, "bf16", seed=25)
    o1, s1 = _run_prefill(inp, 64, n_vs=1)
    o2, s2 = _run_prefill(inp, 64, n_vs=2)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_prefill_split_one_pass_matches_two_pass():
    """With one column slice the transitions come from a pass shared with the increments; with
    two slices from a transition pass of their own, the increments from the zero-start pass.
    Both match the oracle and each other to the bf16 tolerance."""
    inp = _case(1, 900, 2, 128, "bf16", decay="slow", s0=1.0, seed=29)
    o1, s1 = _run_prefill(inp, 64, seg_len=192, n_vs=1)
    o2, s2 = _run_prefill(inp, 64, seg_len=192, n_vs=2)
    o_ref, s_ref = _oracle(inp)
    assert_close("o one pass", o1, o_ref, "bf16")
    assert_close("S_T one pass", s1, s_ref, "bf16")
    assert_close("o two passes", o2, o_ref, "bf16")
    assert_close("o one vs two passes", o1, to_f64(o2), "bf16")
    assert_close("S_T one vs two passes", s1, to_f64(s2), "bf16")


def test_prefill_in_place_state():
    inp = _case(2, 150, 2, 128, "bf16", s0=1.0, seed=26)
    o_ref, s_ref = _oracle(inp)
    o, st = _run_prefill(inp, 64, inplace=True)
    assert_close("o", o, o_ref, "bf16")
    assert_close("S_T", st, s_ref, "bf16")


@pytest.mark.parametrize("seg", [128, 320])
def test_prefill_in_place_state_with_split(seg):
    inp = _case(1, 600, 2, 128, "bf16", decay="slow", s0=1.0, seed=27)
    o_ref, s_ref = _oracle(inp)
    o, st = _run_prefill(inp, 64, seg_len=seg, inplace=True)
    assert_close("o", o, o_ref, "bf16")
    assert_close("S_T", st, s_ref, "bf16")


def test_prefill_zero_tokens_returns_initial_state():
    kda = _kda()
    inp = _case(2, 0, 3, 128, "bf16", s0=1.0, seed=28)
    d = to_device(inp)
    o, st = kda.chunk_prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"],
                              S_T=nan_like(d["S0"]))
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 3, 128)
    assert torch.equal(st, d["S0"])
    o, st = kda.chunk_prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], None,
                              S_T=nan_like(d["S0"]))
    torch.cuda.synchronize()
    assert torch.count_nonzero(st).item() == 0


def test_prefill_zero_initial_state_is_default():
    inp = _case(1, 100, 2, 128, "bf16", s0=0.0, seed=29)
    assert inp["S0"] is None
    o, st = _run_prefill(inp, 64)
    o_ref, s_ref = _oracle(inp)
    assert_close("o", o, o_ref, "bf16")
    assert_close("S_T", st, s_ref, "bf16")


def test_prefill_is_deterministic():
    inp = _case(2, 500, 3, 128, "bf16", seed=30)
    o1, s1 = _run_prefill(inp, 64)
    o2, s2 = _run_prefill(inp, 64)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_prefill_chunk_size_independence_on_device():
    inp = _case(1, 400, 2, 128, "bf16", decay="slow", s0=1.0, seed=31)
    o_ref, s_ref = _oracle(inp)
    for chunk in (16, 32, 64):
        o, st = _run_prefill(inp, chunk)
        assert_close(f"o chunk={chunk}", o, o_ref, "bf16")
        assert_close(f"S_T chunk={chunk}", st, s_ref, "bf16")


def test_prefill_small_bf16_workload():
    """B1 H8 T4096 d128, chunk 64, bf16 q/k/v, fp32 beta / log alpha, S0 ~ N(0, 0.02)."""
    w = gen.WORKLOADS["small_bf16"]
    inp = gen.workload_inputs(w)
    o, st = _run_prefill(inp, w.chunk)
    o_ref, s_ref = _oracle(inp)
    assert_close("o", o, o_ref, "bf16")
    assert_close("S_T", st, s_ref, "bf16")


def test_prefill_fp32_chunk64_matches_chunk32():
    """fp32 with chunk 64 runs as 32-token chunks: the same bits as chunk 32, and the fp32 bar
    against the oracle, on a long-memory sequence with a ragged tail and an automatic split."""
    inp = _case(1, 5000, 2, 128, "f32", decay="slow", s0=1.0, seed=33)
    for seg in (1 << 30, 1024):   # one pass; 1024-token segments (the same plan for both chunks)
        o64, s64 = _run_prefill(inp, 64, seg_len=seg, n_vs=2)
        o32, s32 = _run_prefill(inp, 32, seg_len=seg, n_vs=2)
        assert torch.equal(o64, o32) and torch.equal(s64, s32)
    o_ref, s_ref = _oracle(inp)
    o, st = _run_prefill(inp, 64)   # the automatic plan
    assert_close("o", o, o_ref, "f32")
    assert_close("S_T", st, s_ref, "f32")
    assert_close("o 1024-token segments", o64, o_ref, "f32")


# Solve stress.  Groups of near-parallel unit keys (cosine about 1 - noise^2) and beta ~ U[lo, hi]
# with slow decay, so that the decay does not damp the intra-chunk system: the unit
# lower-triangular (I + A) then has off-diagonal entries near beta instead of near 0.  For unit
# keys and beta in [0, 2] each token's transition is still a contraction.  Run through the two-role
# kernel (chunk 64, one slice), the single-role kernel (chunk 32, two column slices) and a split.
#
# Where keys are near-parallel and beta approaches 2 (each step close to a reflection), the result
# itself is ill-conditioned: one bf16-sized relative perturbation (2^-9) of the inputs moves it by
# sigma = 4e-3 .. 1.2e-2 (against about 2e-3 for the benchmark's inputs), and any method whose matrix
# products take bf16 operands derived from the keys inherits a multiple of that.  Those cases are
# held to rel-L2 <= max(1e-2, 4 sigma) and max-abs <= max(3e-2, 4 sigma max|ref|), sigma measured here
# with the oracle on the same inputs; the milder regimes keep the plain bar, and the fp32 mode keeps
# its plain bar on every case.
SIGMA_FACTOR = 4.0


def _sensitivity(inp, seed):
    """(rel-L2, max-abs) change of o and of S_T when q, k, v and beta are perturbed by relative
    noise uniform in [-2^-9, 2^-9] (one bf16 rounding), oracle against oracle."""
    rng = np.random.default_rng(seed)
    base = {k: to_f64(v) if v is not None else None for k, v in inp.items()}
    o0, s0 = oracle.prefill(base["q"], base["k"], base["v"], base["log_alpha"], base["beta"], base["S0"])
    p = dict(base)
    for key in ("q", "k", "v", "beta"):
        p[key] = base[key] * (1.0 + 2.0 ** -9 * rng.uniform(-1.0, 1.0, base[key].shape))
    o1, s1 = oracle.prefill(p["q"], p["k"], p["v"], p["log_alpha"], p["beta"], p["S0"])
    rel = lambda a, b: float(np.linalg.norm(a - b) / np.linalg.norm(b))  # noqa: E731
    return (rel(o1, o0), float(np.abs(o1 - o0).max())), (rel(s1, s0), float(np.abs(s1 - s0).max())), o0, s0


def _assert_within(name, got, ref, sens):
    rl, ma = TOL["bf16"]
    rl = max(rl, SIGMA_FACTOR * sens[0])
    ma = max(ma, SIGMA_FACTOR * sens[0] * float(np.abs(ref).max()))
    g = to_f64(got)
    assert np.isfinite(g).all()
    r = float(np.linalg.norm(g - ref) / np.linalg.norm(ref))
    m = float(np.abs(g - ref).max())
    print(f"    {name}: rel-L2 {r:.3e} max-abs {m:.3e}; sensitivity {sens[0]:.3e} / {sens[1]:.3e}; "
          f"bound {rl:.3e} / {ma:.3e}", flush=True)
    assert r <= rl and m <= ma, f"{name}: rel-L2 {r:.3e} (<= {rl:.3e}) max-abs {m:.3e} (<= {ma:.3e})"


STRESS = [
    # (T, H, group, noise, beta_lo, beta_hi, chunk, seg_len, n_vs, plain bar)
    (1000, 2, 1, 0.0, 0.0, 2.0, 64, 0, 1, True),       # beta in [0, 2], independent keys
    (2000, 2, 1, 0.0, 0.0, 2.0, 64, 256, 1, True),
    (1000, 2, 1, 0.0, 0.0, 2.0, 32, 0, 2, True),
    (1000, 2, 16, 0.05, 0.0, 1.0, 64, 0, 1, True),     # near-parallel keys, beta in [0, 1]
    (1000, 2, 16, 0.05, 0.0, 2.0, 64, 0, 1, False),    # near-parallel keys, beta up to 2
    (1000, 2, 64, 0.05, 0.0, 2.0, 64, 0, 1, False),
    (1000, 2, 16, 0.02, 1.5, 2.0, 64, 0, 1, False),
    (1000, 2, 8, 0.01, 1.9, 2.0, 64, 0, 1, False),
    (1000, 2, 16, 0.05, 0.0, 2.0, 32, 0, 2, False),
    (2000, 2, 16, 0.05, 0.0, 2.0, 64, 256, 1, False),
    (2000, 2, 64, 0.02, 1.0, 2.0, 64, 320, 1, False),
]


@pytest.mark.parametrize("T,H,group,noise,blo,bhi,chunk,seg,nvs,plain", STRESS)
def test_prefill_solve_stress(T, H, group, noise, blo, bhi, chunk, seg, nvs, plain):
    print(f"stress T={T} group={group} noise={noise} beta U[{blo},{bhi}] chunk={chunk} seg={seg}",
          flush=True)
    seed = T + group + int(100 * noise) + int(10 * blo)
    inp = gen.make_stress_inputs(1, T, H, 128, "bf16", seed=seed, beta_lo=blo, beta_hi=bhi,
                                 group=group, noise=noise)
    o, st = _run_prefill(inp, chunk, seg_len=seg, n_vs=nvs)
    so, ss, o_ref, s_ref = _sensitivity(inp, seed)
    if plain:
        print(f"    sensitivity o {so[0]:.3e}, S_T {ss[0]:.3e}", flush=True)
        assert_close("o", o, o_ref, "bf16")
        assert_close("S_T", st, s_ref, "bf16")
    else:
        _assert_within("o", o, o_ref, so)
        _assert_within("S_T", st, s_ref, ss)


@pytest.mark.parametrize("group,noise,blo,bhi", [(16, 0.05, 0.0, 2.0), (64, 0.02, 1.0, 2.0),
                                                  (8, 0.01, 1.9, 2.0)])
def test_prefill_solve_stress_fp32(group, noise, blo, bhi):
    """The fp32 mode meets its plain bar on the ill-conditioned stress inputs too."""
    inp = gen.make_stress_inputs(1, 1000, 2, 128, "f32", seed=7 + group, beta_lo=blo, beta_hi=bhi,
                                 group=group, noise=noise)
    for chunk in (32, 64):
        o, st = _run_prefill(inp, chunk)
        o_ref, s_ref = _oracle(inp)
        assert_close(f"o chunk {chunk}", o, o_ref, "f32")
        assert_close(f"S_T chunk {chunk}", st, s_ref, "f32")


def test_native_library_is_the_one_loaded():
    kda = _kda()
    lib = kda._lib.LIB_PATH
    maps = open("/proc/self/maps").read()
    assert lib in maps
    hip = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(hip) == 1, f"more than one HIP runtime mapped: {hip}"
