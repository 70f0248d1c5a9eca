"""KDA benchmark on one MI355X: prefill tokens/s (+ decode state GB/s).

One step = one chunked KDA prefill over the model-width batch (B=4, H=56,
T=32768, d_k=d_v=128, chunk 64, bf16 q/k/v, fp32 log_alpha/beta/state) with
all inputs already resident in HBM.  The same run also measures
  * the decode step (256 sequences x 56 heads, fp32 state read-modify-written
    in place, 1000 consecutive steps), reported as achieved state GB/s;
  * the 1M-token prefill (B=1, H=16, T=1,048,576) split into 64K-token
    segments (transitions + increments, on-device prefix scan, rerun);
  * the float64 oracle on the host cores, on a bounded sample of the prefill
    workload (the CPU baseline).
Prints one JSON line on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KDA prefill tokens/s/GPU (H=56,d=128,bf16) + decode state GB/s vs HBM peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix, published

# Algorithmic work per token-head at d_k = d_v = 128, chunk 64 (bf16 q/k/v/o, fp32 log_alpha,
# fp32 beta): bytes = q 256 + k 256 + v 256 + log_alpha 512 + beta 4 + o 256 = 1540.
BYTES_PER_TOKEN_HEAD = 1540
# Useful multiply-adds per token-head: five lower-triangular 16-token-tile products
# (5 * (n+1)/2 * 16 * d with n = 4) + three state products (3 d^2) + the inverse (~1067).
FLOPS_PER_TOKEN_HEAD = 2 * (5 * 2.5 * 16 * 128 + 3 * 128 * 128 + 1067)
# the kernel that runs the model-width workload (one 128-column slice per workgroup)
PREFILL_KERNEL = "kda_prefill_pipe_kernel<8,false>"
# sources of the model-width prefill kernel (a profile's counters hold while their hash matches)
PREFILL_SOURCES = ["kda_prefill_pipe.h", "kda_prefill_kernel.h", "kda_device.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def profiled_value(summary, sources, key="traffic_bytes_per_launch"):
    """A figure recorded in profiles/<summary> from rocprofv3 PMC runs (HBM bytes per launch from
    FETCH_SIZE/WRITE_SIZE, or the MFMA busy fraction), or None when the kernel sources have
    changed since those counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "|", " ")):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "chunked_gated_delta_13_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if rec.get("source_sha256_16") != h.hexdigest()[:16]:
        return None
    try:
        return float(rec[key])
    except (KeyError, ValueError):
        return None


def prefill_bytes(B, T, H, d, with_state=True):
    b = B * T * H * BYTES_PER_TOKEN_HEAD
    if with_state:
        b += 2 * B * H * d * d * 4       # S0 read + S_T write
    return b


def decode_bytes(N, H, d):
    state = N * H * d * d * 4
    per_tok = N * H * (3 * d * 2 + d * 4 + 4 + d * 2)   # q, k, v bf16; log_alpha; beta; o bf16
    return 2 * state + per_tok


def time_loop(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        fn()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, ev0.elapsed_time(ev1) / 1000.0


def bench_prefill(kda, gen, steps, warmup):
    import torch
    w = gen.WORKLOADS["model_width"]
    log(f"[prefill] generating {w.note} on the device")
    d = gen.workload_inputs(w, device="cuda")
    o = torch.empty_like(d["v"])
    st = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        kda.chunk_prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"],
                          chunk=w.chunk, o=o, S_T=st)

    wall, ev = time_loop(step, steps, warmup, stream)
    assert torch.isfinite(o[:, -64:].float()).all() and torch.isfinite(st).all()
    plan = kda.prefill_plan(w.B, w.T, w.H, w.dk, w.dv, w.chunk)
    log(f"[prefill] {steps} steps: wall {wall*1e3:.2f} ms, events {ev*1e3:.2f} ms, plan {plan}")
    return w, d, wall, ev, plan, o


def bench_prefill_ckpt(kda, w, d, steps, warmup, every=4096):
    """Model-width prefill that also checkpoints the state every `every` tokens (a sparse subset
    of the 512-token hash endpoints: every eighth one)."""
    import torch
    o = torch.empty_like(d["v"])
    st = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    ck = torch.empty((w.B, w.T // every, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        kda.chunk_prefill_ckpt(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"],
                               chunk=w.chunk, ckpt_every=every, o=o, S_T=st, S_ckpt=ck)

    wall, ev = time_loop(step, steps, warmup, stream)
    ck_bytes = ck.numel() * 4
    alg = prefill_bytes(w.B, w.T, w.H, w.dk) + ck_bytes
    log(f"[ckpt] {steps} steps: events {ev*1e3:.2f} ms")
    return {"every": every, "checkpoints_per_sequence": w.T // every, "ms_per_step": ev / steps * 1e3,
            "checkpoint_bytes": ck_bytes, "alg_bytes_per_launch": alg,
            "achieved_GBps": alg / (ev / steps) / 1e9,
            "frac_of_hbm_peak": alg / (ev / steps) / 1e9 / HBM_PEAK_GBS}


def bench_prefill_gate(kda, gen, w, d, steps, warmup):
    """Model-width prefill with the fused bounded gate: bf16 raw gate pre-activations replace the
    fp32 log-decay (1284 instead of 1540 algorithmic bytes per token-head)."""
    import torch
    g = gen.make_gate(w.B, w.T, w.H, w.dk, w.dtype, seed=w.seed, device="cuda")
    o = torch.empty_like(d["v"])
    st = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        kda.chunk_prefill_gate(d["q"], d["k"], d["v"], g, d["beta"], d["S0"], chunk=w.chunk, o=o, S_T=st)

    wall, ev = time_loop(step, steps, warmup, stream)
    del g
    alg = prefill_bytes(w.B, w.T, w.H, w.dk) - w.B * w.T * w.H * w.dk * 2
    log(f"[gate] {steps} steps: events {ev*1e3:.2f} ms")
    return {"ms_per_step": ev / steps * 1e3, "tokens_per_s": w.B * w.T * steps / wall,
            "alg_bytes_per_launch": alg, "achieved_GBps": alg / (ev / steps) / 1e9,
            "frac_of_hbm_peak": alg / (ev / steps) / 1e9 / HBM_PEAK_GBS}


def bench_long(kda, gen, steps, warmup):
    """The 1M-token prefill with the workload's 64K-token segments, then with the library's own
    plan (equal segments, few enough that all run at once on fewer workgroups than compute units)."""
    import torch
    w = gen.WORKLOADS["long_1m"]
    log(f"[long] generating {w.note} on the device")
    d = gen.workload_inputs(w, device="cuda")
    o = torch.empty_like(d["v"])
    st = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    res = []
    for seg in (w.segment, 0):
        need = kda.prefill_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv, w.chunk, seg_len=seg)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")

        def step():
            kda.chunk_prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"],
                              chunk=w.chunk, seg_len=seg, o=o, S_T=st, workspace=ws)

        wall, ev = time_loop(step, steps, warmup, stream)
        assert torch.isfinite(st).all()
        log(f"[long] seg_len {seg}: {steps} steps: wall {wall*1e3:.2f} ms, events {ev*1e3:.2f} ms")
        res.append((wall, ev))
        del ws
    del d, o
    torch.cuda.empty_cache()
    return w, res


def bench_decode(kda, gen, steps=1000, warmup=10):
    """The decode workload as defined: `steps` consecutive steps, step s with its own seeded
    token inputs (seed 4 * 10^6 + s), all drawn on the device before the timed region; the
    warm-up steps use further seeds."""
    import torch
    w = gen.DECODE_WORKLOADS["decode_n256"]
    log(f"[decode] {w.note}: state {w.N*w.H*w.dk*w.dv*4/1e9:.3f} GB, {steps} + {warmup} distinct token sets")
    S = gen.make_state(w.N, w.H, w.dk, w.dv, w.s0_std, seed=w.seed, device="cuda")
    seeds = [w.seed * 10**6 + steps + i for i in range(warmup)] + [w.seed * 10**6 + i for i in range(steps)]
    toks = [gen.make_decode_inputs(w.N, w.H, w.dk, w.dv, w.dtype, w.decay, seed=sd, device="cuda")
            for sd in seeds]
    o = torch.empty((w.N, w.H, w.dv), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    it = [0]

    def step():
        t = toks[it[0]]
        it[0] += 1
        kda.decode_step(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], S, o=o)

    wall, ev = time_loop(step, steps, warmup, stream)
    assert it[0] == steps + warmup
    assert torch.isfinite(S).all()
    log(f"[decode] {steps} steps: wall {wall*1e3:.2f} ms, events {ev*1e3:.2f} ms")
    del toks, S
    torch.cuda.empty_cache()
    return w, wall, ev


def spec_bytes(N, H, d, m, accepted):
    """Algorithmic HBM bytes of one verify (state read, drafted inputs, outputs) and one commit.
    A commit moves only the sequences that accept at least one token: their state is read and
    written, and their accepted tokens' k, v, log_alpha and beta are read (queries not needed)."""
    state_head = d * d * 4
    verify = N * H * state_head + N * m * H * (3 * d * 2 + d * 4 + 4 + d * 2)
    moved = int((accepted > 0).sum())
    toks = int(accepted.clamp(0, m).sum())
    commit = moved * H * 2 * state_head + toks * H * (2 * d * 2 + d * 4 + 4)
    return verify, commit


def bench_spec(kda, gen, steps=200, warmup=5):
    """The speculative-decoding workload: every timed step on its own seeded drafted block (block
    i with seed 7 * 10^6 + i), all drawn on the device before the timed regions."""
    import torch
    w = gen.SPEC_WORKLOADS["spec_n256_m4"]
    pool = steps + warmup
    log(f"[spec] {w.note}: state {w.N*w.H*w.dk*w.dv*4/1e9:.3f} GB, {pool} distinct drafted blocks")
    S = gen.make_state(w.N, w.H, w.dk, w.dv, w.s0_std, seed=w.seed, device="cuda")
    blocks = [gen.make_spec_inputs(w.N, w.m, w.H, w.dk, w.dv, w.dtype, w.decay,
                                   seed=w.seed * 10**6 + i, device="cuda") for i in range(pool)]
    o = torch.empty((w.N, w.m, w.H, w.dv), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    it = [0]

    def verify():
        b = blocks[it[0] % pool]
        it[0] += 1
        kda.spec_verify(b["q"], b["k"], b["v"], b["log_alpha"], b["beta"], S, o=o)

    def commit():
        b = blocks[it[0] % pool]
        it[0] += 1
        kda.spec_commit(b["q"], b["k"], b["v"], b["log_alpha"], b["beta"], S, b["accepted"])

    def both():
        b = blocks[it[0] % pool]
        it[0] += 1
        kda.spec_verify(b["q"], b["k"], b["v"], b["log_alpha"], b["beta"], S, o=o)
        kda.spec_commit(b["q"], b["k"], b["v"], b["log_alpha"], b["beta"], S, b["accepted"])

    _, ev_v = time_loop(verify, steps, warmup, stream)
    it[0] = 0
    _, ev_c = time_loop(commit, steps, warmup, stream)
    it[0] = 0
    wall, ev_b = time_loop(both, steps, warmup, stream)
    assert torch.isfinite(S).all()
    acc_mean = sum(float(b["accepted"].float().mean()) for b in blocks) / pool
    per = [spec_bytes(w.N, w.H, w.dk, w.m, b["accepted"].cpu()) for b in blocks]
    vb = sum(p[0] for p in per) / pool
    cb = sum(p[1] for p in per) / pool
    res = {"workload": w.note, "steps": steps, "m": w.m,
           "verify_us": ev_v / steps * 1e6, "verify_GBps": vb / (ev_v / steps) / 1e9,
           "commit_us": ev_c / steps * 1e6, "commit_GBps": cb / (ev_c / steps) / 1e9,
           "step_us": ev_b / steps * 1e6,
           "frac_of_hbm_peak": (vb + cb) / (ev_b / steps) / 1e9 / HBM_PEAK_GBS,
           "accepted_tokens_per_s": w.N * acc_mean * steps / wall,
           "alg_bytes_per_step": vb + cb}
    log(f"[spec] verify {res['verify_us']:.1f} us ({res['verify_GBps']:.0f} GB/s), commit "
        f"{res['commit_us']:.1f} us ({res['commit_GBps']:.0f} GB/s)")
    del blocks, S
    torch.cuda.empty_cache()
    return res


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(gen_inputs, w, o_dev, budget_s=15.0):
    """Oracle (float64, OpenMP) on the host cores over a bounded sample of the prefill workload:
    the first P (sequence, head) pairs in sequence-major order, all T tokens each.  The oracle's
    outputs for the sample are also compared with the device's outputs of the timed launches
    (o_dev): rel-L2 and max-abs over the sample, beside the bf16 rounding floor."""
    import oracle
    import torch
    cores = oracle.default_threads()

    def gather(pairs):
        out = []
        for key in ("q", "k", "v", "log_alpha", "beta"):
            x = gen_inputs[key]
            out.append(torch.stack([x[b, :, h] for b, h in pairs], dim=1)[None].cpu())
        s0 = torch.stack([gen_inputs["S0"][b, h] for b, h in pairs])[None].cpu()
        return out, s0

    all_pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    args, s0 = gather(all_pairs[:1])
    t0 = time.perf_counter()
    oracle.prefill(*args, S0=s0, nthreads=cores)
    t1 = time.perf_counter() - t0
    # the oracle parallelises over (head, 32-column block): 4 units per head at d_v = 128
    n = int(min(len(all_pairs), max(1, budget_s / max(t1, 1e-3) * max(1, cores // 4))))
    pairs = all_pairs[:n]
    args, s0 = gather(pairs)
    t0 = time.perf_counter()
    o_ref, _ = oracle.prefill(*args, S0=s0, nthreads=cores)
    el = time.perf_counter() - t0
    token_heads = w.T * n
    tok_s = token_heads / w.H / el
    log(f"[cpu] oracle on {n} (sequence, head) pairs x {w.T} tokens: {el:.2f} s, {cores} threads")
    # parity of the timed launches' outputs on the sample (float64 sums)
    got = torch.stack([o_dev[b, :, h] for b, h in pairs], dim=1)[None].cpu().double()
    y = torch.from_numpy(o_ref)
    dif = got - y
    fl = y.to(torch.bfloat16).double() - y
    den = float((y * y).sum())
    parity = {"pairs": n, "o_rel_l2": (float((dif * dif).sum()) / den) ** 0.5,
              "o_max_abs": float(dif.abs().max()),
              "bf16_floor_rel_l2": (float((fl * fl).sum()) / den) ** 0.5,
              "bf16_floor_max_abs": float(fl.abs().max())}
    log(f"[cpu] parity of the timed outputs on the sample: {parity}")
    del args, s0, o_ref, got, y, dif, fl
    return {"value": tok_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"first {n} of {len(all_pairs)} (sequence, head) pairs, all {w.T} tokens each "
                      f"({token_heads} token-heads in {el:.1f} s); tokens/s = token-heads/s / {w.H}"}, parity


def cpu_baseline_decode(gen, steps=10):
    """Oracle decode steps over every state of the decode workload (256 x 56), one step at a time
    (the state carried from step to step), timed per step."""
    import oracle
    w = gen.DECODE_WORKLOADS["decode_n256"]
    cores = oracle.default_threads()
    S = gen.make_state(w.N, w.H, w.dk, w.dv, w.s0_std, seed=w.seed, device="cpu")
    toks = [gen.make_decode_inputs(w.N, w.H, w.dk, w.dv, w.dtype, w.decay, seed=w.seed * 10**6 + i,
                                   device="cpu") for i in range(steps)]
    t0 = time.perf_counter()
    for t in toks:
        _, S = oracle.decode_step(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], S, nthreads=cores)
    el = time.perf_counter() - t0
    log(f"[cpu] oracle decode: {steps} steps over {w.N} x {w.H} states: {el:.2f} s, {cores} threads")
    return {"value": w.N * steps / el, "unit": "tokens/s", "us_per_step": el / steps * 1e6,
            "cores": cores, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{steps} full steps (all {w.N * w.H} states each)"}


def cpu_baseline_long(gen, heads=1):
    """Oracle on `heads` of the 16 heads of the 1M-token workload, all 1,048,576 tokens, scaled to
    the 16 heads (heads are independent and the oracle's per-head cost does not depend on h)."""
    import oracle
    w = gen.WORKLOADS["long_1m"]
    cores = oracle.default_threads()
    d = gen.workload_inputs(w, device="cpu", H=heads)
    t0 = time.perf_counter()
    oracle.prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], nthreads=cores,
                   col_block=max(1, 128 * heads // max(1, cores)))
    el = time.perf_counter() - t0
    full = el * w.H / heads
    log(f"[cpu] oracle on {heads} head(s) x {w.T} tokens: {el:.2f} s ({full:.1f} s scaled to {w.H} heads)")
    del d
    return {"value": w.B * w.T / full, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{heads} of {w.H} heads, all {w.T} tokens ({el:.1f} s), scaled linearly to {w.H} heads"}


def measure_peaks():
    """Re-measured peaks on this GPU: dense bf16 GEMMs through torch.matmul (8192^3 and 16384^3,
    the faster reported), and HBM streams from the bandwidth probes of libkda_peaks.so (a 4 GiB
    read stream, a 2 GiB + 2 GiB device copy and a 2 GiB in-place read-modify-write, 16-byte
    non-temporal accesses), with torch's own device copy beside them."""
    import ctypes
    import torch
    from chunked_gated_delta_13_amd import build as kbuild
    res = {}
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(reps):
            fn()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / 1e3 / reps

    best = 0.0
    for n in (8192, 16384):
        a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
        b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
        t = timed(lambda: a @ b, 10)
        best = max(best, 2 * n ** 3 / t / 1e12)
        del a, b
    res["bf16_gemm_TFLOPs"] = best
    lib = ctypes.CDLL(kbuild.PEAKS_LIB)
    lib.kda_peak_read_sink_floats.restype = ctypes.c_size_t
    lib.kda_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    lib.kda_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    x = torch.ones(1 << 30, dtype=torch.float32, device="cuda")           # 4 GiB
    sink = torch.empty(lib.kda_peak_read_sink_floats(), dtype=torch.float32, device="cuda")
    sp = ctypes.c_void_p(stream.cuda_stream)
    nb = x.numel() * 4

    def rd():
        assert lib.kda_peak_read(ctypes.c_void_p(x.data_ptr()), nb, ctypes.c_void_p(sink.data_ptr()), sp) == 0

    res["hbm_read_GBps"] = nb / timed(rd, 10) / 1e9
    half = 1 << 29                                                       # 2 GiB of floats
    src, dst = x[:half], x[half:]

    def cp():
        assert lib.kda_peak_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()),
                                 half * 4, sp) == 0

    res["hbm_copy_GBps"] = 2 * half * 4 / timed(cp, 10) / 1e9
    lib.kda_peak_rmw.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float, ctypes.c_float, ctypes.c_void_p]

    def rmw():
        assert lib.kda_peak_rmw(ctypes.c_void_p(src.data_ptr()), half * 4, 1.0, 0.0, sp) == 0

    res["hbm_rmw_GBps"] = 2 * half * 4 / timed(rmw, 10) / 1e9
    res["torch_copy_GBps"] = 2 * half * 4 / timed(lambda: dst.copy_(src), 10) / 1e9
    del x, sink, src, dst
    torch.cuda.empty_cache()
    log(f"[peaks] {res}")
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-spec", action="store_true")
    ap.add_argument("--no-ckpt", action="store_true")
    ap.add_argument("--no-gate", action="store_true")
    ap.add_argument("--spec-only", action="store_true")
    ap.add_argument("--prefill-only", action="store_true")
    ap.add_argument("--decode-only", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device-to-device copy (known traffic) so that "
                         "HBM byte counters can be scaled")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import chunked_gated_delta_13_amd as kda
    from chunked_gated_delta_13_amd import inputs as gen
    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    kda.load_library()
    torch.cuda.set_device(0)

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[calibration] 3 copies of 1 GiB (1073741824 bytes read + written each)")
        del src, dst
    if args.spec_only:
        log(json.dumps(bench_spec(kda, gen)))
        return
    if args.decode_only:
        wd, dwall, dev_s = bench_decode(kda, gen, args.decode_steps)
        step_s = dev_s / args.decode_steps
        gbs = decode_bytes(wd.N, wd.H, wd.dk) / step_s / 1e9
        log(f"[decode] {step_s * 1e6:.1f} us per step, {gbs:.1f} GB/s")
        return

    w, d, wall, ev, plan, o_dev = bench_prefill(kda, gen, args.steps, args.warmup)
    tokens = w.B * w.T
    tok_s = tokens * args.steps / wall
    launch_s = ev / args.steps                 # one kernel launch per step (no split)
    alg_bytes = prefill_bytes(w.B, w.T, w.H, w.dk)
    achieved = alg_bytes / launch_s / 1e9
    useful_tflops = FLOPS_PER_TOKEN_HEAD * w.B * w.T * w.H / launch_s / 1e12
    result = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "KDA chunked prefill B4 H56 T32768 d128 chunk64 bf16 (7168 hidden)",
                   "B": w.B, "T": w.T, "H": w.H, "dk": w.dk, "dv": w.dv, "chunk": w.chunk,
                   "tokens_per_step": tokens, "seg_len": plan[0], "n_vs": plan[1],
                   "parallelism": "1 GPU"},
        "roofline": {"bound": "hbm", "kernel": PREFILL_KERNEL,
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": profiled_value("kda_prefill_pipe_kernel_model_width.md", PREFILL_SOURCES),
                     "mfma_busy_frac_rocprof": profiled_value("kda_prefill_pipe_kernel_model_width.md",
                                                              PREFILL_SOURCES, "mfma_busy_frac"),
                     "alg_bytes_per_launch": alg_bytes, "launch_ms": launch_s * 1e3,
                     "useful_tflops": useful_tflops,
                     "useful_frac_of_bf16_peak": useful_tflops / BF16_PEAK_TFLOPS},
    }
    if not args.prefill_only and not args.no_ckpt:
        ckr = bench_prefill_ckpt(kda, w, d, args.steps, args.warmup)
        ckr["overhead_vs_plain"] = ckr["ms_per_step"] / (launch_s * 1e3) - 1.0
        result["prefill_checkpoints"] = ckr
    if not args.prefill_only and not args.no_gate:
        result["prefill_fused_gate"] = bench_prefill_gate(kda, gen, w, d, args.steps, args.warmup)
    if not args.prefill_only and not args.no_cpu_baseline:
        result["cpu_baseline"], result["parity_sampled_vs_oracle"] = cpu_baseline(d, w, o_dev)
        result["cpu_baseline"]["gpu_speedup"] = tok_s / result["cpu_baseline"]["value"]
    del d, o_dev
    torch.cuda.empty_cache()

    if not args.prefill_only and not args.no_decode:
        wd, dwall, dev_s = bench_decode(kda, gen, args.decode_steps)
        step_s = dev_s / args.decode_steps
        gbs = decode_bytes(wd.N, wd.H, wd.dk) / step_s / 1e9
        result["decode"] = {"workload": wd.note, "steps": args.decode_steps,
                            "us_per_step": step_s * 1e6, "state_GBps": gbs,
                            "frac_of_hbm_peak": gbs / HBM_PEAK_GBS,
                            "alg_bytes_per_step": decode_bytes(wd.N, wd.H, wd.dk),
                            "traffic": profiled_value("kda_decode_kernel_n256.md",
                                                      ["kda_decode.hip", "kda_device.h"]),
                            "tokens_per_s": wd.N * args.decode_steps / dwall}
        if not args.no_cpu_baseline:
            result["decode"]["cpu_baseline"] = cpu_baseline_decode(gen)
            result["decode"]["cpu_baseline"]["gpu_speedup"] = (result["decode"]["tokens_per_s"] /
                                                               result["decode"]["cpu_baseline"]["value"])
    if not args.prefill_only and not args.no_spec:
        result["spec_decode"] = bench_spec(kda, gen)
    if not args.prefill_only and not args.no_long:
        nsteps = max(2, args.steps // 5)
        wl, lres = bench_long(kda, gen, nsteps, 1)
        (lwall, _), (awall, _) = lres
        auto_seg, _ = kda.prefill_plan(wl.B, wl.T, wl.H, wl.dk, wl.dv, wl.chunk)
        # algorithmic bytes of one pass over the sequence: what any split must move at least
        one_pass = wl.B * wl.T * wl.H * BYTES_PER_TOKEN_HEAD + 2 * wl.B * wl.H * wl.dk * wl.dv * 4
        result["long_context"] = {"workload": wl.note, "seg_len": wl.segment, "steps": nsteps,
                                  "ms_per_step": lwall / nsteps * 1e3,
                                  "tokens_per_s": wl.B * wl.T * nsteps / lwall,
                                  "alg_bytes_one_pass": one_pass,
                                  "frac_of_hbm_peak": one_pass * nsteps / lwall / (HBM_PEAK_GBS * 1e9),
                                  "automatic_plan": {"seg_len": auto_seg,
                                                     "ms_per_step": awall / nsteps * 1e3,
                                                     "tokens_per_s": wl.B * wl.T * nsteps / awall,
                                                     "frac_of_hbm_peak": one_pass * nsteps / awall / (HBM_PEAK_GBS * 1e9)}}
        if not args.no_cpu_baseline:
            result["long_context"]["cpu_baseline"] = cpu_baseline_long(gen)
            result["long_context"]["cpu_baseline"]["gpu_speedup"] = (result["long_context"]["tokens_per_s"] /
                                                                     result["long_context"]["cpu_baseline"]["value"])
    if not args.prefill_only:
        peaks = measure_peaks()
        rf = result["roofline"]
        rf["peak_measured"] = dict(peaks)
        rf["frac_of_measured_read"] = rf["achieved"] / peaks["hbm_read_GBps"]
        rf["useful_frac_of_measured_gemm"] = rf["useful_tflops"] / peaks["bf16_gemm_TFLOPs"]
        if "decode" in result:
            result["decode"]["frac_of_measured_rmw"] = result["decode"]["state_GBps"] / peaks["hbm_rmw_GBps"]
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
