"""Full-size workloads, in the launch configuration the benchmark times, compared with the
float64 oracle output by output: the oracle runs on a few heads at a time and rel-L2 / max-abs are
accumulated in float64 over the whole tensor (no float64 copy of a whole output is held).

* model width: B=4, H=56, T=32768, d=128, chunk 64, bf16 (automatic plan, no split): all 224
  (sequence, head) pairs, every output and every final state;
* 1M-token context: B=1, H=16, T=1,048,576: the workload's 64K-token segments and the automatic
  plan, all 16 heads, every output and final state;
* model width with the fused gate (bf16 raw pre-activation in place of log alpha) and with state
  checkpoints every 4096 tokens, as the benchmark times them: all 224 pairs, every output, final
  state and checkpoint;
* decode: 256 sequences x 56 heads, 1000 consecutive steps from S ~ N(0, 0.02^2): every output of
  every step and the final states of 32 seeded sequences x all 56 heads (1792 states; the
  other sequences must stay finite).  A decode step is one token of the recurrence, so 1000 steps
  of one state are the oracle's recurrence over those 1000 tokens.

Every output buffer starts filled with NaN, so an element the device never writes fails.
"""
import numpy as np
import pytest
import torch

import oracle
from chunked_gated_delta_13_amd import inputs as gen
from tests.parity import Accum, assert_close, nan_like, to_f64

pytestmark = pytest.mark.gpu


def _kda():
    import chunked_gated_delta_13_amd as kda
    kda.load_library()
    return kda


def _heads(d, b, h0, h1):
    """Inputs of sequence b, heads h0..h1-1 as host tensors shaped [1, T, h1-h0, ...]."""
    sl = lambda x: x[b:b + 1, :, h0:h1].contiguous().cpu()  # noqa: E731
    return (sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["log_alpha"]), sl(d["beta"]),
            None if d["S0"] is None else d["S0"][b:b + 1, h0:h1].contiguous().cpu())


def _compare_all_heads(d, outs, group, col_block, label, gate=None, ck=None, every=0):
    """Every (b, h) of each (o, S_T) in outs against the oracle, `group` heads per oracle call.
    With `gate`, the oracle takes the raw gate in place of log alpha; with `ck` (checkpoints of
    the first output pair, [B, T // every, H, d, d]), the checkpoints are compared too."""
    B, T, H, _ = d["q"].shape
    accs = [(Accum(f"{name} o", "bf16"), Accum(f"{name} S_T", "bf16")) for name, _, _ in outs]
    acc_ck = Accum(f"{label} checkpoints", "bf16") if ck is not None else None
    for b in range(B):
        for h0 in range(0, H, group):
            h1 = min(H, h0 + group)
            print(f"  {label}: oracle on b={b} heads {h0}..{h1 - 1}", flush=True)
            q, k, v, la, bt, s0 = _heads(d, b, h0, h1)
            if gate is not None:
                g = gate[b:b + 1, :, h0:h1].contiguous().cpu()
                o_ref, s_ref = oracle.prefill_gate(q, k, v, g, bt, s0)
            elif ck is not None:
                o_ref, s_ref, ck_ref = oracle.prefill_ckpt(q, k, v, la, bt, s0, every)
                for h in range(h0, h1):
                    acc_ck.add(ck[b:b + 1, :, h:h + 1], ck_ref[:, :, h - h0:h - h0 + 1], (b, h))
            else:
                o_ref, s_ref = oracle.prefill(q, k, v, la, bt, s0, col_block=col_block)
            for (_, o, st), (ao, ast) in zip(outs, accs):
                for h in range(h0, h1):
                    ao.add(o[b:b + 1, :, h:h + 1], o_ref[:, :, h - h0:h - h0 + 1], (b, h))
                    ast.add(st[b:b + 1, h:h + 1], s_ref[:, h - h0:h - h0 + 1], (b, h))
            del q, k, v, la, bt, s0, o_ref, s_ref
    for ao, ast in accs:
        ao.check()
        ast.check()
    if acc_ck is not None:
        acc_ck.check()


def test_model_width_prefill_all_heads():
    kda = _kda()
    w = gen.WORKLOADS["model_width"]
    print(f"model width: {w.note}", flush=True)
    d = gen.workload_inputs(w, device="cuda")
    o = nan_like(d["v"])
    st = nan_like(d["S0"])
    kda.chunk_prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], chunk=w.chunk,
                      o=o, S_T=st)
    torch.cuda.synchronize()
    _compare_all_heads(d, [("model width", o, st)], group=8, col_block=32, label="model width")


def test_model_width_gate_all_heads():
    """The fused bounded gate at model width, as timed: the gate pre-activations the benchmark
    draws (bf16, N(0, 2)), every output and final state."""
    kda = _kda()
    w = gen.WORKLOADS["model_width"]
    print(f"model width, fused gate: {w.note}", flush=True)
    d = gen.workload_inputs(w, device="cuda")
    g = gen.make_gate(w.B, w.T, w.H, w.dk, w.dtype, seed=w.seed, device="cuda")
    o = nan_like(d["v"])
    st = nan_like(d["S0"])
    kda.chunk_prefill_gate(d["q"], d["k"], d["v"], g, d["beta"], d["S0"], chunk=w.chunk, o=o, S_T=st)
    torch.cuda.synchronize()
    _compare_all_heads(d, [("model width, gate", o, st)], group=8, col_block=32, label="gate", gate=g)


def test_model_width_checkpoints_all_heads():
    """State checkpoints every 4096 tokens at model width, as timed: every checkpoint, output and
    final state."""
    kda = _kda()
    w = gen.WORKLOADS["model_width"]
    every = 4096
    print(f"model width, checkpoints every {every}: {w.note}", flush=True)
    d = gen.workload_inputs(w, device="cuda")
    o = nan_like(d["v"])
    st = nan_like(d["S0"])
    ck = torch.full((w.B, w.T // every, w.H, w.dk, w.dv), float("nan"), dtype=torch.float32, device="cuda")
    kda.chunk_prefill_ckpt(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], chunk=w.chunk,
                           ckpt_every=every, o=o, S_T=st, S_ckpt=ck)
    torch.cuda.synchronize()
    _compare_all_heads(d, [("model width, checkpoints", o, st)], group=8, col_block=32, label="checkpoints",
                       ck=ck, every=every)


def test_long_context_all_heads_both_plans():
    """The workload's 64K-token segments and the library's own plan (equal segments, all of them
    running at once), every head."""
    kda = _kda()
    w = gen.WORKLOADS["long_1m"]
    auto_seg, _ = kda.prefill_plan(w.B, w.T, w.H, w.dk, w.dv, w.chunk)
    print(f"long context: {w.note}; automatic plan: segments of {auto_seg}", flush=True)
    d = gen.workload_inputs(w, device="cuda")
    runs = []
    for seg in (w.segment, 0):
        o = nan_like(d["v"])
        st = nan_like(d["S0"])
        kda.chunk_prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], chunk=w.chunk,
                          seg_len=seg, o=o, S_T=st)
        runs.append((f"seg_len {seg}", o, st))
    # the same call again gives bit-identical results (no atomics, fixed reduction order)
    o2 = nan_like(d["v"])
    st2 = nan_like(d["S0"])
    kda.chunk_prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], chunk=w.chunk,
                      seg_len=w.segment, o=o2, S_T=st2)
    torch.cuda.synchronize()
    assert torch.equal(runs[0][1], o2) and torch.equal(runs[0][2], st2)
    del o2, st2
    _compare_all_heads(d, runs, group=2, col_block=8, label="1M tokens")


def test_long_context_slow_decay_split_matches_unsplit():
    """A 64K-token sequence with very slow decay (the slow recipe scaled by 0.01) split into 8K
    segments matches the unsplit run and the oracle.  The delta write itself forgets (each token
    shrinks the state along its key), so over an 8K segment the entry state reaches the segment's
    end only as rounding noise; it shapes the outputs right after each boundary instead.  Those
    must follow the entry state the scan delivered: run from a zero state they would differ."""
    kda = _kda()
    T, seg, w = 65536, 8192, 256
    d = gen.make_prefill_inputs(1, T, 2, 128, 128, "bf16", "slow", 1.0, seed=41,
                                bound_frac=0.0, device="cuda")
    d["log_alpha"].mul_(0.01)
    o1, s1 = nan_like(d["v"]), nan_like(d["S0"])
    o2, s2 = nan_like(d["v"]), nan_like(d["S0"])
    kda.chunk_prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], chunk=64,
                      seg_len=seg, o=o1, S_T=s1)
    kda.chunk_prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], chunk=64,
                      seg_len=1 << 30, o=o2, S_T=s2)   # one pass, no split
    cut = lambda x: x[:, seg:seg + w].contiguous()   # noqa: E731  (the first tokens of segment 1)
    oz, _ = kda.chunk_prefill(cut(d["q"]), cut(d["k"]), cut(d["v"]), cut(d["log_alpha"]),
                              cut(d["beta"]), None, chunk=64)
    torch.cuda.synchronize()
    assert_close("S_T split vs unsplit", s1, to_f64(s2), "bf16")
    assert_close("o split vs unsplit", o1, to_f64(o2), "bf16")
    assert_close("o after the first boundary, split vs unsplit", cut(o1), to_f64(cut(o2)), "bf16")
    ref = cut(o2).double()
    gap = float(torch.linalg.vector_norm(oz.double() - ref) / torch.linalg.vector_norm(ref))
    print(f"  outputs after the boundary from a zero entry state: rel-L2 {gap:.3e}", flush=True)
    assert gap > 0.05
    _compare_all_heads(d, [("slow decay, 8K segments", o1, s1)], group=2, col_block=8, label="slow")


def test_decode_1000_steps_full_heads():
    kda = _kda()
    w = gen.DECODE_WORKLOADS["decode_n256"]
    print(f"decode: {w.note}", flush=True)
    S = gen.make_state(w.N, w.H, w.dk, w.dv, w.s0_std, seed=w.seed, device="cuda")
    P = 32
    picks = torch.from_numpy(np.sort(np.random.default_rng(0).choice(w.N, P, replace=False))).cuda()
    S_start = S[picks].cpu()
    keep = {k: [] for k in ("q", "k", "v", "log_alpha", "beta")}
    outs = []
    o = torch.empty((w.N, w.H, w.dv), dtype=torch.bfloat16, device="cuda")
    for step in range(w.steps):
        t = gen.make_decode_inputs(w.N, w.H, w.dk, w.dv, w.dtype, w.decay,
                                   seed=w.seed * 10**6 + step, device="cuda")
        o.fill_(float("nan"))
        kda.decode_step(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], S, o=o)
        outs.append(o[picks].clone())
        if step % 100 == 99:   # every output of every sequence written and finite
            assert bool(torch.isfinite(o.float()).all()), step
        for key in keep:
            keep[key].append(t[key][picks])
    torch.cuda.synchronize()
    assert torch.isfinite(S).all()
    # the picked sequences' 1000 tokens as one sequence each: [P, 1000, H, ...]
    seq = {key: torch.stack(v, dim=1).cpu() for key, v in keep.items()}
    o_all = torch.stack(outs, dim=1)                     # [P, 1000, H, dv]
    print(f"  oracle on {P} sequences x {w.H} heads x {w.steps} steps", flush=True)
    o_ref, S_ref = oracle.prefill(seq["q"], seq["k"], seq["v"], seq["log_alpha"], seq["beta"], S_start)
    ao = Accum("decode o (every step)", "bf16")
    for i in range(P):
        ao.add(o_all[i:i + 1], o_ref[i:i + 1], int(picks[i]))
    ao.check()
    ast = Accum("decode S after 1000 steps", "bf16")
    for i in range(P):
        ast.add(S[picks[i]][None], S_ref[i:i + 1], int(picks[i]))
    ast.check()


def test_spec_decode_full_batch_full_heads():
    """The speculative-decoding workload at its full size (256 sequences x 56 heads, 4 drafted
    tokens, seeded accepted counts), 50 verify + commit rounds, checked on every output and
    state of 32 seeded sequences x all 56 heads against the oracle."""
    kda = _kda()
    w = gen.SPEC_WORKLOADS["spec_n256_m4"]
    print(f"spec: {w.note}", flush=True)
    S = gen.make_state(w.N, w.H, w.dk, w.dv, w.s0_std, seed=w.seed, device="cuda")
    P = 32
    picks = torch.from_numpy(np.sort(np.random.default_rng(1).choice(w.N, P, replace=False))).cuda()
    S_ref = to_f64(S[picks])                             # [P, H, dk, dv]
    o = torch.empty((w.N, w.m, w.H, w.dv), dtype=torch.bfloat16, device="cuda")
    ao = Accum("spec verify o", "bf16")
    for rnd in range(50):
        b = gen.make_spec_inputs(w.N, w.m, w.H, w.dk, w.dv, w.dtype, w.decay,
                                 seed=w.seed * 10**6 + rnd, device="cuda")
        o.fill_(float("nan"))
        kda.spec_verify(b["q"], b["k"], b["v"], b["log_alpha"], b["beta"], S, o=o)
        kda.spec_commit(b["q"], b["k"], b["v"], b["log_alpha"], b["beta"], S, b["accepted"])
        sub = {k: b[k][picks].cpu() for k in ("q", "k", "v", "log_alpha", "beta")}
        acc = b["accepted"][picks].cpu().numpy()
        o_ref = oracle.spec_verify(sub["q"], sub["k"], sub["v"], sub["log_alpha"], sub["beta"], S_ref)
        S_ref = oracle.spec_commit(sub["q"], sub["k"], sub["v"], sub["log_alpha"], sub["beta"], S_ref, acc)
        ao.add(o[picks], o_ref, rnd)
    torch.cuda.synchronize()
    ao.check()
    assert_close("S after 50 rounds", S[picks], S_ref, "bf16")
    assert torch.isfinite(S).all()
