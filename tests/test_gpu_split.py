"""The sequence split's short cut, against the float64 oracle.

A segment's entry state reaches its outputs only through the segment's transition, and that
transition dies out along the segment (every token's transition is a contraction for unit keys and
beta in [0, 2], and the decay shrinks it further).  The split's transition pass stops once every
entry of the transition is below 2^-126, the segments run from a zero start with their outputs,
and only the chunks before that point are rerun from the true entry states.  Where a transition
never dies (no decay and beta = 0: the transition is the identity), the full two-pass split runs.

The input patterns put both kinds of unit in one launch:
  fast   log alpha = -5 sigmoid(N(0, 2)) everywhere: every transition dies within a chunk or two;
  mixed  head 1 with log alpha = 0 and beta = 0 everywhere: its transitions never die, and its
         state stays S0 exactly;
  late   head 0 with log alpha = 0, beta = 0 for the first 600 tokens (transitions of segments
         inside that range never die; the segment holding token 600 dies part-way); head 1 the
         same for the first 100 tokens of every 256-token window (every segment dies a few chunks
         in).
"""
import pytest
import torch

import oracle
from chunked_gated_delta_13_amd import inputs as gen
from tests.parity import assert_close, nan_like, to_device, to_f64

pytestmark = pytest.mark.gpu


def _kda():
    import chunked_gated_delta_13_amd as kda
    kda.load_library()
    return kda


def _inputs(dtype, d, T, pattern, seed):
    inp = gen.make_prefill_inputs(2, T, 2, d, d, dtype, "sig2", 1.0, seed, 0.0, "cpu")
    la, beta = inp["log_alpha"], inp["beta"]
    if pattern == "mixed":
        la[:, :, 1] = 0.0
        beta[:, :, 1] = 0.0
    elif pattern == "late":
        la[:, :600, 0] = 0.0
        beta[:, :600, 0] = 0.0
        window = (torch.arange(T) % 256) < 100
        la[:, window, 1] = 0.0
        beta[:, window, 1] = 0.0
    return inp


def _prefill(kda, d, chunk, seg, nvs):
    o = nan_like(d["v"])
    st = nan_like(d["S0"])
    kda.chunk_prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], chunk=chunk,
                      seg_len=seg, n_vs=nvs, o=o, S_T=st)
    torch.cuda.synchronize()
    return o, st


CASES = [
    # dtype, d, chunk, seg, n_vs, T, pattern
    ("bf16", 128, 64, 256, 1, 1000, "fast"),    # shared transition/increment pass, ragged last segment
    ("bf16", 128, 64, 256, 1, 1000, "mixed"),
    ("bf16", 128, 64, 256, 1, 1000, "late"),
    ("bf16", 128, 64, 512, 1, 1000, "mixed"),   # two segments: no scan
    ("bf16", 128, 32, 192, 1, 1000, "late"),    # 32-token chunks (single-role kernel throughout)
    ("bf16", 128, 16, 128, 1, 700, "late"),
    ("bf16", 128, 64, 256, 2, 1000, "late"),    # two column slices: the 4-wave transition pass
    ("bf16", 64, 64, 256, 1, 1000, "late"),
    ("f32", 64, 32, 256, 1, 1000, "late"),
    ("f32", 128, 16, 128, 2, 700, "mixed"),
    ("f32", 128, 64, 256, 1, 1000, "fast"),
]


@pytest.mark.parametrize("dtype,d,chunk,seg,nvs,T,pattern", CASES)
def test_split_short_cut_matches_oracle(dtype, d, chunk, seg, nvs, T, pattern):
    kda = _kda()
    print(f"split dtype={dtype} d={d} chunk={chunk} seg={seg} n_vs={nvs} T={T} {pattern}", flush=True)
    inp = _inputs(dtype, d, T, pattern, seed=300 + T + d + chunk)
    dd = to_device(inp)
    o, st = _prefill(kda, dd, chunk, seg, nvs)
    o_ref, s_ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["S0"])
    assert_close("o", o, o_ref, dtype)
    assert_close("S_T", st, s_ref, dtype)
    # against the unsplit launch on the same inputs
    o1, st1 = _prefill(kda, dd, chunk, 0, nvs)   # too short for the automatic plan to split
    assert_close("o split vs unsplit", o, to_f64(o1), dtype)
    assert_close("S_T split vs unsplit", st, to_f64(st1), dtype)
    if pattern == "mixed":   # the identity transitions keep head 1's state at S0, bit for bit
        assert torch.equal(st[:, 1], dd["S0"][:, 1])


def test_split_short_cut_is_deterministic_and_matches_no_alloc():
    """Two runs give the same bits; the allocation-free entry point (segment 0 inside the
    zero-start launch, one stream) gives the same bits as the workspace path (segment 0 on the
    library's side stream)."""
    kda = _kda()
    inp = _inputs("bf16", 128, 3000, "late", seed=71)
    dd = to_device(inp)
    o1, st1 = _prefill(kda, dd, 64, 512, 1)
    o2, st2 = _prefill(kda, dd, 64, 512, 1)
    assert torch.equal(o1, o2) and torch.equal(st1, st2)
    o3 = nan_like(dd["v"])
    st3 = nan_like(dd["S0"])
    kda.chunk_prefill_noalloc(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"], dd["S0"], chunk=64,
                              seg_len=512, o=o3, S_T=st3)
    torch.cuda.synchronize()
    assert torch.equal(o1, o3) and torch.equal(st1, st3)


def test_split_transition_pass_stops_where_transitions_die():
    """The mechanism itself, read back from the caller's workspace (the transition pass's chunk
    counts follow the transitions, increments and entry states: int32 [B*H, n_seg - 1, n_vs] in a
    region sized for two slices).  Fast decay: every count is a few chunks.  An identity head
    (log alpha = 0, beta = 0): -1, never died, so the full two-pass split ran there.  A head
    that is the identity for its first 600 tokens: -1 in the segment that lies inside that
    range, a few chunks past token 600 in the segment holding it, a few chunks after that."""
    kda = _kda()
    B, T, H, d, seg = 2, 1000, 2, 128, 256
    ns = -(-T // seg)
    for pattern in ("mixed", "late"):
        inp = _inputs("bf16", d, T, pattern, seed=91)
        dd = to_device(inp)
        need = kda.prefill_workspace_bytes(B, T, H, d, d, 64, seg_len=seg)
        ws = torch.full((need,), 0x7f, dtype=torch.uint8, device="cuda")
        kda.chunk_prefill(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"], dd["S0"], chunk=64,
                          seg_len=seg, workspace=ws)
        torch.cuda.synchronize()
        SS = d * d * 4
        off = B * H * ((ns - 1) * 2 + ns) * SS
        z = ws[off:off + B * H * (ns - 1) * 4].view(torch.int32).view(B, H, ns - 1).cpu()
        print(f"{pattern}: chunk counts of segments 1..{ns - 1} per (b, h):\n{z}", flush=True)
        if pattern == "mixed":
            assert ((z[:, 0] >= 1) & (z[:, 0] <= 3)).all()   # fast decay: dead within a few chunks
            assert (z[:, 1] == -1).all()                     # identity head: never dies
        else:
            # head 0: segment 1 = tokens 256..511 lies inside the identity range; segment 2 =
            # tokens 512..767 holds token 600 (chunk 1 of the segment); segment 3 decays at once
            assert (z[:, 0, 0] == -1).all()
            assert ((z[:, 0, 1] >= 2) & (z[:, 0, 1] <= 4)).all()
            assert ((z[:, 0, 2] >= 1) & (z[:, 0, 2] <= 3)).all()
            # head 1: the first 100 tokens of every segment are the identity (chunk 1 holds token
            # 100), then fast decay
            assert ((z[:, 1] >= 2) & (z[:, 1] <= 4)).all()
