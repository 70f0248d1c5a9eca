"""Prefill with prefix-reuse checkpoints on the device vs the float64 oracle.

Checkpoints are states after every `ckpt_every` tokens ("Kimi K3's
architecture", section "The bill comes due in the serving stack"); with a
sequence split they come from the pass that runs every segment from its true
entry state.  Every call goes through the C ABI of libkda.so.
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


@pytest.mark.parametrize("dtype,d,T,chunk,every,seg,decay", [
    ("bf16", 128, 1000, 64, 128, 0, "slow"),       # 7 checkpoints, ragged tail, no split
    ("bf16", 128, 1000, 64, 128, 256, "slow"),     # the same through the sequence split
    ("bf16", 128, 1024, 64, 128, 256, "sig2"),     # split whose transitions die within a segment
    ("bf16", 128, 1000, 64, 64, 192, "sig2"),      # ... checkpoints inside the rerun chunks too
    ("f32", 64, 1000, 32, 64, 256, "sig2"),        # ... on the 4-wave transition pass
    ("bf16", 64, 640, 32, 64, 0, "slow"),
    ("f32", 64, 300, 16, 32, 0, "slow"),
    ("bf16", 128, 512, 64, 512, 0, "slow"),        # one checkpoint, at the last token
    ("bf16", 128, 12288, 64, 4096, 0, "slow"),     # automatic split: 13 segments of 960 tokens
    ("f32", 128, 700, 64, 128, 0, "slow"),         # fp32 with 64-token chunks
])
def test_prefill_checkpoints_match_oracle(dtype, d, T, chunk, every, seg, decay):
    kda = _kda()
    print(f"ckpt dtype={dtype} d={d} T={T} chunk={chunk} every={every} seg={seg} decay={decay}", flush=True)
    inp = gen.make_prefill_inputs(2, T, 2, d, d, dtype, decay, 1.0, 90 + T, 0.0, "cpu")
    dd = to_device(inp)
    ck0 = torch.full((2, T // every, 2, d, d), float("nan"), dtype=torch.float32, device="cuda")
    o, st, ck = kda.chunk_prefill_ckpt(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"], dd["S0"],
                                       chunk=chunk, ckpt_every=every, seg_len=seg, o=nan_like(dd["v"]),
                                       S_T=nan_like(dd["S0"]), S_ckpt=ck0)
    torch.cuda.synchronize()
    o_ref, s_ref, ck_ref = oracle.prefill_ckpt(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                                               inp["S0"], every)
    assert ck.shape == ck_ref.shape
    assert_close("checkpoints", ck, ck_ref, dtype)
    assert_close("o", o, o_ref, dtype)
    assert_close("S_T", st, s_ref, dtype)
    # checkpoints do not change the run: same bits as the plain prefill
    o2, st2 = kda.chunk_prefill(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"], dd["S0"],
                                chunk=chunk, seg_len=seg)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(st, st2)
    if T % every == 0:
        assert torch.equal(ck[:, -1], st)


def test_resume_from_device_checkpoint():
    """A prefill resumed from a checkpoint reproduces the rest of the run."""
    kda = _kda()
    T, every = 768, 256
    inp = gen.make_prefill_inputs(2, T, 3, 128, 128, "bf16", "slow", 1.0, 97, 0.0, "cpu")
    dd = to_device(inp)
    o, st, ck = kda.chunk_prefill_ckpt(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"], dd["S0"],
                                       chunk=64, ckpt_every=every)
    p = every
    tail = {k: v[:, p:].contiguous() for k, v in dd.items() if k != "S0"}
    o_r, st_r = kda.chunk_prefill(tail["q"], tail["k"], tail["v"], tail["log_alpha"], tail["beta"],
                                  ck[:, 0].contiguous(), chunk=64)
    torch.cuda.synchronize()
    assert_close("resumed o", o_r, to_f64(o[:, p:]), "bf16")
    assert_close("resumed S_T", st_r, to_f64(st), "bf16")
