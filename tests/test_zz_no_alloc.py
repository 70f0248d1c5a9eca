"""The allocation-free prefill (kda_chunk_prefill_noalloc) against kda_chunk_prefill_ex.

Two calls in a row through the C ABI, the second on a smaller input, each a sequence split whose
transitions, increments and entry states live in the library's fixed device array; a third call
that needs no scratch.  Each result must equal, bit for bit, the same prefill through
kda_chunk_prefill_ex with a caller workspace (the same kernels on the same plan), and both must
meet the bf16 parity bar against the float64 oracle.  Outputs start as NaN, so an element that a
call never writes cannot pass.
"""
import pytest
import torch

import oracle
from chunked_gated_delta_13_amd import inputs as gen
from tests.parity import assert_close, nan_like, to_device

pytestmark = pytest.mark.gpu


def _kda():
    import chunked_gated_delta_13_amd as kda
    kda.load_library()
    return kda


# (B, T, H, seg_len): an explicit 8-segment split, then a smaller one on the automatic plan,
# then a short sequence that is not split at all
CALLS = [(1, 8192, 2, 1024), (1, 3000, 1, 0), (2, 300, 2, 0)]


def test_noalloc_matches_workspace_prefill_twice():
    kda = _kda()
    for i, (B, T, H, seg) in enumerate(CALLS):
        print(f"noalloc call {i}: B={B} T={T} H={H} seg_len={seg}", flush=True)
        inp = gen.make_prefill_inputs(B, T, H, 128, 128, "bf16", "slow", 1.0, seed=90 + i)
        d = to_device(inp)
        need = kda.prefill_workspace_bytes(B, T, H, 128, 128, 64, seg_len=seg)
        if i < 2:
            assert need > 0, "these calls are meant to split the sequence"
        o_na = nan_like(d["v"])
        s_na = nan_like(d["S0"])
        kda.chunk_prefill_noalloc(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"],
                                  chunk=64, seg_len=seg, o=o_na, S_T=s_na)
        o_ws = nan_like(d["v"])
        s_ws = nan_like(d["S0"])
        kda.chunk_prefill(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], chunk=64,
                          seg_len=seg, o=o_ws, S_T=s_ws)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ws) and torch.equal(s_na, s_ws)
        o_ref, s_ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"],
                                      inp["S0"])
        assert_close("o", o_na, o_ref, "bf16")
        assert_close("S_T", s_na, s_ref, "bf16")
