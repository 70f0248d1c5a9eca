"""Prefill with the fused bounded gate on the device vs the float64 oracle.

The decay input is the raw gate pre-activation x (bf16, N(0, 2)); the kernel
forms log alpha = -5 * sigmoid(x) on load.  Every call goes through the C ABI.
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


@pytest.mark.parametrize("B,T,chunk,seg,decay", [(2, 700, 64, 0, "sig2"), (2, 1000, 64, 256, "slow"),
                                                 (2, 1000, 64, 256, "sig2"),   # split, transitions die
                                                 (2, 333, 32, 0, "sig2"), (2, 200, 16, 0, "sig2"),
                                                 (1, 12288, 64, 0, "slow")])   # automatic split
def test_prefill_gate_matches_oracle(B, T, chunk, seg, decay):
    kda = _kda()
    print(f"gate B={B} T={T} chunk={chunk} seg={seg}", flush=True)
    inp = gen.make_prefill_inputs(B, T, 2, 128, 128, "bf16", decay, 1.0, 110 + T, 0.0, "cpu")
    g = gen.make_gate(B, T, 2, 128, "bf16", seed=110 + T)
    if decay == "slow":
        g = (g.float() - 8.0).to(torch.bfloat16)    # long memory: sigmoid(x) small
    dd = to_device(inp)
    o, st = kda.chunk_prefill_gate(dd["q"], dd["k"], dd["v"], g.cuda(), dd["beta"], dd["S0"], chunk=chunk,
                                   seg_len=seg, o=nan_like(dd["v"]), S_T=nan_like(dd["S0"]))
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.prefill_gate(inp["q"], inp["k"], inp["v"], g, inp["beta"], inp["S0"])
    assert_close("o", o, o_ref, "bf16")
    assert_close("S_T", st, s_ref, "bf16")


def test_prefill_gate_unsupported_shapes_raise():
    kda = _kda()
    inp = to_device(gen.make_prefill_inputs(1, 64, 1, 64, 64, "bf16", "sig2", 0.0, 1, 0.0, "cpu"))
    g = torch.zeros((1, 64, 1, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError):
        kda.chunk_prefill_gate(inp["q"], inp["k"], inp["v"], g, inp["beta"])
