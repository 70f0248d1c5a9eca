"""The allocation-free prefill under HIP graph capture: the callers it exists for.

A sequence split through kda_chunk_prefill_noalloc issues kernels only, all on the caller's
stream (no allocation, no memset, no second stream), so it can be captured into a graph.  The
graph is replayed several times, with the program's own eager work and synchronisations between
the replays, and every replay must give the same bits as the eager call.
"""
import pytest
import torch

from chunked_gated_delta_13_amd import inputs as gen
from tests.parity import nan_like, to_device

pytestmark = pytest.mark.gpu


def _kda():
    import chunked_gated_delta_13_amd as kda
    kda.load_library()
    return kda


@pytest.mark.parametrize("T,H,seg,decay", [(3000, 2, 512, "sig2"),    # transitions die: short reruns
                                           (2000, 2, 256, "slow"),    # transitions live: full split
                                           (700, 3, 0, "sig2")])      # no split
def test_noalloc_prefill_replays_in_a_graph(T, H, seg, decay):
    kda = _kda()
    print(f"graph capture T={T} H={H} seg={seg} {decay}", flush=True)
    d = to_device(gen.make_prefill_inputs(1, T, H, 128, 128, "bf16", decay, 1.0, 500 + T, 0.0, "cpu"))

    def call(o, st):
        kda.chunk_prefill_noalloc(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], chunk=64,
                                  seg_len=seg, o=o, S_T=st)

    o_ref, st_ref = nan_like(d["v"]), nan_like(d["S0"])
    call(o_ref, st_ref)          # eager (also looks up the scratch array's address once)
    torch.cuda.synchronize()
    assert torch.isfinite(o_ref.float()).all() and torch.isfinite(st_ref).all()

    o, st = torch.empty_like(o_ref), torch.empty_like(st_ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # a warm-up on a side stream before capture
        call(o, st)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(o, st)
    for i in range(3):
        o.fill_(float("nan"))        # eager work between replays
        st.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(st, st_ref), f"replay {i}"
