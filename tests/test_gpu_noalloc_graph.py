"""kda_chunk_fwd_gated_noalloc under HIP graph capture, the use it exists for.

The call is captured once into a graph (after one eager call, which also sets
up the library's per-device scratch) and the graph is replayed several times.
Between replays the program does its own eager work: it clears the graph's
output tensors with fill kernels and makes another no-allocation call on
different inputs, which reuses the same scratch.  Every replay must equal the
eager result bit for bit.  Cases: a long few-chain shape that takes the
sequence split in 15 segments (its three kernels and the chaining between
them write the scratch), a short one split in 4, and a one-pass shape."""
import pytest
import torch

from linear_attention_sequence_gate_amd import _lib, inputs
from kda_testutil import say

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16


def _noalloc(x, o, S):
    return _lib.kda_chunk_fwd_gated_noalloc(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"],
                                            x["S0"], final_state=S, o=o)


def _outputs(x):
    B, T, H, _ = x["q"].shape
    dk, dv = x["q"].shape[-1], x["v"].shape[-1]
    return (torch.empty((B, T, H, dv), device="cuda", dtype=x["q"].dtype),
            torch.empty((B, H, dk, dv), device="cuda", dtype=torch.float32))


@pytest.mark.parametrize("B,T,H,nseg", [(1, 6000, 2, 12), (2, 700, 4, 4), (8, 700, 16, 1)])
def test_noalloc_call_replays_in_a_captured_graph(B, T, H, nseg):
    segs = _lib.kda_chunk_fwd_auto_segments(B, T, H, 128, 128, _lib.KDA_BF16)
    say("noalloc graph", f"B{B} T{T} H{H}", f"segments {segs}")
    assert segs == nseg
    x = inputs.make_prefill_inputs(B, T, H, 128, 128, BF16, 950 + T, device="cuda", s0_std=0.02)
    other = inputs.make_prefill_inputs(1, 3000, 2, 128, 128, BF16, 951, device="cuda", s0_std=0.02)
    o_e, S_e = _outputs(x)
    _noalloc(x, o_e, S_e)
    o_x, S_x = _outputs(other)
    torch.cuda.synchronize()

    o_g, S_g = _outputs(x)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            _noalloc(x, o_g, S_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(3):
        o_g.zero_()
        S_g.zero_()
        _noalloc(other, o_x, S_x)          # eager use of the same scratch in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), ("o", rep)
        assert torch.equal(S_g, S_e), ("S", rep)
    assert torch.isfinite(o_e.float()).all() and torch.isfinite(S_e).all()
