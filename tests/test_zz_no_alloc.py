"""kda_chunk_fwd_gated_noalloc against kda_chunk_fwd_gated, through the C ABI.

The no-allocation entry point runs the same kernels with the library's fixed
device scratch as its workspace, so with the same segment count its outputs
and final states equal the workspace call's bit for bit.  Each case makes two
calls in a row, the second smaller, so the second runs over the scratch the
first left behind.  Covered: the sequence split (explicit and automatic
segment counts, whose per-segment states live in the scratch), a shape
without the fused gate (g staged in the scratch), and sizes whose explicit
split exceeds the scratch (an error before any launch).
"""
import pytest
import torch

from linear_attention_sequence_gate_amd import _lib, inputs
from kda_testutil import say

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16


def _pair(x, flags):
    """(o, S_T) of the workspace call and of the no-allocation call."""
    o_ref, S_ref = _lib.kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"],
                                            x["S0"], flags=flags)
    B, T, H, _ = x["q"].shape
    dk, dv = x["q"].shape[-1], x["v"].shape[-1]
    o = torch.empty((B, T, H, dv), device="cuda", dtype=x["q"].dtype)
    S = torch.empty((B, H, dk, dv), device="cuda", dtype=torch.float32)
    o2, S2 = _lib.kda_chunk_fwd_gated_noalloc(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"],
                                              x["S0"], final_state=S, o=o, flags=flags)
    torch.cuda.synchronize()
    assert o2 is o and S2 is S
    return (o_ref, S_ref), (o, S)


def _check_equal(label, ref, got):
    (o_ref, S_ref), (o, S) = ref, got
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all(), label
    assert torch.equal(o, o_ref), label
    assert torch.equal(S, S_ref), label


@pytest.mark.parametrize("cases", [
    # (B, T, H, segments): explicit splits, the second call smaller
    ((1, 5000, 2, 4), (1, 3000, 2, 3)),
    # automatic count: B1 H4 T40000 splits (its buffers fit the scratch), then a
    # one-pass call
    ((1, 40000, 4, 0), (2, 700, 3, 0)),
])
def test_noalloc_split_equals_workspace_call(cases):
    for i, (B, T, H, nseg) in enumerate(cases):
        flags = _lib.kda_flag_segments(nseg)
        auto = _lib.kda_chunk_fwd_auto_segments(B, T, H, 128, 128, _lib.KDA_BF16)
        say("noalloc split", i, "B", B, "T", T, "H", H, "segments", nseg or f"auto={auto}")
        x = inputs.make_prefill_inputs(B, T, H, 128, 128, BF16, 900 + i + T, device="cuda",
                                       s0_std=0.02, stress_heads_mean=3.0)
        ref, got = _pair(x, flags)
        _check_equal(f"split call {i}", ref, got)


def test_noalloc_staged_gate_equals_workspace_call():
    """fp32, dk = dv = 64: no fused gate, so g is staged in the scratch."""
    for i, (B, T, H) in enumerate(((2, 400, 3), (1, 150, 3))):
        say("noalloc staged gate", i, "B", B, "T", T, "H", H)
        x = inputs.make_prefill_inputs(B, T, H, 64, 64, torch.float32, 950 + i, device="cuda",
                                       s0_std=0.1)
        ref, got = _pair(x, 0)
        _check_equal(f"staged-gate call {i}", ref, got)


def test_noalloc_rejects_a_split_beyond_the_scratch():
    """B4 H32 T8192 d128 in 8 segments needs about 160 MB of per-segment
    states: rejected before any launch, the outputs untouched; the same sizes
    in one pass need no scratch and run."""
    B, T, H = 4, 8192, 32
    say("noalloc too large")
    x = inputs.make_prefill_inputs(B, T, H, 128, 128, BF16, 960, device="cuda")
    need = _lib.kda_chunk_fwd_workspace_size(B, T, H, 128, 128, _lib.KDA_BF16, 8)
    assert need > _lib.KDA_NOALLOC_SCRATCH_BYTES
    o = torch.full((B, T, H, 128), 7.0, device="cuda", dtype=BF16)
    with pytest.raises(_lib.KdaError) as err:
        _lib.kda_chunk_fwd_gated_noalloc(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"],
                                         o=o, flags=_lib.kda_flag_segments(8))
    assert err.value.code == _lib.KDA_ERR_INVALID_ARGUMENT
    assert "scratch" in str(err.value)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
    ref, got = _pair(x, _lib.kda_flag_segments(1))
    _check_equal("one pass at the rejected size", ref, got)
