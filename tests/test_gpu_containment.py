"""A NaN in one chain's inputs stays in that chain: every other (sequence,
head) chain's outputs and final state are bit-identical to a clean run.  The
chains share no arithmetic in any kernel (the dv-slice workgroups of a chain,
the sequence split's transitions and chaining, and the decode step all work
per chain), so this holds exactly.  Covered: the fused prefill and the gate
followed by the chunk kernel in one pass, a forced sequence split in both
schemes (the poisoned segment's transition is never exactly zero, so its last
phase runs whole), and the decode step.  Inside the poisoned chain a one-pass
call carries the NaN in the state to the end; a split drops it at the next
segment whose transition vanished (M = 0 is applied by taking L), so its
final state need not be NaN."""
import pytest
import torch

from linear_attention_sequence_gate_amd import (_lib, kda_chunk_fwd, kda_chunk_fwd_gated,
                                                 kda_decode_step, kda_gate, inputs)
from kda_testutil import prefill_device, say

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16


def _others_equal(a, b, bad_b, bad_h, head_axis, nan=True):
    """a and b agree bit for bit outside chain (bad_b, bad_h); with `nan`, a's
    copy of that chain holds a NaN."""
    for bi in range(a.shape[0]):
        for hi in range(a.shape[head_axis]):
            if (bi, hi) != (bad_b, bad_h):
                sa = a[bi].select(head_axis - 1, hi)
                sb = b[bi].select(head_axis - 1, hi)
                assert torch.equal(sa, sb), (bi, hi)
    if nan:
        assert torch.isnan(a[bad_b].select(head_axis - 1, bad_h).float()).any()


@pytest.mark.parametrize("path", ["gated", "two_kernel", "split_stop", "split_rerun"])
def test_prefill_nan_stays_in_its_chain(path):
    say("containment prefill", path)
    B, T, H = 2, 1500, 3
    x = prefill_device(B, T, H, 128, 128, BF16, 990, s0_std=0.02)
    bad_b, bad_h, bad_t = 1, 2, 700
    xp = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in x.items()}
    xp["q"][bad_b, bad_t, bad_h, 5] = float("nan")
    xp["k"][bad_b, bad_t + 3, bad_h, 9] = float("nan")
    split = path.startswith("split")
    flags = _lib.kda_flag_segments(5 if split else 1)
    if path == "split_rerun":
        flags |= _lib.KDA_FLAG_SPLIT_FULL_RERUN

    def run(inp):
        if path == "two_kernel":
            g = kda_gate(inp["z"], inp["A"])
            return kda_chunk_fwd(inp["q"], inp["k"], inp["v"], g, inp["beta"], inp["S0"], flags=flags)
        return kda_chunk_fwd_gated(inp["q"], inp["k"], inp["v"], inp["z"], inp["A"], inp["beta"],
                                   inp["S0"], flags=flags)

    o_c, S_c = run(x)
    o_p, S_p = run(xp)
    torch.cuda.synchronize()
    _others_equal(o_p, o_c, bad_b, bad_h, head_axis=2)     # o [B, T, H, dv]
    assert torch.isnan(o_p[bad_b, bad_t, bad_h].float()).any()
    _others_equal(S_p, S_c, bad_b, bad_h, head_axis=1, nan=not split)   # S [B, H, dk, dv]


def test_decode_nan_stays_in_its_state():
    say("containment decode")
    N, H = 16, 4
    st = inputs.make_decode_state(N, H, 128, 128, 991, device="cuda")
    x = inputs.make_decode_step_inputs(N, H, 128, 128, BF16, 991, 0, device="cuda")
    bad_n, bad_h = 5, 1
    S_c = st["S"].clone()
    S_p = st["S"].clone()
    S_p[bad_n, bad_h, 3, 7] = float("nan")
    o_c = kda_decode_step(x["q"], x["k"], x["v"], x["z"], st["A"], x["beta"], S_c)
    o_p = kda_decode_step(x["q"], x["k"], x["v"], x["z"], st["A"], x["beta"], S_p)
    torch.cuda.synchronize()
    _others_equal(o_p, o_c, bad_n, bad_h, head_axis=1)     # o [N, H, dv]
    _others_equal(S_p, S_c, bad_n, bad_h, head_axis=1)     # state [N, H, dk, dv]
