"""One workgroup per chain (all 128 state columns, each chunk's operands
formed once) against one per 64-column slice: every state column runs the
same arithmetic on the same operand tiles in both layouts, so outputs and
final states are bit-identical -- in one pass and in both sequence-split
schemes (a split that stopped at a different chunk would differ by
rounding), with the gate fused or g given, ragged lengths, an initial state
or none, in-place continuation, pooled states and packed sequences.  Also
against the oracle on its own, and the plan the library picks."""
import pytest
import torch

import oracle
from linear_attention_sequence_gate_amd import (_lib, kda_chunk_fwd, kda_chunk_fwd_gated,
                                                 kda_chunk_fwd_pooled, kda_chunk_fwd_varlen_pooled_gated,
                                                 kda_gate, inputs)
from kda_testutil import TOL, prefill_device, rho, say

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16
CH, SL = _lib.KDA_FLAG_WORKGROUP_PER_CHAIN, _lib.KDA_FLAG_WORKGROUP_PER_SLICE
seg = _lib.kda_flag_segments
RERUN = _lib.KDA_FLAG_SPLIT_FULL_RERUN


def _both(fn):
    """fn(layout_flag) -> (o, S) for both layouts, compared bit for bit (the
    callers fix the segment count: the library may pick another for each
    layout)."""
    a = fn(SL)
    b = fn(CH)
    torch.cuda.synchronize()
    for x, y, name in ((a[0], b[0], "o"), (a[1], b[1], "S")):
        if x is None:
            continue
        d = (x.float() - y.float()).abs().max().item()
        assert torch.equal(x, y), (name, d)
    return b


@pytest.mark.parametrize("T", [1, 31, 32, 33, 700, 2011])
@pytest.mark.parametrize("gated", [True, False])
def test_one_pass_bit_identical(T, gated):
    say("wide one pass", T, gated)
    x = prefill_device(2, T, 3, 128, 128, BF16, 1200 + T, s0_std=0.3 if T % 2 else 0.0)
    g = kda_gate(x["z"], x["A"]) if not gated else None

    def run(lay):
        if gated:
            return kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"], x["S0"],
                                       flags=lay | seg(1))
        return kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], x["S0"], flags=lay | seg(1))
    _both(run)


@pytest.mark.parametrize("P,rerun", [(2, False), (3, False), (5, False), (3, True), (6, True)])
@pytest.mark.parametrize("gated", [True, False])
def test_split_bit_identical(P, rerun, gated):
    say("wide split", P, rerun, gated)
    x = prefill_device(1, 3000, 4, 128, 128, BF16, 1300 + P, s0_std=0.3)
    # head 1 keeps memory (its transitions never vanish), the others decay
    z = x["z"].float()
    z[:, :, 1] -= 6.0
    x["z"] = z.to(BF16)
    g = kda_gate(x["z"], x["A"]) if not gated else None
    fl = seg(P) | (RERUN if rerun else 0)

    def run(lay):
        if gated:
            return kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"], x["S0"],
                                       flags=lay | fl)
        return kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], x["S0"], flags=lay | fl)
    _both(run)


def test_in_place_continuation_and_no_state():
    say("wide in place")
    x = prefill_device(1, 1500, 2, 128, 128, BF16, 1400, s0_std=0.3)
    h = 600
    part = {n: x[n][:, :h].contiguous() for n in ("q", "k", "v", "z", "beta")}
    rest = {n: x[n][:, h:].contiguous() for n in ("q", "k", "v", "z", "beta")}

    def run(lay):
        S = x["S0"].clone()
        o1, _ = kda_chunk_fwd_gated(part["q"], part["k"], part["v"], part["z"], x["A"], part["beta"],
                                    S, final_state=S, flags=lay | seg(1))
        o2, _ = kda_chunk_fwd_gated(rest["q"], rest["k"], rest["v"], rest["z"], x["A"], rest["beta"],
                                    S, final_state=S, flags=lay | seg(3))
        o3, S3 = kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"], None,
                                     flags=lay | seg(2))
        return torch.cat([o1, o2, o3], 1), torch.cat([S, S3])
    _both(run)


def test_pooled_bit_identical():
    say("wide pooled")
    n_slots, H, T = 6, 2, 400
    x = prefill_device(3, T, H, 128, 128, BF16, 1500)
    g = kda_gate(x["z"], x["A"])
    gen = torch.Generator(device="cuda").manual_seed(1501)
    pool0 = torch.randn(n_slots, H, 128, 128, device="cuda", generator=gen) * 0.3
    slots = torch.tensor([4, -1, 2], dtype=torch.int32, device="cuda")

    def run(lay):
        pool = pool0.clone()
        o = torch.full((3, T, H, 128), 5.0, device="cuda", dtype=BF16)
        kda_chunk_fwd_pooled(x["q"], x["k"], x["v"], g, x["beta"], pool, slots, o=o, flags=lay | seg(2))
        return o, pool
    o, pool = _both(run)
    assert (o[1] == 5.0).all()
    assert torch.equal(pool[[0, 1, 3, 5]], pool0[[0, 1, 3, 5]])


def test_varlen_bit_identical():
    say("wide varlen")
    lens = [1, 200, 33, 1024, 7]
    total, H = sum(lens), 2
    x = prefill_device(1, total, H, 128, 128, BF16, 1600)
    cu = torch.tensor([0] + list(torch.tensor(lens).cumsum(0)), dtype=torch.int64, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(1601)
    pool0 = torch.randn(len(lens), H, 128, 128, device="cuda", generator=gen) * 0.3
    slots = torch.arange(len(lens), dtype=torch.int32, device="cuda")

    def run(lay):
        pool = pool0.clone()
        o = kda_chunk_fwd_varlen_pooled_gated(x["q"][0], x["k"][0], x["v"][0], x["z"][0], x["A"],
                                              x["beta"][0], pool, slots, cu, flags=lay)
        return o, pool
    _both(run)


def test_wide_against_oracle():
    """Ragged length over many chunks, decay-stress heads, initial state; the
    per-chain layout forced in one pass and in a split."""
    say("wide vs oracle")
    x = prefill_device(2, 1337, 3, 128, 128, BF16, 1700, s0_std=0.3, stress=3.0)
    g_ref = oracle.gate(x["z"], x["A"])
    o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], g_ref, x["beta"], x["S0"])
    for fl in (CH | seg(1), CH | seg(3), CH | seg(4) | RERUN):
        o, S = kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"], x["S0"], flags=fl)
        torch.cuda.synchronize()
        ro, rs = rho(o, o_ref), rho(S, S_ref)
        print(f"    flags {fl:#x}: rho(o)={ro:.3e} rho(S)={rs:.3e}", flush=True)
        assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
        assert ro <= TOL[BF16] and rs <= TOL[BF16], (fl, ro, rs)


def test_library_plan_at_the_benchmark_size():
    """B4 H32 T32768: the library's choice is one workgroup per chain over
    two segments; the call with flags 0 gives what that forced plan gives,
    bit for bit (the full-size parity test checks it against the oracle)."""
    say("wide plan B4 H32")
    assert _lib.kda_chunk_fwd_plan(4, 32768, 32, 128, 128, _lib.KDA_BF16) == (2, True)
    w = inputs.WORKLOADS["prefill_b4_h32_t32k"]
    x = inputs.workload_prefill_inputs(w, device="cuda", T=4096)
    P, wide = _lib.kda_chunk_fwd_plan(4, 4096, 32, 128, 128, _lib.KDA_BF16)
    o0, S0 = kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"], x["S0"])
    o1, S1 = kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"], x["S0"],
                                 flags=seg(P) | (CH if wide else SL))
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(S0, S1)


@pytest.mark.parametrize("P", [2, 3])
def test_split_filling_the_gpu_bit_identical(P):
    """A split whose segment workgroups alone fill the GPU runs its
    transitions in a launch of their own before the segments: both layouts
    still agree bit for bit, and with the oracle on sampled chains."""
    say("wide split filling the GPU", P)
    B, T, H = 4, 1500, 32                           # 128 chains: P x 128 or P x 256 workgroups
    x = inputs.make_prefill_inputs(B, T, H, 128, 128, BF16, 1800 + P, device="cuda", s0_std=0.1,
                                   stress_heads_mean=3.0)
    z = x["z"].float()
    z[:, :, 5] -= 12.0                              # head 5 keeps memory in every sequence
    x["z"] = z.to(BF16)

    def run(lay):
        return kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"], x["S0"],
                                   flags=lay | seg(P))
    o, S = _both(run)
    for b, h in ((0, 5), (3, 0), (2, 17)):
        xs = {n: x[n][b:b + 1, :, h:h + 1].contiguous() for n in ("q", "k", "v", "z", "beta")}
        g_ref = oracle.gate(xs["z"], x["A"][h:h + 1].contiguous())
        o_ref, S_ref = oracle.forward(xs["q"], xs["k"], xs["v"], g_ref, xs["beta"],
                                      x["S0"][b:b + 1, h:h + 1].contiguous())
        ro, rs = rho(o[b:b + 1, :, h:h + 1], o_ref), rho(S[b:b + 1, h:h + 1], S_ref)
        assert ro <= TOL[BF16] and rs <= TOL[BF16], (b, h, ro, rs)
