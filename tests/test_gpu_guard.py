"""The guarded two-segment split: where the library picks two segments of
one workgroup per chain and one pass would be faster if no transition
vanished, a probe launch runs each chain's second-segment transition for a
few chunks and the device takes the split only if every one vanished there,
else the one pass.  With vanishing gates the call equals the forced split
bit for bit, with gates that keep memory (in every chain, or in one) the
forced one pass; one captured graph follows the data on every replay; and
the result is within the bar of the oracle."""
import pytest
import torch

import oracle
from linear_attention_sequence_gate_amd import _lib, kda_chunk_fwd, kda_chunk_fwd_gated, kda_gate, inputs
from kda_testutil import TOL, rho, say

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16
CH, SL, seg = _lib.KDA_FLAG_WORKGROUP_PER_CHAIN, _lib.KDA_FLAG_WORKGROUP_PER_SLICE, _lib.kda_flag_segments
B, T, H = 16, 4096, 8              # 128 chains: two segments fill the GPU


def _inputs(seed):
    return inputs.make_prefill_inputs(B, T, H, 128, 128, BF16, seed, device="cuda", s0_std=0.1,
                                      stress_heads_mean=3.0)


def _keep_memory(x, chains=None):
    """z - 12 (g about -3e-5 per token) in the given (b, h) chains, or all."""
    z = x["z"].float()
    if chains is None:
        z -= 12.0
    else:
        for b, h in chains:
            z[b, :, h] -= 12.0
    return dict(x, z=z.to(BF16))


def _run(x, flags, ws=None):
    return kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"], x["S0"], flags=flags,
                               workspace=ws)


def test_plan_is_guarded():
    assert _lib.kda_chunk_fwd_plan(B, T, H, 128, 128, _lib.KDA_BF16, with_guard=True) == (2, True, True)
    assert _lib.kda_chunk_fwd_plan(4, 32768, 32, 128, 128, _lib.KDA_BF16, with_guard=True) == (2, True, True)
    # an explicit count, or another scheme, is never guarded
    assert _lib.kda_chunk_fwd_plan(B, T, H, 128, 128, _lib.KDA_BF16, seg(2), with_guard=True)[2] is False
    assert _lib.kda_chunk_fwd_plan(B, T, H, 128, 128, _lib.KDA_BF16, _lib.KDA_FLAG_SPLIT_FULL_RERUN,
                                   with_guard=True)[2] is False
    # the fallback: one pass in 64-column slices
    assert _lib.kda_chunk_fwd_plan(B, T, H, 128, 128, _lib.KDA_BF16, seg(1)) == (1, False)


@pytest.mark.parametrize("case", ["vanishing", "all_keep_memory", "one_chain_keeps_memory"])
def test_guard_takes_the_split_or_the_one_pass(case):
    say("guard", case)
    x = _inputs(2100)
    if case == "all_keep_memory":
        x = _keep_memory(x)
    elif case == "one_chain_keeps_memory":
        x = _keep_memory(x, [(11, 5)])
    got = _run(x, 0)
    ref = _run(x, CH | seg(2)) if case == "vanishing" else _run(x, SL | seg(1))
    torch.cuda.synchronize()
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), case


def test_guard_with_g_input():
    say("guard, g input")
    x = _keep_memory(_inputs(2200), [(0, 0)])
    g = kda_gate(x["z"], x["A"])
    got = kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], x["S0"])
    ref = kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], x["S0"], flags=SL | seg(1))
    x2 = _inputs(2201)
    g2 = kda_gate(x2["z"], x2["A"])
    got2 = kda_chunk_fwd(x2["q"], x2["k"], x2["v"], g2, x2["beta"], x2["S0"])
    ref2 = kda_chunk_fwd(x2["q"], x2["k"], x2["v"], g2, x2["beta"], x2["S0"], flags=CH | seg(2))
    torch.cuda.synchronize()
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
    assert torch.equal(got2[0], ref2[0]) and torch.equal(got2[1], ref2[1])


def test_guard_in_a_captured_graph_follows_the_data():
    """Captured once with vanishing gates; the replays see z rewritten in
    place to gates that keep memory and back: each replay takes the path its
    data asks for (the probe and the guards decide on the device)."""
    say("guard in a graph")
    x = _inputs(2300)
    z_fast = x["z"].clone()
    z_slow = _keep_memory(x, [(3, 2)])["z"]
    z = x["z"]                                        # the buffer the graph reads
    o = torch.empty(B, T, H, 128, device="cuda", dtype=BF16)
    S = torch.empty(B, H, 128, 128, device="cuda")
    ws = torch.empty(_lib.kda_chunk_fwd_gated_workspace_size(B, T, H, 128, 128, _lib.KDA_BF16),
                     device="cuda", dtype=torch.uint8)
    expect = {}
    for name, zz, fl in (("fast", z_fast, CH | seg(2)), ("slow", z_slow, SL | seg(1))):
        z.copy_(zz)
        expect[name] = _run(x, fl, ws)
        torch.cuda.synchronize()
        expect[name] = (expect[name][0].clone(), expect[name][1].clone())
    z.copy_(z_fast)
    run = lambda: kda_chunk_fwd_gated(x["q"], x["k"], x["v"], z, x["A"], x["beta"], x["S0"],
                                      final_state=S, o=o, workspace=ws)
    run()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for name in ("slow", "fast", "slow", "fast"):
        z.copy_(z_fast if name == "fast" else z_slow)
        o.zero_()
        S.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, expect[name][0]) and torch.equal(S, expect[name][1]), name


def test_guard_against_the_oracle():
    """Both paths of the guard against the fp64 oracle on 16 of the 128
    chains (every token, and the final states)."""
    say("guard vs oracle")
    for case in ("vanishing", "one_chain_keeps_memory"):
        x = _inputs(2400)
        if case != "vanishing":
            x = _keep_memory(x, [(1, 1)])
        o, S = _run(x, 0)
        torch.cuda.synchronize()
        sel = [(b, h) for b in (0, 1, 7, 15) for h in (0, 1, 4, 7)]
        for b, h in sel:
            xs = {n: x[n][b:b + 1, :, h:h + 1].contiguous() for n in ("q", "k", "v", "z", "beta")}
            g_ref = oracle.gate(xs["z"], x["A"][h:h + 1].contiguous())
            o_ref, S_ref = oracle.forward(xs["q"], xs["k"], xs["v"], g_ref, xs["beta"],
                                          x["S0"][b:b + 1, h:h + 1].contiguous())
            ro = rho(o[b:b + 1, :, h:h + 1], o_ref)
            rs = rho(S[b:b + 1, h:h + 1], S_ref)
            assert ro <= TOL[BF16] and rs <= TOL[BF16], (case, b, h, ro, rs)
        print(f"    {case}: 16 chains within the bar", flush=True)


def test_guard_with_a_skipped_slot():
    """A pooled call at a guarded size whose last sequence's slot lies outside
    the pool: the skipped sequence's transition records read as vanished, so
    the call equals the forced split on the same pool bit for bit, and the
    other slots are untouched."""
    from linear_attention_sequence_gate_amd import kda_chunk_fwd_pooled
    say("guard, pooled with a skipped slot")
    x = _inputs(2500)
    g = kda_gate(x["z"], x["A"])
    n_slots = B + 2
    gen = torch.Generator(device="cuda").manual_seed(2501)
    pool0 = torch.randn(n_slots, H, 128, 128, device="cuda", generator=gen) * 0.1
    slots = torch.tensor(list(range(2, B + 1)) + [-7], dtype=torch.int32, device="cuda")
    out = {}
    for name, fl in (("plan", 0), ("split", CH | seg(2))):
        pool = pool0.clone()
        o = torch.full((B, T, H, 128), 3.0, device="cuda", dtype=BF16)
        kda_chunk_fwd_pooled(x["q"], x["k"], x["v"], g, x["beta"], pool, slots, o=o, flags=fl)
        torch.cuda.synchronize()
        out[name] = (o, pool)
    assert torch.equal(out["plan"][0], out["split"][0]) and torch.equal(out["plan"][1], out["split"][1])
    assert (out["plan"][0][B - 1] == 3.0).all()
    assert torch.equal(out["plan"][1][[0, 1]], pool0[[0, 1]])


@pytest.mark.parametrize("case", ["vanishing", "one_chain_keeps_memory"])
def test_guard_at_dv64(case):
    """dv = 64 (64-column slices only): the guarded split and its one-pass
    fallback run in that layout; bit-equal to the forced split or the forced
    one pass, and within the bar of the oracle on sampled chains."""
    say("guard dv=64", case)
    assert _lib.kda_chunk_fwd_plan(B, T, H, 128, 64, _lib.KDA_BF16, with_guard=True) == (2, False, True)
    x = inputs.make_prefill_inputs(B, T, H, 128, 64, BF16, 2600, device="cuda", s0_std=0.1,
                                   stress_heads_mean=3.0)
    if case != "vanishing":
        x = _keep_memory(x, [(9, 3)])
    got = _run(x, 0)
    ref = _run(x, seg(2)) if case == "vanishing" else _run(x, seg(1))
    torch.cuda.synchronize()
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), case
    o, S = got
    for b, h in ((9, 3), (0, 0), (15, 7)):
        xs = {n: x[n][b:b + 1, :, h:h + 1].contiguous() for n in ("q", "k", "v", "z", "beta")}
        g_ref = oracle.gate(xs["z"], x["A"][h:h + 1].contiguous())
        o_ref, S_ref = oracle.forward(xs["q"], xs["k"], xs["v"], g_ref, xs["beta"],
                                      x["S0"][b:b + 1, h:h + 1].contiguous())
        ro, rs = rho(o[b:b + 1, :, h:h + 1], o_ref), rho(S[b:b + 1, h:h + 1], S_ref)
        assert ro <= TOL[BF16] and rs <= TOL[BF16], (case, b, h, ro, rs)
