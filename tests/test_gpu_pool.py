"""GPU checks of the slot-indexed state pool: the pooled calls equal the plain
calls bit for bit on states gathered from the slots, slots outside the pool
are skipped, reset zeroes only its slots, and a continuous-batching run
(requests joining and leaving between decode steps) matches the oracle on
each request's whole token stream."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_gate_amd import (_lib, inputs, kda_chunk_fwd, kda_chunk_fwd_pooled,
                                                kda_chunk_fwd_varlen_pooled, kda_decode_step,
                                                kda_decode_step_pooled, kda_gate,
                                                kda_state_pool_reset)
from kda_testutil import TOL, rho, say

pytestmark = pytest.mark.gpu


def _pool(n_slots, H, dk, dv, seed):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn(n_slots, H, dk, dv, device="cuda", generator=gen) * 0.02


def _slots(lst):
    return torch.tensor(lst, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("dtype,dk,dv", [(torch.float32, 64, 64), (torch.bfloat16, 128, 128),
                                         (torch.bfloat16, 32, 64)])
def test_pooled_decode_equals_plain_on_gathered_states(dtype, dk, dv):
    say("pooled decode", dtype, dk, dv)
    n_slots, H = 10, 3
    slots = [7, 2, 9, 0]
    pool = _pool(n_slots, H, dk, dv, 500)
    before = pool.clone()
    S = pool[slots].clone()
    A = inputs.make_decode_state(len(slots), H, dk, dv, 501, device="cuda")["A"]
    for t in range(3):
        x = inputs.make_decode_step_inputs(len(slots), H, dk, dv, dtype, 501, t, device="cuda")
        o_ref = kda_decode_step(x["q"], x["k"], x["v"], x["z"], A, x["beta"], S)
        o = kda_decode_step_pooled(x["q"], x["k"], x["v"], x["z"], A, x["beta"], pool, _slots(slots))
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref)
        assert torch.equal(pool[slots], S)
    others = [i for i in range(n_slots) if i not in slots]
    assert torch.equal(pool[others], before[others])


def test_pooled_decode_skips_slots_outside_the_pool():
    say("pooled decode, invalid slots")
    n_slots, H, dk, dv = 6, 2, 64, 64
    slots = [3, -1, 6, 5]
    pool = _pool(n_slots, H, dk, dv, 502)
    before = pool.clone()
    A = inputs.make_decode_state(4, H, dk, dv, 503, device="cuda")["A"]
    x = inputs.make_decode_step_inputs(4, H, dk, dv, torch.float32, 503, 0, device="cuda")
    o = torch.full((4, H, dv), 7.0, device="cuda")
    kda_decode_step_pooled(x["q"], x["k"], x["v"], x["z"], A, x["beta"], pool, _slots(slots), o=o)
    S = before[[3, 5]].clone()
    o_ref = kda_decode_step(x["q"][[0, 3]].contiguous(), x["k"][[0, 3]].contiguous(),
                            x["v"][[0, 3]].contiguous(), x["z"][[0, 3]].contiguous(), A,
                            x["beta"][[0, 3]].contiguous(), S)
    torch.cuda.synchronize()
    assert torch.equal(o[[0, 3]], o_ref) and torch.equal(pool[[3, 5]], S)
    assert (o[[1, 2]] == 7.0).all()                      # skipped: output untouched
    assert torch.equal(pool[[0, 1, 2, 4]], before[[0, 1, 2, 4]])


@pytest.mark.parametrize("dtype,dk,dv,T,nseg", [(torch.bfloat16, 128, 128, 300, 1),
                                                (torch.bfloat16, 128, 64, 1000, 3),
                                                (torch.float32, 64, 64, 200, 1)])
def test_pooled_prefill_equals_plain_on_gathered_states(dtype, dk, dv, T, nseg):
    say("pooled prefill", dtype, dk, dv, T, nseg)
    n_slots, H = 8, 2
    slots = [4, 1, 6, -3]                                 # the last sequence is skipped
    x = inputs.make_prefill_inputs(4, T, H, dk, dv, dtype, 504, device="cuda")
    g = kda_gate(x["z"], x["A"])
    pool = _pool(n_slots, H, dk, dv, 505)
    before = pool.clone()
    flags = _lib.kda_flag_segments(nseg)
    S0 = pool[slots[:3]].clone()
    o_ref, S_ref = kda_chunk_fwd(x["q"][:3].contiguous(), x["k"][:3].contiguous(),
                                 x["v"][:3].contiguous(), g[:3].contiguous(),
                                 x["beta"][:3].contiguous(), S0, flags=flags)
    o = torch.zeros(4, T, H, dv, device="cuda", dtype=dtype)
    kda_chunk_fwd_pooled(x["q"], x["k"], x["v"], g, x["beta"], pool, _slots(slots), o=o, flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(o[:3], o_ref) and torch.equal(pool[slots[:3]], S_ref)
    assert (o[3] == 0).all()
    assert torch.equal(pool[[0, 2, 3, 5, 7]], before[[0, 2, 3, 5, 7]])


def test_pool_reset():
    say("pool reset")
    pool = _pool(7, 2, 32, 128, 506)
    before = pool.clone()
    kda_state_pool_reset(pool, _slots([5, 1, 9, -2]))
    torch.cuda.synchronize()
    assert (pool[[1, 5]] == 0).all()
    assert torch.equal(pool[[0, 2, 3, 4, 6]], before[[0, 2, 3, 4, 6]])


@pytest.mark.parametrize("dtype,d", [(torch.float32, 64), (torch.bfloat16, 128)])
def test_continuous_batching_matches_the_oracle(dtype, d):
    """Three requests share a pool of six slots.  A (prompt 100) and B (prompt
    37) are prefilled, decode three steps together; C (prompt 64) joins for two
    steps (the batch order changes); A leaves and B, C decode two more.  Every
    output of each request is compared with the oracle over its whole stream."""
    say("continuous batching", dtype, d)
    H = 2
    n_slots = 6
    prompts = {"A": 100, "B": 37, "C": 64}
    n_dec = {"A": 5, "B": 7, "C": 4}
    slot_of = {"A": 2, "B": 5, "C": 0}
    reqs = {}
    A_gate = None
    for i, (r, p) in enumerate(prompts.items()):
        x = inputs.make_prefill_inputs(1, p + n_dec[r], H, d, d, dtype, 510 + i, device="cuda")
        if A_gate is None:
            A_gate = x["A"]
        reqs[r] = dict(x=x, pos=p, out=torch.empty(1, p + n_dec[r], H, d, device="cuda", dtype=dtype))
    pool = _pool(n_slots, H, d, d, 520)                   # stale contents from earlier requests

    def prefill(r):
        x, p = reqs[r]["x"], prompts[r]
        sl = lambda t: t[:, :p].contiguous()
        kda_state_pool_reset(pool, _slots([slot_of[r]]))
        g = kda_gate(sl(x["z"]), A_gate)
        o = kda_chunk_fwd_pooled(sl(x["q"]), sl(x["k"]), sl(x["v"]), g, sl(x["beta"]), pool,
                                 _slots([slot_of[r]]))
        reqs[r]["out"][:, :p] = o

    def decode(batch):
        pos = [reqs[r]["pos"] for r in batch]
        pick = lambda key: torch.stack([reqs[r]["x"][key][0, t] for r, t in zip(batch, pos)]).contiguous()
        o = kda_decode_step_pooled(pick("q"), pick("k"), pick("v"), pick("z"), A_gate, pick("beta"),
                                   pool, _slots([slot_of[r] for r in batch]))
        for i, r in enumerate(batch):
            reqs[r]["out"][0, reqs[r]["pos"]] = o[i]
            reqs[r]["pos"] += 1

    prefill("A")
    prefill("B")
    for _ in range(3):
        decode(["A", "B"])
    prefill("C")
    for _ in range(2):
        decode(["C", "A", "B"])
    for _ in range(2):
        decode(["B", "C"])
    torch.cuda.synchronize()
    for r, st in reqs.items():
        L = prompts[r] + n_dec[r]
        assert st["pos"] == L, (r, st["pos"])
        x = st["x"]
        g_ref = oracle.gate(x["z"], A_gate)
        o_ref, _ = oracle.forward(x["q"], x["k"], x["v"], g_ref, x["beta"], None)
        ro = rho(st["out"], o_ref)
        print(f"    {r}: rho(o)={ro:.3e}", flush=True)
        assert np.isfinite(st["out"].float().cpu().numpy()).all()
        assert ro <= TOL[dtype], (r, ro)


@pytest.mark.parametrize("dv,flags", [(128, 0), (64, 0), (128, _lib.KDA_FLAG_PAIRWISE_DIAGONAL)])
def test_varlen_pooled_prefill_equals_per_sequence_calls(dv, flags):
    """Five prompts of 37, 0, 300, 64 and 1 tokens packed in one call equal
    five separate pooled calls bit for bit (the empty one leaves its slot as
    it was); one sequence is also checked against the oracle."""
    say("varlen pooled prefill", dv, flags)
    lens = [37, 0, 300, 64, 1]
    H, total = 2, sum(lens)
    x = inputs.make_prefill_inputs(1, total, H, 128, dv, torch.bfloat16, 530, device="cuda")
    g = kda_gate(x["z"], x["A"])
    q, k, v = x["q"][0], x["k"][0], x["v"][0]
    gg, beta = g[0], x["beta"][0]
    cu_list = [0]
    for L in lens:
        cu_list.append(cu_list[-1] + L)
    cu = torch.tensor(cu_list, dtype=torch.int64, device="cuda")
    slots = [3, 6, 0, 7, 5]
    pool = _pool(8, H, 128, dv, 531)
    before = pool.clone()
    o = kda_chunk_fwd_varlen_pooled(q, k, v, gg, beta, pool, _slots(slots), cu, flags=flags)
    ref_pool = before.clone()
    for b, L in enumerate(lens):
        if L == 0:
            continue
        a_, e_ = cu_list[b], cu_list[b + 1]
        sl = lambda t: t[a_:e_].unsqueeze(0).clone()      # own, aligned allocation
        ob = kda_chunk_fwd_pooled(sl(q), sl(k), sl(v), sl(gg), sl(beta), ref_pool, _slots([slots[b]]),
                                  flags=flags)
        torch.cuda.synchronize()
        assert torch.equal(o[a_:e_], ob[0]), b
    torch.cuda.synchronize()
    assert torch.equal(pool, ref_pool)
    assert torch.equal(pool[6], before[6])               # the empty sequence's slot
    a_, e_ = cu_list[2], cu_list[3]
    S0 = before[0].unsqueeze(0)
    o_ref, S_ref = oracle.forward(q[a_:e_].unsqueeze(0).clone(), k[a_:e_].unsqueeze(0).clone(),
                                  v[a_:e_].unsqueeze(0).clone(), gg[a_:e_].unsqueeze(0).float().cpu(),
                                  beta[a_:e_].unsqueeze(0).clone(), S0)
    assert rho(o[a_:e_].unsqueeze(0), o_ref) <= TOL[torch.bfloat16]
    assert rho(pool[0].unsqueeze(0), S_ref) <= TOL[torch.bfloat16]


def test_varlen_pooled_gated_equals_per_sequence_gated_calls():
    """The fused-gate serving prefill: prompts of 37, 0, 300, 64 and 1 tokens
    packed in one kda_chunk_fwd_varlen_pooled_gated call equal separate
    kda_chunk_fwd_gated calls from the slots' states bit for bit (the same
    kernel instance); one sequence is also checked against the oracle's fp64
    gate and recurrence."""
    from linear_attention_sequence_gate_amd import kda_chunk_fwd_gated, kda_chunk_fwd_varlen_pooled_gated
    say("varlen pooled prefill, gate fused")
    lens = [37, 0, 300, 64, 1]
    H, total, dv = 2, sum(lens), 128
    x = inputs.make_prefill_inputs(1, total, H, 128, dv, torch.bfloat16, 540, device="cuda",
                                   stress_heads_mean=3.0)
    q, k, v, z, beta = x["q"][0], x["k"][0], x["v"][0], x["z"][0], x["beta"][0]
    cu_list = [0]
    for L in lens:
        cu_list.append(cu_list[-1] + L)
    cu = torch.tensor(cu_list, dtype=torch.int64, device="cuda")
    slots = [3, 6, 0, 7, 5]
    pool = _pool(8, H, 128, dv, 541)
    before = pool.clone()
    o = kda_chunk_fwd_varlen_pooled_gated(q, k, v, z, x["A"], beta, pool, _slots(slots), cu)
    torch.cuda.synchronize()
    for b, L in enumerate(lens):
        if L == 0:
            continue
        a_, e_ = cu_list[b], cu_list[b + 1]
        sl = lambda t: t[a_:e_].unsqueeze(0).clone()      # own, aligned allocation
        S = before[slots[b]].unsqueeze(0).clone()
        ob, _ = kda_chunk_fwd_gated(sl(q), sl(k), sl(v), sl(z), x["A"], sl(beta), S, final_state=S)
        torch.cuda.synchronize()
        assert torch.equal(o[a_:e_], ob[0]), b
        assert torch.equal(pool[slots[b]], S[0]), b
    assert torch.equal(pool[6], before[6])               # the empty sequence's slot
    a_, e_ = cu_list[2], cu_list[3]
    g64 = oracle.gate(z[a_:e_].unsqueeze(0), x["A"])
    o_ref, S_ref = oracle.forward(q[a_:e_].unsqueeze(0), k[a_:e_].unsqueeze(0), v[a_:e_].unsqueeze(0),
                                  g64, beta[a_:e_].unsqueeze(0), before[0].unsqueeze(0))
    assert rho(o[a_:e_].unsqueeze(0), o_ref) <= TOL[torch.bfloat16]
    assert rho(pool[0].unsqueeze(0), S_ref) <= TOL[torch.bfloat16]
