"""GPU parity of kda_decode_step against the oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_gate_amd import inputs, kda_chunk_fwd, kda_decode_step, kda_gate
from kda_testutil import TOL, rho, say

pytestmark = pytest.mark.gpu


def _step_inputs(N, H, dk, dv, dtype, seed, step):
    return inputs.make_decode_step_inputs(N, H, dk, dv, dtype, seed, step, device="cuda")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 128), (128, 32), (128, 128)])
def test_decode_steps_match_oracle(dtype, dk, dv):
    N, H, steps = 3, 2, 5
    say("decode", dtype, dk, dv)
    st = inputs.make_decode_state(N, H, dk, dv, 77, device="cuda")
    S = st["S"].clone()
    S_ref = st["S"].double().cpu().numpy()
    for t in range(steps):
        x = _step_inputs(N, H, dk, dv, dtype, 77, t)
        o = kda_decode_step(x["q"], x["k"], x["v"], x["z"], st["A"], x["beta"], S)
        torch.cuda.synchronize()
        o_ref, S_ref = oracle.decode_step(x["q"], x["k"], x["v"], x["z"], st["A"], x["beta"], S_ref)
        assert rho(o, o_ref) <= TOL[dtype], (t, rho(o, o_ref))
        assert rho(S, S_ref) <= TOL[dtype], (t, rho(S, S_ref))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 32), (128, 64)])
def test_decode_persistent_grid_heads(dtype, dk, dv):
    """More heads than the persistent grid's 1024 workgroups, not a multiple of
    it (37 x 40 = 1480): workgroups walk several heads and prefetch the next
    head's state while writing the current one.  Two steps, every head."""
    N, H = 37, 40
    say("decode persistent grid", dtype, dk, dv)
    st = inputs.make_decode_state(N, H, dk, dv, 79, device="cuda")
    S = st["S"].clone()
    S_ref = st["S"].double().cpu().numpy()
    for t in range(2):
        x = _step_inputs(N, H, dk, dv, dtype, 79, t)
        o = kda_decode_step(x["q"], x["k"], x["v"], x["z"], st["A"], x["beta"], S)
        torch.cuda.synchronize()
        o_ref, S_ref = oracle.decode_step(x["q"], x["k"], x["v"], x["z"], st["A"], x["beta"], S_ref)
        assert rho(o, o_ref) <= TOL[dtype], (t, rho(o, o_ref))
        assert rho(S, S_ref) <= TOL[dtype], (t, rho(S, S_ref))


def test_decode_matches_prefill_on_gpu():
    """T decode steps equal one chunked prefill of the same T tokens (gate fused
    in decode, separate in prefill): the state is the whole carry."""
    N, H, dk, dv, T = 2, 3, 64, 64, 37
    say("decode vs prefill")
    x = inputs.make_prefill_inputs(N, T, H, dk, dv, torch.float32, 78, device="cuda", s0_std=0.02)
    g = kda_gate(x["z"], x["A"])
    o_pre, S_pre = kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], x["S0"])
    S = x["S0"].clone()
    outs = []
    for t in range(T):
        sl = lambda a: a[:, t].contiguous()
        outs.append(kda_decode_step(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["z"]), x["A"],
                                    sl(x["beta"]), S))
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, dim=1)
    assert rho(o_dec, o_pre) <= 1e-4
    assert rho(S, S_pre) <= 1e-4


def test_decode_full_size_one_step_all_heads():
    """256 sequences x H32 x d128 bf16, fp32 state (512 MiB) updated in place:
    one step checked on every head."""
    w = inputs.WORKLOADS["decode_256x32"]
    say("decode full size, 1 step, all heads")
    st = inputs.make_decode_state(w.B, w.H, w.dk, w.dv, w.seed, device="cuda", s0_std=w.s0_std)
    S = st["S"].clone()
    x = _step_inputs(w.B, w.H, w.dk, w.dv, w.dtype, w.seed, 0)
    o = kda_decode_step(x["q"], x["k"], x["v"], x["z"], st["A"], x["beta"], S)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.decode_step(x["q"], x["k"], x["v"], x["z"], st["A"], x["beta"], st["S"])
    assert rho(o, o_ref) <= TOL[w.dtype]
    assert rho(S, S_ref) <= TOL[w.dtype]
    del st, S, x
    torch.cuda.empty_cache()


def test_decode_full_size_1000_steps_sampled():
    """1000 consecutive in-place steps with fresh seeded inputs; a seeded subset
    of 32 (sequence, head) pairs followed by the oracle through all 1000 steps
    (pairs are independent, so the subset is exact)."""
    w = inputs.WORKLOADS["decode_256x32"]
    say("decode full size, 1000 steps, sampled pairs")
    st = inputs.make_decode_state(w.B, w.H, w.dk, w.dv, w.seed, device="cuda", s0_std=w.s0_std)
    S = st["S"].clone()
    pick = torch.randperm(w.B * w.H, generator=torch.Generator().manual_seed(3))[:32]
    n_idx, h_idx = (pick // w.H).cuda(), (pick % w.H).cuda()
    # the sampled pairs become the 32 "heads" of one oracle problem, each with its own A row
    S_ref = st["S"][n_idx, h_idx].double().cpu().numpy()[None]        # [1,32,dk,dv]
    A_sub = st["A"][h_idx].contiguous()
    worst_o = 0.0
    for t in range(w.decode_steps):
        x = _step_inputs(w.B, w.H, w.dk, w.dv, w.dtype, w.seed, t)
        o = kda_decode_step(x["q"], x["k"], x["v"], x["z"], st["A"], x["beta"], S)
        sub = {n: x[n][n_idx, h_idx].unsqueeze(0) for n in ("q", "k", "v", "z", "beta")}
        o_ref, S_ref = oracle.decode_step(sub["q"], sub["k"], sub["v"], sub["z"], A_sub,
                                          sub["beta"], S_ref)
        worst_o = max(worst_o, rho(o[n_idx, h_idx].unsqueeze(0), o_ref))
        if t % 250 == 0:
            say("decode step", t, "worst rho(o) so far", worst_o)
    torch.cuda.synchronize()
    assert worst_o <= TOL[w.dtype]
    assert rho(S[n_idx, h_idx].unsqueeze(0), S_ref) <= TOL[w.dtype]
    del st, S
    torch.cuda.empty_cache()


def test_decode_continues_a_fused_gate_prefill():
    """bf16, dk = dv = 128: kda_chunk_fwd_gated over T0 tokens, then T1 decode
    steps, equal one kda_chunk_fwd_gated over all of them (the state is the
    whole carry; the two paths evaluate the gate by different formulas of the
    same function)."""
    from linear_attention_sequence_gate_amd import kda_chunk_fwd_gated
    N, H, d, T0, T1 = 2, 4, 128, 200, 12
    say("fused prefill then decode vs one fused prefill")
    x = inputs.make_prefill_inputs(N, T0 + T1, H, d, d, torch.bfloat16, 79, device="cuda",
                                   s0_std=0.02, stress_heads_mean=3.0)
    o_all, S_all = kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"], x["S0"])
    head = {n: x[n][:, :T0].clone() for n in ("q", "k", "v", "z", "beta")}
    o_head, S = kda_chunk_fwd_gated(head["q"], head["k"], head["v"], head["z"], x["A"],
                                    head["beta"], x["S0"])
    outs = []
    for t in range(T0, T0 + T1):
        sl = lambda a: a[:, t].contiguous()
        outs.append(kda_decode_step(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["z"]), x["A"],
                                    sl(x["beta"]), S))
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, dim=1)
    # the head's last chunk is partial: its decay factors are formed over the
    # padded subtile, so equal up to rounding (bf16 outputs: a flipped ulp)
    assert rho(o_head, o_all[:, :T0]) <= TOL[torch.bfloat16]
    assert rho(o_dec, o_all[:, T0:]) <= TOL[torch.bfloat16]
    # the chunked path's products take bf16 operands (about 3e-3 from the
    # oracle on either side), so the two states meet at the bf16 bar
    assert rho(S, S_all) <= TOL[torch.bfloat16]
