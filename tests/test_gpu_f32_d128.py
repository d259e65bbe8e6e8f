"""GPU parity of the fp32 prefill at dk = 128 against the oracle.  Those
shapes run 16-token chunks through device buffers (X, P, At and the decayed
operands of every chunk), then a forward state pass that writes o, all in fp32
arithmetic, so the bar is the fp32 one: ragged tails, every dv, initial state
or none, in-place continuation, the decay-stress gate, a long sequence, the
gated entry point (g staged in the workspace first), and the pooled call
(states in a slot-indexed pool)."""
import pytest
import torch

import oracle
from linear_attention_sequence_gate_amd import kda_chunk_fwd, kda_chunk_fwd_gated, kda_chunk_fwd_pooled
from kda_testutil import TOL, oracle_gate_f32, prefill_device, rho, say

pytestmark = pytest.mark.gpu

F32 = torch.float32


def _check(o, S, o_ref, S_ref, label):
    ro, rs = rho(o, o_ref), rho(S, S_ref)
    print(f"    {label}: rho(o)={ro:.3e} rho(S)={rs:.3e}", flush=True)
    assert torch.isfinite(o).all() and torch.isfinite(S).all(), label
    assert ro <= TOL[F32] and rs <= TOL[F32], (label, ro, rs)


@pytest.mark.parametrize("T", [1, 15, 16, 17, 48, 100, 333])
@pytest.mark.parametrize("dv", [32, 64, 128])
def test_f32_d128_tails_and_state(T, dv):
    say("fp32 dk=128", f"T={T} dv={dv}")
    x = prefill_device(2, T, 3, 128, dv, F32, 800 + T + dv, s0_std=0.3, stress=3.0)
    g = oracle_gate_f32(x["z"], x["A"])
    o, S = kda_chunk_fwd(x["q"], x["k"], x["v"], g.cuda(), x["beta"], x["S0"])
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], g, x["beta"], x["S0"])
    _check(o, S, o_ref, S_ref, f"T={T} dv={dv}")


def test_f32_d128_zero_start_in_place_and_long():
    """No initial state; the same call continued in place over a second
    half; and 4096 tokens (256 chunks) in one call."""
    say("fp32 dk=128 zero start / in place / long")
    x = prefill_device(1, 4096, 2, 128, 128, F32, 880, s0_std=0.0)
    g = oracle_gate_f32(x["z"], x["A"])
    gd = g.cuda()
    o, S = kda_chunk_fwd(x["q"], x["k"], x["v"], gd, x["beta"], None)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], g, x["beta"], None)
    _check(o, S, o_ref, S_ref, "T=4096 from zero")
    # the first 1000 tokens, then the rest continued from the state in place
    h = 1000
    part = {n: x[n][:, :h].contiguous() for n in ("q", "k", "v", "beta")}
    rest = {n: x[n][:, h:].contiguous() for n in ("q", "k", "v", "beta")}
    o1, S1 = kda_chunk_fwd(part["q"], part["k"], part["v"], gd[:, :h].contiguous(), part["beta"], None)
    o2, _ = kda_chunk_fwd(rest["q"], rest["k"], rest["v"], gd[:, h:].contiguous(), rest["beta"], S1,
                          final_state=S1)
    torch.cuda.synchronize()
    _check(torch.cat([o1, o2], 1), S1, o_ref, S_ref, "1000 + 3096 in place")


def test_f32_d128_gated():
    say("fp32 dk=128 gated")
    x = prefill_device(1, 300, 4, 128, 64, F32, 890, s0_std=0.3, stress=3.0)
    o, S = kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"], x["S0"])
    torch.cuda.synchronize()
    g_ref = oracle.gate(x["z"], x["A"])
    o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], g_ref, x["beta"], x["S0"])
    _check(o, S, o_ref, S_ref, "gated")


def test_f32_d128_pooled_equals_plain_on_gathered_states():
    """Sequences 0..2 use pool slots 4, 1, 6; sequence 3's slot is outside the
    pool, so its output and every other slot stay untouched.  Bit-equal to the
    plain call on the gathered states, and within the bar of the oracle."""
    say("fp32 dk=128 pooled")
    n_slots, H, T, dv = 8, 2, 150, 64
    x = prefill_device(4, T, H, 128, dv, F32, 895)
    g = oracle_gate_f32(x["z"], x["A"])
    gd = g.cuda()
    gen = torch.Generator(device="cuda").manual_seed(896)
    pool = torch.randn(n_slots, H, 128, dv, device="cuda", generator=gen) * 0.3
    before = pool.clone()
    slots = [4, 1, 6, -3]
    S0 = pool[slots[:3]].clone()
    o_ref, S_ref = kda_chunk_fwd(x["q"][:3].contiguous(), x["k"][:3].contiguous(),
                                 x["v"][:3].contiguous(), gd[:3].contiguous(),
                                 x["beta"][:3].contiguous(), S0)
    o = torch.full((4, T, H, dv), 7.0, device="cuda", dtype=F32)
    kda_chunk_fwd_pooled(x["q"], x["k"], x["v"], gd, x["beta"], pool,
                         torch.tensor(slots, dtype=torch.int32, device="cuda"), o=o)
    torch.cuda.synchronize()
    assert torch.equal(o[:3], o_ref) and torch.equal(pool[slots[:3]], S_ref)
    assert (o[3] == 7.0).all()
    assert torch.equal(pool[[0, 2, 3, 5, 7]], before[[0, 2, 3, 5, 7]])
    oo, So = oracle.forward(x["q"][:3], x["k"][:3], x["v"][:3], g[:3], x["beta"][:3],
                            before[slots[:3]].cpu())
    _check(o[:3], pool[slots[:3]], oo, So, "pooled vs oracle")
