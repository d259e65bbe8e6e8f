"""GPU parity of kda_chunk_fwd against the oracle at sizes the oracle runs in
seconds: several 64-token chunks, ragged tails, initial states, decay-stress
heads, the degenerate gates (g = 0 and g at the floor), plus GPU-side
properties (split invariance, determinism, in-place state, range check)."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_gate_amd import _lib, inputs, kda_chunk_fwd, kda_gate
from kda_testutil import TOL, oracle_gate_f32, prefill_device, rho, say

pytestmark = pytest.mark.gpu


def _run_and_compare(x, g_f32, dtype, label):
    """GPU chunk_fwd on (x, g) vs the oracle on the same values."""
    say("chunk", label)
    g_dev = g_f32.cuda()
    o, ST = kda_chunk_fwd(x["q"], x["k"], x["v"], g_dev, x["beta"], x["S0"])
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], g_f32, x["beta"], x["S0"])
    ro, rs = rho(o, o_ref), rho(ST, S_ref)
    print(f"    rho(o)={ro:.3e} rho(S)={rs:.3e}", flush=True)
    assert np.isfinite(o.float().cpu().numpy()).all()
    assert ro <= TOL[dtype] and rs <= TOL[dtype], (ro, rs)
    return ro, rs


def test_small_f32_workload():
    """B1 H1 T128 d32 fp32, zero initial state."""
    w = inputs.WORKLOADS["small_f32"]
    x = inputs.workload_prefill_inputs(w, device="cuda")
    _run_and_compare(x, oracle_gate_f32(x["z"], x["A"]), w.dtype, w.name)


@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 65, 130, 200])
@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 128), (32, 64)])
def test_f32_tails_and_state(T, dk, dv):
    x = prefill_device(2, T, 3, dk, dv, torch.float32, 100 + T, s0_std=0.3, stress=3.0)
    _run_and_compare(x, oracle_gate_f32(x["z"], x["A"]), torch.float32, f"f32 T={T} dk={dk} dv={dv}")


@pytest.mark.parametrize("T", [1, 17, 64, 200, 333])
@pytest.mark.parametrize("dk,dv", [(128, 128), (128, 64), (64, 64), (32, 128)])
def test_bf16_tails_and_state(T, dk, dv):
    x = prefill_device(2, T, 4, dk, dv, torch.bfloat16, 200 + T, s0_std=0.02, stress=3.0)
    _run_and_compare(x, oracle_gate_f32(x["z"], x["A"]), torch.bfloat16,
                     f"bf16 T={T} dk={dk} dv={dv}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("gval", [0.0, -5.0, -2.5])
def test_constant_gate_edges(dtype, gval):
    """g = 0 (no decay), g = -5 everywhere (every 16-token tile sums to exactly
    -80, the bound) and a mid value."""
    dk = 64
    x = prefill_device(1, 150, 2, dk, dk, dtype, 300, s0_std=0.1)
    g = torch.full((1, 150, 2, dk), gval, dtype=torch.float32)
    _run_and_compare(x, g, dtype, f"constant g={gval} {dtype}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_beta_zero_pure_decay(dtype):
    """beta = 0: nothing is written, the state only decays.  The gate is slowed
    (z - 6 gives g ~ -0.01) so the initial state survives 100 tokens instead of
    underflowing, which would leave nothing to compare."""
    x = prefill_device(1, 100, 2, 64, 64, dtype, 301, s0_std=0.5)
    x["beta"] = torch.zeros_like(x["beta"])
    g = oracle_gate_f32(x["z"].float() - 6.0, x["A"])
    _run_and_compare(x, g, dtype, f"beta=0 {dtype}")


def test_split_invariance_on_gpu():
    """prefill(T) == prefill(T1) -> state -> prefill(T - T1), for cuts inside and
    at chunk boundaries (chunks realign at each call)."""
    say("split invariance")
    T = 300
    x = prefill_device(2, T, 2, 64, 64, torch.float32, 302, s0_std=0.05)
    g = kda_gate(x["z"], x["A"])
    o, S = kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], x["S0"])
    for T1 in (1, 64, 100, 299):
        sl = lambda a, s: a[:, s].contiguous()
        a_, b_ = slice(0, T1), slice(T1, T)
        o1, S1 = kda_chunk_fwd(sl(x["q"], a_), sl(x["k"], a_), sl(x["v"], a_), sl(g, a_),
                               sl(x["beta"], a_), x["S0"])
        o2, S2 = kda_chunk_fwd(sl(x["q"], b_), sl(x["k"], b_), sl(x["v"], b_), sl(g, b_),
                               sl(x["beta"], b_), S1)
        torch.cuda.synchronize()
        assert rho(torch.cat([o1, o2], dim=1), o) <= 1e-5
        assert rho(S2, S) <= 1e-5


def test_deterministic_and_in_place_state():
    say("determinism + in-place state")
    x = prefill_device(2, 257, 4, 128, 128, torch.bfloat16, 303, s0_std=0.02, stress=3.0)
    g = kda_gate(x["z"], x["A"])
    o1, S1 = kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], x["S0"])
    o2, S2 = kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], x["S0"])
    S_inplace = x["S0"].clone()
    o3, _ = kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], S_inplace, final_state=S_inplace)
    o4, none = kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], x["S0"], want_final_state=False)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    assert torch.equal(o1, o3) and torch.equal(S1, S_inplace)
    assert torch.equal(o1, o4)


def test_range_check_flag():
    say("range check")
    x = prefill_device(1, 40, 1, 32, 32, torch.float32, 304)
    g = oracle_gate_f32(x["z"], x["A"]).cuda()
    o, S = kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], flags=_lib.KDA_FLAG_CHECK_RANGE)
    torch.cuda.synchronize()
    bad = g.clone()
    bad[0, 3, 0, 5] = -5.5
    with pytest.raises(_lib.KdaError) as ei:
        kda_chunk_fwd(x["q"], x["k"], x["v"], bad, x["beta"], flags=_lib.KDA_FLAG_CHECK_RANGE)
    assert ei.value.code == _lib.KDA_ERR_RANGE
    bad = g.clone()
    bad[0, 0, 0, 0] = 0.5
    with pytest.raises(_lib.KdaError):
        kda_chunk_fwd(x["q"], x["k"], x["v"], bad, x["beta"], flags=_lib.KDA_FLAG_CHECK_RANGE)


def test_end_to_end_gate_then_chunk():
    """The whole hot path on the GPU (kda_gate -> kda_chunk_fwd) against the
    oracle's gate and recurrence from the same z, A."""
    say("end to end gate + chunk")
    x = prefill_device(1, 256, 4, 128, 128, torch.bfloat16, 305, stress=3.0)
    g = kda_gate(x["z"], x["A"])
    o, S = kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"])
    torch.cuda.synchronize()
    g_ref = oracle.gate(x["z"], x["A"])
    o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], g_ref, x["beta"])
    assert rho(o, o_ref) <= TOL[torch.bfloat16] and rho(S, S_ref) <= TOL[torch.bfloat16]
