"""GPU parity of kda_chunk_bwd (reverse mode of the recurrence) against the
oracle's reverse mode on the same inputs: fp32 and bf16, every (dk, dv) family,
T around the 8-token checkpoint spacing, with and without the initial state
and the final-state gradient, and with the gate floor removed."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_gate_amd import kda_chunk_bwd
from kda_testutil import TOL, oracle_gate_f32, prefill_device, rho, say

pytestmark = pytest.mark.gpu


def _run(dtype, B, T, H, dk, dv, seed, s0=True, dst=True, g=None):
    x = prefill_device(B, T, H, dk, dv, dtype, seed, s0_std=0.3 if s0 else 0.0)
    g_f32 = oracle_gate_f32(x["z"], x["A"]) if g is None else g
    gen = torch.Generator(device="cuda").manual_seed(seed + 1)
    d_o = torch.randn(B, T, H, dv, device="cuda", generator=gen).to(dtype)
    dST = torch.randn(B, H, dk, dv, device="cuda", generator=gen) if dst else None
    out = kda_chunk_bwd(x["q"], x["k"], x["v"], g_f32.cuda(), x["beta"], x["S0"], d_o, dST)
    torch.cuda.synchronize()
    ref = oracle.backward_np(x["q"], x["k"], x["v"], g_f32, x["beta"], x["S0"], d_o, dST)
    res = {}
    for name, rname in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dg", "dg"), ("dbeta", "dbeta"),
                        ("d_initial_state", "dS0")):
        r = rho(out[name], ref[rname])
        res[name] = r
        assert np.isfinite(out[name].cpu().numpy()).all(), name
    print("    " + " ".join(f"{k}={v:.1e}" for k, v in res.items()), flush=True)
    for name, r in res.items():
        assert r <= TOL[dtype], (name, r)


@pytest.mark.parametrize("T", [1, 8, 9, 37])
def test_backward_f32_small(T):
    say("backward f32", T)
    _run(torch.float32, 2, T, 2, 32, 32, 700 + T)


@pytest.mark.parametrize("dk,dv,T", [(64, 128, 20), (128, 64, 17), (32, 64, 24)])
def test_backward_f32_shapes(dk, dv, T):
    say("backward f32", dk, dv, T)
    _run(torch.float32, 1, T, 2, dk, dv, 710 + T, s0=False)


@pytest.mark.parametrize("dk,dv,T", [(128, 128, 70), (32, 64, 13), (64, 32, 33)])
def test_backward_bf16(dk, dv, T):
    say("backward bf16", dk, dv, T)
    _run(torch.bfloat16, 1, T, 3, dk, dv, 720 + T, dst=False)


def test_backward_without_the_floor():
    """The token-level reverse mode assumes nothing about the decay range."""
    say("backward without the floor")
    T, H, d = 40, 2, 64
    g = -20.0 * torch.rand(1, T, H, d, generator=torch.Generator().manual_seed(731))
    _run(torch.float32, 1, T, H, d, d, 730, g=g)
