"""GPU parity of the position-pair diagonal path (KDA_FLAG_PAIRWISE_DIAGONAL,
the path the gate floor made unnecessary) against the oracle: with the floor
(also against the dense path), and with the floor removed (g uniform in
[-20, 0], 16-token decay sums down to -320, where the dense diagonal tiles'
reciprocal decay factor would overflow), with ragged tails, initial states
and the sequence split."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_gate_amd import _lib, kda_chunk_fwd, kda_gate
from kda_testutil import TOL, oracle_gate_f32, prefill_device, rho, say

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16
PW = _lib.KDA_FLAG_PAIRWISE_DIAGONAL


def _no_floor_g(B, T, H, dk, seed):
    gen = torch.Generator().manual_seed(seed)
    return -20.0 * torch.rand(B, T, H, dk, generator=gen, dtype=torch.float32)


def _check(x, g_f32, flags, label, dense_too=False):
    say("pairwise", label)
    g = g_f32.cuda()
    o, S = kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], x["S0"], flags=flags)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], g_f32, x["beta"], x["S0"])
    ro, rs = rho(o, o_ref), rho(S, S_ref)
    print(f"    rho(o)={ro:.3e} rho(S)={rs:.3e}", flush=True)
    assert np.isfinite(o.float().cpu().numpy()).all() and torch.isfinite(S).all()
    assert ro <= TOL[BF16] and rs <= TOL[BF16], (ro, rs)
    if dense_too:
        o_d, S_d = kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], x["S0"])
        torch.cuda.synchronize()
        assert rho(o, o_d) <= TOL[BF16] and rho(S, S_d) <= TOL[BF16]


@pytest.mark.parametrize("T", [1, 17, 64, 333])
@pytest.mark.parametrize("dv", [64, 128])
def test_pairwise_with_the_floor(T, dv):
    x = prefill_device(2, T, 3, 128, dv, BF16, 600 + T, s0_std=0.02, stress=3.0)
    _check(x, oracle_gate_f32(x["z"], x["A"]), PW, f"floor T={T} dv={dv}", dense_too=True)


@pytest.mark.parametrize("T", [16, 100, 517])
def test_pairwise_without_the_floor(T):
    x = prefill_device(1, T, 4, 128, 128, BF16, 610 + T, s0_std=0.02)
    g = _no_floor_g(1, T, 4, 128, 611 + T)
    sums = g.reshape(1, -1, 4, 128)[:, : (T // 16) * 16].reshape(1, -1, 16, 4, 128).sum(2)
    if T >= 16:
        assert sums.min() < -200           # far outside the floor's (-80, 0]
    _check(x, g, PW, f"no floor T={T}")


def test_pairwise_without_the_floor_split_and_range_flag():
    """The split path with position pairs; and the dense path's range check
    rejects the same input (it relies on the floor)."""
    T = 2000
    x = prefill_device(1, T, 2, 128, 128, BF16, 620, s0_std=0.02)
    g = _no_floor_g(1, T, 2, 128, 621)
    _check(x, g, PW | _lib.kda_flag_segments(3), "no floor, 3 segments")
    with pytest.raises(_lib.KdaError) as ei:
        kda_chunk_fwd(x["q"], x["k"], x["v"], g.cuda(), x["beta"], x["S0"],
                      flags=_lib.KDA_FLAG_CHECK_RANGE)
    assert ei.value.code == _lib.KDA_ERR_RANGE
