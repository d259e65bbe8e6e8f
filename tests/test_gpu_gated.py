"""GPU parity of kda_chunk_fwd_gated (the gate evaluated inside the chunk
call) against the oracle's fp64 gate and recurrence, at sizes the oracle runs
in seconds: ragged tails, initial states, decay-stress heads, the sequence
split, the position-pair diagonal path, and the shapes that stage g through
the workspace.  Also: agreement with kda_gate + kda_chunk_fwd on the same
inputs, and the host-side rejections."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_gate_amd import _lib, kda_chunk_fwd, kda_gate
from linear_attention_sequence_gate_amd._lib import KDA_FLAG_PAIRWISE_DIAGONAL, kda_flag_segments
from kda_testutil import TOL, prefill_device, rho, say

pytestmark = pytest.mark.gpu


def _gated_vs_oracle(x, dtype, label, flags=0):
    """Both sides start from z and A: the oracle's gate is fp64 (never rounded
    to fp32), the library's is evaluated inside the call."""
    say("gated", label)
    o, ST = _lib.kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"], x["S0"],
                                     flags=flags)
    torch.cuda.synchronize()
    g64 = oracle.gate(x["z"], x["A"])
    o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], g64, x["beta"], x["S0"])
    ro, rs = rho(o, o_ref), rho(ST, S_ref)
    print(f"    rho(o)={ro:.3e} rho(S)={rs:.3e}", flush=True)
    assert np.isfinite(o.float().cpu().numpy()).all()
    assert ro <= TOL[dtype] and rs <= TOL[dtype], (ro, rs)
    return o, ST


@pytest.mark.parametrize("T", [1, 31, 32, 33, 200, 333])
@pytest.mark.parametrize("dv", [128, 64])
def test_fused_tails_and_state(T, dv):
    """The fused shapes (bf16, dk = 128), decay-stress heads near the floor."""
    x = prefill_device(2, T, 4, 128, dv, torch.bfloat16, 900 + T, s0_std=0.02, stress=3.0)
    _gated_vs_oracle(x, torch.bfloat16, f"fused T={T} dv={dv}")


@pytest.mark.parametrize("dtype,dk,dv", [(torch.float32, 32, 32), (torch.float32, 64, 128),
                                         (torch.bfloat16, 64, 64), (torch.bfloat16, 32, 128)])
def test_staged_shapes(dtype, dk, dv):
    """Shapes without the fused kernel: the gate kernel fills the workspace first."""
    x = prefill_device(2, 150, 3, dk, dv, dtype, 950 + dk + dv, s0_std=0.1, stress=3.0)
    _gated_vs_oracle(x, dtype, f"staged {dtype} dk={dk} dv={dv}")


def test_gate_extremes():
    """z far out on both sides: g = 0 (no decay) and g = -5 (every 16-token
    tile sums to the -80 bound) where the in-kernel exponential overflows to
    +inf and underflows to 0."""
    x = prefill_device(1, 96, 3, 128, 128, torch.bfloat16, 960, s0_std=0.1)
    z = x["z"].clone()
    z[:, :, 0] = -200.0          # exp(A) z very negative: sigmoid -> 0, g -> 0
    z[:, :, 1] = 200.0           # very positive: g -> -5
    x["z"] = z
    _gated_vs_oracle(x, torch.bfloat16, "gate extremes")


def test_matches_separate_gate_and_chunk():
    """kda_chunk_fwd_gated == kda_gate + kda_chunk_fwd up to fp32 rounding of
    the gate (a few ulp in alpha)."""
    x = prefill_device(2, 500, 4, 128, 128, torch.bfloat16, 970, s0_std=0.02, stress=3.0)
    say("gated vs separate")
    o1, S1 = _lib.kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"], x["S0"])
    g = kda_gate(x["z"], x["A"])
    o2, S2 = kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], x["S0"])
    torch.cuda.synchronize()
    do = (o1.float() - o2.float()).abs().max().item() / o2.float().abs().max().item()
    ds = (S1 - S2).abs().max().item() / S2.abs().max().item()
    print(f"    gated vs separate: o {do:.2e}  S {ds:.2e}", flush=True)
    # o is bf16: a one-ulp flip of a rounded output is 2^-8 of its magnitude
    assert do <= 8e-3 and ds <= 1e-4, (do, ds)


@pytest.mark.parametrize("nseg", [2, 3, 5])
def test_sequence_split(nseg):
    """The fused gate in every phase of the sequence split."""
    x = prefill_device(1, 700, 2, 128, 128, torch.bfloat16, 980 + nseg, s0_std=0.02, stress=3.0)
    _gated_vs_oracle(x, torch.bfloat16, f"split nseg={nseg}", flags=kda_flag_segments(nseg))


def test_pairwise_diagonal():
    x = prefill_device(1, 130, 2, 128, 128, torch.bfloat16, 990, s0_std=0.02, stress=3.0)
    _gated_vs_oracle(x, torch.bfloat16, "pairwise", flags=KDA_FLAG_PAIRWISE_DIAGONAL)


def test_in_place_continuation():
    """initial_state == final_state, cut into two calls."""
    x = prefill_device(1, 300, 2, 128, 128, torch.bfloat16, 995, s0_std=0.02)
    say("gated in place")
    S = x["S0"].clone()
    parts = []
    for t0, t1 in ((0, 110), (110, 300)):
        sl = {n: x[n][:, t0:t1].clone() for n in ("q", "k", "v", "z", "beta")}   # fresh, aligned
        o, _ = _lib.kda_chunk_fwd_gated(sl["q"], sl["k"], sl["v"], sl["z"], x["A"], sl["beta"], S,
                                        final_state=S)
        parts.append(o)
    torch.cuda.synchronize()
    o = torch.cat(parts, dim=1)
    g64 = oracle.gate(x["z"], x["A"])
    o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], g64, x["beta"], x["S0"])
    assert rho(o, o_ref) <= TOL[torch.bfloat16] and rho(S, S_ref) <= TOL[torch.bfloat16]


def test_rejections():
    """Host-side validation: the range check flag and a missing z or A."""
    x = prefill_device(1, 64, 2, 128, 128, torch.bfloat16, 999)
    with pytest.raises(_lib.KdaError) as e:
        _lib.kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"],
                                 flags=_lib.KDA_FLAG_CHECK_RANGE)
    assert e.value.code == -1
    L = _lib.load_library()
    o = torch.empty_like(x["v"])
    P = ctypes.c_void_p
    r = L.kda_chunk_fwd_gated(P(x["q"].data_ptr()), P(x["k"].data_ptr()), P(x["v"].data_ptr()),
                              None, P(x["A"].data_ptr()), P(x["beta"].data_ptr()), None, None,
                              P(o.data_ptr()), None, 0, 1, 64, 2, 128, 128, 1, 0, None)
    assert r == -1
    # staged shapes need the workspace for g
    y = prefill_device(1, 64, 2, 64, 64, torch.bfloat16, 998)
    r = L.kda_chunk_fwd_gated(P(y["q"].data_ptr()), P(y["k"].data_ptr()), P(y["v"].data_ptr()),
                              P(y["z"].data_ptr()), P(y["A"].data_ptr()), P(y["beta"].data_ptr()),
                              None, None, P(torch.empty_like(y["v"]).data_ptr()), None, 0,
                              1, 64, 2, 64, 64, 1, 0, None)
    assert r == -1
    torch.cuda.synchronize()
