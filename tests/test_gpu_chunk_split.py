"""GPU parity of the sequence-parallel prefill path (each sequence cut into
segments; segment transitions chained as S -> M S + L) against the oracle and
against the one-pass kernel on the same inputs: forced segment counts with
ragged last segments, initial states, in-place continuation, the automatic
choice for a long few-chain input, and determinism.  Every forced split runs
both schemes: the default one, whose last phase stops where a segment's
transition became zero (keeping the first phase's zero-start o after it),
and KDA_FLAG_SPLIT_FULL_RERUN, whose last phase reruns whole segments."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_gate_amd import _lib, kda_chunk_fwd, kda_chunk_fwd_gated, kda_gate
from kda_testutil import TOL, oracle_gate_f32, prefill_device, rho, say

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16


SCHEMES = {"stop": 0, "rerun": _lib.KDA_FLAG_SPLIT_FULL_RERUN}


def _split(x, g, nseg, scheme="stop", **kw):
    return kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], x["S0"],
                         flags=_lib.kda_flag_segments(nseg) | SCHEMES[scheme], **kw)


def _check_schemes(x, g, nseg, o_ref, S_ref, o_1, S_1):
    """Both schemes of an nseg split against the oracle and one pass."""
    for scheme in SCHEMES:
        o_s, S_s = _split(x, g, nseg, scheme)
        torch.cuda.synchronize()
        ro, rs = rho(o_s, o_ref), rho(S_s, S_ref)
        r1o, r1s = rho(o_s, o_1), rho(S_s, S_1)
        print(f"    {scheme}: vs oracle rho(o)={ro:.3e} rho(S)={rs:.3e}; vs one pass {r1o:.3e} {r1s:.3e}",
              flush=True)
        assert torch.isfinite(o_s.float()).all() and torch.isfinite(S_s).all(), scheme
        assert ro <= TOL[BF16] and rs <= TOL[BF16], (scheme, ro, rs)
        assert r1o <= TOL[BF16] and r1s <= TOL[BF16], (scheme, r1o, r1s)


@pytest.mark.parametrize("nseg,B,T,H,dv", [
    (2, 1, 70, 2, 128),       # 64 + 6 tokens
    (3, 2, 1000, 2, 64),      # 352, 352, 296
    (5, 1, 777, 3, 128),      # four of 160, then 137
    (4, 1, 4096, 2, 128),
    (9, 1, 2000, 1, 128),     # seven middle segments chained
])
def test_forced_split_matches_oracle_and_one_pass(nseg, B, T, H, dv):
    say("split", f"nseg={nseg} B={B} T={T} H={H} dv={dv}")
    x = prefill_device(B, T, H, 128, dv, BF16, 400 + nseg, s0_std=0.02, stress=3.0)
    g_f32 = oracle_gate_f32(x["z"], x["A"])
    g = g_f32.cuda()
    o_1, S_1 = _split(x, g, 1)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], g_f32, x["beta"], x["S0"])
    _check_schemes(x, g, nseg, o_ref, S_ref, o_1, S_1)


def test_split_in_place_state_zero_start_and_determinism():
    say("split in-place / zero start / determinism")
    x = prefill_device(1, 900, 2, 128, 128, BF16, 410, s0_std=0.02)
    g_f32 = oracle_gate_f32(x["z"], x["A"])
    g = g_f32.cuda()
    o1, S1 = _split(x, g, 3)
    o2, S2 = _split(x, g, 3)
    S_in = x["S0"].clone()
    o3, _ = kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], S_in, final_state=S_in,
                          flags=_lib.kda_flag_segments(3))
    oz, Sz = kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], None,
                           flags=_lib.kda_flag_segments(3))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    assert torch.equal(o1, o3) and torch.equal(S1, S_in)
    oz_ref, Sz_ref = oracle.forward(x["q"], x["k"], x["v"], g_f32, x["beta"], None)
    assert rho(oz, oz_ref) <= TOL[BF16] and rho(Sz, Sz_ref) <= TOL[BF16]


def test_automatic_split_for_a_long_few_chain_input():
    """B1 H2 T12400: 4 workgroups in one pass, so the library splits on its own
    (23 segments of 544 tokens); the whole path gate -> chunk against the
    oracle."""
    say("automatic split B1 H2 T12400")
    B, T, H = 1, 12400, 2
    assert _lib.kda_chunk_fwd_workspace_size(B, T, H, 128, 128, 1) > 256
    x = prefill_device(B, T, H, 128, 128, BF16, 411, s0_std=0.02, stress=3.0)
    g = kda_gate(x["z"], x["A"])
    o, S = kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], x["S0"])
    o_1, S_1 = kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], x["S0"],
                             flags=_lib.kda_flag_segments(1))
    torch.cuda.synchronize()
    g_ref = oracle.gate(x["z"], x["A"])
    o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], g_ref, x["beta"], x["S0"])
    ro, rs = rho(o, o_ref), rho(S, S_ref)
    print(f"    rho(o)={ro:.3e} rho(S)={rs:.3e}; vs one pass {rho(o, o_1):.3e} {rho(S, S_1):.3e}",
          flush=True)
    assert ro <= TOL[BF16] and rs <= TOL[BF16], (ro, rs)


@pytest.mark.parametrize("nseg,B,T,H", [
    (5, 1, 900, 2),        # 3 chaining steps
    (6, 1, 1100, 2),       # 4
    (12, 2, 2200, 1),      # 10
    (40, 1, 5000, 1),      # 38 chaining steps
    (129, 1, 16512, 1),    # 127 entries of 128-token segments: the log-depth scan, 7 levels
])
def test_split_with_slow_decay_chains_the_transitions(nseg, B, T, H):
    """A slowed gate (z - 6: g near -0.01 a token) keeps the state, and so each
    segment's transition M, far from zero across a whole segment: the chained
    initial states (serial steps for few segments, the log-depth scan of the
    affine maps for more) carry real weight.  Against the oracle and against
    one pass."""
    say("split, slow decay", f"nseg={nseg} B={B} T={T} H={H}")
    x = prefill_device(B, T, H, 128, 128, BF16, 420 + nseg, s0_std=0.3)
    g_f32 = oracle_gate_f32(x["z"].float() - 6.0, x["A"])
    g = g_f32.cuda()
    o_1, S_1 = _split(x, g, 1)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], g_f32, x["beta"], x["S0"])
    _check_schemes(x, g, nseg, o_ref, S_ref, o_1, S_1)


@pytest.mark.parametrize("nseg", [4, 7, 12])
def test_split_transitions_that_end_early_and_that_run_on(nseg):
    """A middle segment's transition columns (v = 0, initial state I) stop as
    soon as their state is exactly zero.  One launch mixes the cases: head 0
    takes the plain gate (its transitions vanish within a few chunks), head 1
    a slowed gate (z - 6) on every token (they never vanish), head 2 the
    slowed gate on the first 1500 tokens only (some stop mid-segment), head 3
    on the tokens from 1500 on (early transitions vanish, later ones do not:
    the chaining copies L for the first and multiplies for the others, from
    the copied state).  v and the initial state are zero over the first 1000
    tokens, so v-column workgroups also carry an all-zero state for a while
    and must not stop.  Both the g-input and the fused-gate kernels, against
    the oracle and against one pass."""
    say("split, transitions ending early", f"nseg={nseg}")
    B, T, H = 1, 3000, 4
    x = prefill_device(B, T, H, 128, 128, BF16, 430 + nseg)
    x["v"][:, :1000] = 0
    z = x["z"].float()
    z[:, :, 1] -= 6.0
    z[:, :1500, 2] -= 6.0
    z[:, 1500:, 3] -= 6.0
    x["z"] = z.to(BF16)
    g_f32 = oracle_gate_f32(x["z"], x["A"])
    g = g_f32.cuda()
    o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], g_f32, x["beta"], None)
    fl = _lib.kda_flag_segments
    runs = {}
    for scheme, sf in SCHEMES.items():
        runs["g input, " + scheme] = (kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], None,
                                                    flags=fl(nseg) | sf),
                                      kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], None,
                                                    flags=fl(1)))
        runs["gate fused, " + scheme] = tuple(
            kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"], None,
                                flags=fl(n) | (sf if n > 1 else 0)) for n in (nseg, 1))
    torch.cuda.synchronize()
    for name, ((o_s, S_s), (o_1, S_1)) in runs.items():
        ro, rs = rho(o_s, o_ref), rho(S_s, S_ref)
        r1o, r1s = rho(o_s, o_1), rho(S_s, S_1)
        print(f"    {name}: vs oracle rho(o)={ro:.3e} rho(S)={rs:.3e}; vs one pass {r1o:.3e} {r1s:.3e}",
              flush=True)
        assert torch.isfinite(o_s.float()).all() and torch.isfinite(S_s).all()
        assert ro <= TOL[BF16] and rs <= TOL[BF16], (name, ro, rs)
        assert r1o <= TOL[BF16] and r1s <= TOL[BF16], (name, r1o, r1s)


def test_automatic_count_within_a_smaller_workspace():
    """B1 H4 T40000 with a workspace sized for eight segments (the library
    would pick more): the call takes the best count whose buffers fit, and
    its result is within the bar of the oracle (two heads checked)."""
    say("split within a capped workspace")
    B, T, H = 1, 40000, 4
    x = prefill_device(B, T, H, 128, 128, torch.bfloat16, 7100, s0_std=0.1)
    P_free = _lib.kda_chunk_fwd_auto_segments(B, T, H, 128, 128, _lib.KDA_BF16)
    small = _lib.kda_chunk_fwd_workspace_size(B, T, H, 128, 128, _lib.KDA_BF16, 8)
    assert P_free > 8 and small < _lib.kda_chunk_fwd_workspace_size(B, T, H, 128, 128, _lib.KDA_BF16)
    ws = torch.empty(small, device="cuda", dtype=torch.uint8)
    o, S = kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"], x["S0"], workspace=ws)
    torch.cuda.synchronize()
    for h in (0, 3):
        xs = {n: x[n][:, :, h:h + 1].contiguous() for n in ("q", "k", "v", "z", "beta")}
        g_ref = oracle.gate(xs["z"], x["A"][h:h + 1].contiguous())
        o_ref, S_ref = oracle.forward(xs["q"], xs["k"], xs["v"], g_ref, xs["beta"],
                                      x["S0"][:, h:h + 1].contiguous())
        ro, rs = rho(o[:, :, h:h + 1], o_ref), rho(S[:, h:h + 1], S_ref)
        print(f"    head {h}: rho(o)={ro:.3e} rho(S)={rs:.3e}", flush=True)
        assert ro <= TOL[torch.bfloat16] and rs <= TOL[torch.bfloat16], (h, ro, rs)
