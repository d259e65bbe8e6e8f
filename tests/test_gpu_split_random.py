"""A seeded random sweep of the sequence split against the oracle: batch,
heads, a ragged length, the segment count, the scheme (the last phase stopping
where a segment's transition vanished, or rerunning whole segments), the
workgroup layout (per chain, per 64-column slice, or the library's; dv = 128),
dv, an initial state or none, the fused gate or a given g, and per head a gate that
decays fast, slowly everywhere, or slowly over a random token range only, so
that transitions vanish within a chunk or two, late, never, or in some
segments and not in others (the chaining then mixes skipped steps and
products).  Every case is within the bf16 bar on o and the final state."""
import random

import pytest
import torch

import oracle
from linear_attention_sequence_gate_amd import _lib, kda_chunk_fwd, kda_chunk_fwd_gated
from kda_testutil import TOL, oracle_gate_f32, prefill_device, rho, say

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16
N_CASES = 24


def _draw(i):
    r = random.Random(9500 + i)
    B, H = r.choice([(1, 1), (1, 2), (1, 3), (2, 2), (1, 5), (2, 3)])
    T = r.randint(64, 3000)
    slow = []
    for _ in range(H):
        kind = r.choice(["fast", "fast", "slow", "range"])
        lo = r.randint(0, T - 1)
        hi = r.randint(lo + 1, T)
        slow.append((kind, lo, hi))
    dv = r.choice([64, 128])
    return dict(B=B, H=H, T=T, dv=dv, nseg=r.randint(2, 14),
                rerun=r.random() < 0.4, s0=r.random() < 0.5, fused=r.random() < 0.5,
                layout=r.choice(["chain", "slice", "auto"]) if dv == 128 else "auto",
                slow=slow, seed=9600 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_split_case_matches_oracle(i):
    c = _draw(i)
    say("random split", i, {k: v for k, v in c.items() if k != "slow"},
        [s[0] for s in c["slow"]])
    x = prefill_device(c["B"], c["T"], c["H"], 128, c["dv"], BF16, c["seed"],
                       s0_std=0.3 if c["s0"] else 0.0)
    z = x["z"].float()
    for h, (kind, lo, hi) in enumerate(c["slow"]):
        if kind == "slow":
            z[:, :, h] -= 6.0
        elif kind == "range":
            z[:, lo:hi, h] -= 6.0
    x["z"] = z.to(BF16)
    flags = _lib.kda_flag_segments(c["nseg"]) | (_lib.KDA_FLAG_SPLIT_FULL_RERUN if c["rerun"] else 0)
    flags |= {"chain": _lib.KDA_FLAG_WORKGROUP_PER_CHAIN, "slice": _lib.KDA_FLAG_WORKGROUP_PER_SLICE,
              "auto": 0}[c["layout"]]
    if c["fused"]:
        o, S = kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"], x["S0"],
                                   flags=flags)
        g_ref = oracle.gate(x["z"], x["A"])
    else:
        g_ref = oracle_gate_f32(x["z"], x["A"])
        o, S = kda_chunk_fwd(x["q"], x["k"], x["v"], g_ref.cuda(), x["beta"], x["S0"], flags=flags)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], g_ref, x["beta"], x["S0"])
    ro, rs = rho(o, o_ref), rho(S, S_ref)
    print(f"    rho(o)={ro:.3e} rho(S)={rs:.3e}", flush=True)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    assert ro <= TOL[BF16] and rs <= TOL[BF16], (c, ro, rs)
