"""A seeded random sweep of prefill cases against the oracle: dtype, dk, dv,
batch, heads, a ragged sequence length, an initial state or none, the
decay-stress gate or the plain one, and the path (gate fused into the chunk
kernel, gate then chunk, a forced sequence split in either scheme, the position-pair diagonal
tiles), each drawn independently, so that combinations the dedicated tests do
not pair up are exercised.  Every case is within the oracle bar on o and the
final state."""
import random

import pytest
import torch

import oracle
from linear_attention_sequence_gate_amd import _lib, kda_chunk_fwd, kda_chunk_fwd_gated, kda_gate
from kda_testutil import TOL, prefill_device, rho, say

pytestmark = pytest.mark.gpu

N_CASES = 32


def _draw(i):
    r = random.Random(7000 + i)
    dtype = r.choice([torch.bfloat16, torch.bfloat16, torch.float32])
    dk = r.choice([32, 64] if dtype == torch.float32 else [32, 64, 128, 128])
    dv = r.choice([32, 64, 128])
    paths = ["gated", "two_kernel"]
    if dtype == torch.bfloat16 and dk == 128 and dv in (64, 128):
        paths += ["split", "pairwise"]
    return dict(dtype=dtype, dk=dk, dv=dv, B=r.randint(1, 3), H=r.choice([1, 2, 3, 5]),
                T=r.randint(1, 700), s0=r.random() < 0.5, stress=r.random() < 0.3,
                path=r.choice(paths), nseg=r.randint(2, 6), seed=7100 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_prefill_case_matches_oracle(i):
    c = _draw(i)
    say("random case", i, {k: (str(v) if k == "dtype" else v) for k, v in c.items()})
    x = prefill_device(c["B"], c["T"], c["H"], c["dk"], c["dv"], c["dtype"], c["seed"],
                       s0_std=0.3 if c["s0"] else 0.0, stress=3.0 if c["stress"] else None)
    path = c["path"]
    if path == "gated":
        o, S = kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"], x["S0"])
    else:
        g = kda_gate(x["z"], x["A"])
        flags = 0
        if path == "split":
            # either split scheme, from a generator of its own so that the
            # other draws stay what they were
            rerun = random.Random(9000 + i).random() < 0.5
            flags = _lib.kda_flag_segments(c["nseg"]) | (_lib.KDA_FLAG_SPLIT_FULL_RERUN if rerun else 0)
        elif path == "pairwise":
            flags = _lib.KDA_FLAG_PAIRWISE_DIAGONAL
        o, S = kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], x["S0"], flags=flags)
    torch.cuda.synchronize()
    g_ref = oracle.gate(x["z"], x["A"])
    o_ref, S_ref = oracle.forward(x["q"], x["k"], x["v"], g_ref, x["beta"], x["S0"])
    ro, rs = rho(o, o_ref), rho(S, S_ref)
    print(f"    rho(o)={ro:.3e} rho(S)={rs:.3e}", flush=True)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    assert ro <= TOL[c["dtype"]] and rs <= TOL[c["dtype"]], (c, ro, rs)
