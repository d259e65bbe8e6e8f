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


@pytest.mark.timeout(900)
def test_decode_full_size_1000_steps_all_pairs():
    """1000 consecutive in-place steps with fresh seeded inputs, every one of
    the 256 x 32 (sequence, head) pairs followed by the oracle through all
    1000 steps: every step's outputs and the final states."""
    w = inputs.WORKLOADS["decode_256x32"]
    say("decode full size, 1000 steps, all pairs")
    st = inputs.make_decode_state(w.B, w.H, w.dk, w.dv, w.seed, device="cuda", s0_std=w.s0_std)
    S = st["S"].clone()
    S_ref = np.ascontiguousarray(st["S"].double().cpu().numpy())
    A_host = st["A"].cpu()
    acc_o = oracle.RhoAccumulator()
    for t in range(w.decode_steps):
        x = _step_inputs(w.B, w.H, w.dk, w.dv, w.dtype, w.seed, t)
        o = kda_decode_step(x["q"], x["k"], x["v"], x["z"], st["A"], x["beta"], S)
        o_ref, _ = oracle.decode_step(x["q"], x["k"], x["v"], x["z"], A_host, x["beta"], S_ref,
                                      inplace=True)
        acc_o.add(o, o_ref)
        if t % 250 == 0:
            say("decode step", t, "rho(o) so far", acc_o.value())
    torch.cuda.synchronize()
    rs = rho(S, S_ref)
    print(f"    rho(o) over 1000 steps={acc_o.value():.3e} rho(final S)={rs:.3e}", flush=True)
    assert acc_o.value() <= TOL[w.dtype]
    assert rs <= TOL[w.dtype]
    del st, S
    torch.cuda.empty_cache()


def test_decode_continues_a_fused_gate_prefill():
    """bf16, dk = dv = 128: kda_chunk_fwd_gated over T0 tokens, then T1 decode
    steps.  Both legs against the oracle:
      - the prefill's outputs and state, and the decode outputs and state,
        against the oracle's token loop over all T0 + T1 tokens (bf16 bar);
      - the decode steps started from the prefill's own GPU state, against
        the oracle's decode steps started from that same state: the decode
        kernel's arithmetic is fp32 throughout, so its state meets 1e-4, and
        its bf16 outputs meet bf16's unit roundoff (2^-8, half an ulp relative
        to the value) of the largest output plus that: 2^-8 + 1e-4."""
    from linear_attention_sequence_gate_amd import kda_chunk_fwd_gated
    N, H, d, T0, T1 = 2, 4, 128, 200, 12
    say("fused prefill then decode, against the oracle")
    x = inputs.make_prefill_inputs(N, T0 + T1, H, d, d, torch.bfloat16, 79, device="cuda",
                                   s0_std=0.02, stress_heads_mean=3.0)
    head = {n: x[n][:, :T0].clone() for n in ("q", "k", "v", "z", "beta")}
    o_head, S = kda_chunk_fwd_gated(head["q"], head["k"], head["v"], head["z"], x["A"],
                                    head["beta"], x["S0"])
    torch.cuda.synchronize()
    S_start = np.ascontiguousarray(S.double().cpu().numpy())    # the prefill's own state
    outs = []
    for t in range(T0, T0 + T1):
        sl = lambda a: a[:, t].contiguous()
        outs.append(kda_decode_step(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["z"]), x["A"],
                                    sl(x["beta"]), S))
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, dim=1)

    g_ref = oracle.gate(x["z"], x["A"])
    o_all, S_all = oracle.forward(x["q"], x["k"], x["v"], g_ref, x["beta"], x["S0"])
    assert rho(o_head, o_all[:, :T0]) <= TOL[torch.bfloat16]
    assert rho(o_dec, o_all[:, T0:]) <= TOL[torch.bfloat16]
    assert rho(S, S_all) <= TOL[torch.bfloat16]

    S_ref = S_start
    o_ref = []
    A_host = x["A"].cpu()
    for t in range(T0, T0 + T1):
        sl = lambda a: a[:, t]
        o_t, S_ref = oracle.decode_step(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["z"]), A_host,
                                        sl(x["beta"]), S_ref, inplace=True)
        o_ref.append(o_t)
    o_ref = np.stack(o_ref, axis=1)
    ro, rs = rho(o_dec, o_ref), rho(S, S_ref)
    print(f"    decode from the prefill's state: rho(o)={ro:.3e} rho(S)={rs:.3e}", flush=True)
    assert rs <= 1e-4
    assert ro <= 2.0 ** -8 + 1e-4
