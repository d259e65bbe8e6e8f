"""Full-size prefill workloads, end to end on the GPU, against the oracle's gate
and recurrence on sampled chains (chains are independent, so a sampled chain
is checked exactly).  Both forms of the step run: kda_chunk_fwd_gated (the
gate inside the chunk kernel, the launch configuration the benchmark times)
and kda_gate -> kda_chunk_fwd."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_gate_amd import inputs, kda_chunk_fwd, kda_chunk_fwd_gated, kda_gate
from kda_testutil import TOL, head_slice, rho, say, to_host64

pytestmark = pytest.mark.gpu


PATHS = ["fused", "two_kernel"]


def _gpu_run(w, path="fused"):
    x = inputs.workload_prefill_inputs(w, device="cuda")
    if path == "fused":
        o, ST = kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"], x["S0"])
    else:
        g = kda_gate(x["z"], x["A"])
        o, ST = kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], x["S0"])
        del g
    torch.cuda.synchronize()
    return x, o, ST


def _oracle_chain(x, b, h, t1=None, want_o=True):
    z = to_host64(head_slice(x["z"], b, h, 0, t1))
    g = oracle.gate(z, to_host64(x["A"][h:h + 1]))
    S0 = None if x["S0"] is None else to_host64(x["S0"][b:b + 1, h:h + 1].contiguous())
    return oracle.forward(to_host64(head_slice(x["q"], b, h, 0, t1)),
                          to_host64(head_slice(x["k"], b, h, 0, t1)),
                          to_host64(head_slice(x["v"], b, h, 0, t1)), g,
                          to_host64(x["beta"][b:b + 1, :t1, h:h + 1].contiguous()), S0,
                          want_o=want_o, col_block=8)


@pytest.mark.parametrize("path", PATHS)
def test_prefill_h8_t4k_all_heads(path):
    """B1 H8 T4096 d128 bf16, zero initial state: every head, every token."""
    w = inputs.WORKLOADS["prefill_h8_t4k"]
    say("full size", w.name, path)
    x, o, ST = _gpu_run(w, path)
    worst_o = worst_s = 0.0
    for h in range(w.H):
        o_ref, S_ref = _oracle_chain(x, 0, h)
        worst_o = max(worst_o, rho(head_slice(o, 0, h), o_ref))
        worst_s = max(worst_s, rho(ST[0:1, h:h + 1], S_ref))
    print(f"    worst rho(o)={worst_o:.3e} rho(S)={worst_s:.3e}", flush=True)
    assert worst_o <= TOL[w.dtype] and worst_s <= TOL[w.dtype]


@pytest.mark.parametrize("path", PATHS)
def test_prefill_b4_h32_t32k_sampled_chains(path):
    """B4 H32 T32768 d128 bf16 with heads 16..31 in decay stress: four whole
    chains (two ordinary, two stressed) checked on every token and on the
    final state."""
    w = inputs.WORKLOADS["prefill_b4_h32_t32k"]
    say("full size", w.name, path)
    x, o, ST = _gpu_run(w, path)
    assert torch.isfinite(o).all()
    for (b, h) in ((0, 3), (2, 10), (1, 20), (3, 31)):
        say("  chain", b, h)
        o_ref, S_ref = _oracle_chain(x, b, h)
        ro = rho(head_slice(o, b, h), o_ref)
        rs = rho(ST[b:b + 1, h:h + 1], S_ref)
        print(f"    b={b} h={h} rho(o)={ro:.3e} rho(S)={rs:.3e}", flush=True)
        assert ro <= TOL[w.dtype] and rs <= TOL[w.dtype]
    del x, o, ST
    torch.cuda.empty_cache()


@pytest.mark.parametrize("path", PATHS)
def test_prefill_h32_t1m_first_tokens_and_final_state(path):
    """B1 H32 T1048576 d128 bf16, initial state ~ N(0, 0.02): outputs of the
    first 8192 tokens on four heads, and the final state of two heads (their
    oracle runs over all 2^20 tokens).  Both paths take the library's
    sequence split at this size."""
    w = inputs.WORKLOADS["prefill_h32_t1m"]
    say("full size", w.name, path)
    x, o, ST = _gpu_run(w, path)
    assert torch.isfinite(o[:, :8192]).all() and torch.isfinite(ST).all()
    for h in (0, 9, 17, 30):
        o_ref, _ = _oracle_chain(x, 0, h, t1=8192)
        ro = rho(head_slice(o, 0, h, 0, 8192), o_ref)
        print(f"    h={h} first 8192 tokens rho(o)={ro:.3e}", flush=True)
        assert ro <= TOL[w.dtype]
    for h in (5, 26):
        say("  final state, head", h)
        _, S_ref = _oracle_chain(x, 0, h, want_o=False)
        rs = rho(ST[0:1, h:h + 1], S_ref)
        print(f"    h={h} final state rho(S)={rs:.3e}", flush=True)
        assert rs <= TOL[w.dtype]
    del x, o, ST
    torch.cuda.empty_cache()
