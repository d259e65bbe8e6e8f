"""Helpers for the GPU parity tests: device inputs from the shared seeded
generator, host copies for the oracle, and the parity metric.

Tolerances (max|gpu - oracle| / max|oracle|, separately for o and the final
state): 1e-4 for fp32 inputs, 1e-2 for bf16 inputs.  Gradients are fp32
arithmetic whatever the input dtype (both sides read the same rounded inputs),
so they are held to 1e-4 (GRAD_TOL).
"""
import sys

import numpy as np
import torch

import oracle
from linear_attention_sequence_gate_amd import inputs

TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-2}
GRAD_TOL = 1e-4


def say(*a):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def rho(x, ref) -> float:
    return oracle.rho(x, ref)


def to_host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def head_slice(x: torch.Tensor, b: int, h: int, t0: int = 0, t1=None) -> torch.Tensor:
    """[B,T,H,...] -> [1, t1-t0, 1, ...] contiguous copy of one (b, h) chain."""
    return x[b:b + 1, t0:t1, h:h + 1].contiguous()


def prefill_device(B, T, H, dk, dv, dtype, seed, s0_std=0.0, stress=None, device="cuda"):
    return inputs.make_prefill_inputs(B, T, H, dk, dv, dtype, seed, device=device,
                                      s0_std=s0_std, stress_heads_mean=stress)


def oracle_gate_f32(z: torch.Tensor, A: torch.Tensor) -> torch.Tensor:
    """The oracle's gate rounded once to fp32 (an input both sides then share)."""
    return torch.from_numpy(oracle.gate(z, A)).to(torch.float32)


def oracle_chain(x: dict, g_host: np.ndarray, b: int, h: int, t1=None, want_o=True,
                 col_block=8):
    """Oracle forward for one (b, h) chain of a device problem, first t1 tokens."""
    q = to_host64(head_slice(x["q"], b, h, 0, t1))
    k = to_host64(head_slice(x["k"], b, h, 0, t1))
    v = to_host64(head_slice(x["v"], b, h, 0, t1))
    beta = to_host64(x["beta"][b:b + 1, :t1, h:h + 1].contiguous())
    gg = np.ascontiguousarray(g_host)
    S0 = None
    if x.get("S0") is not None:
        S0 = to_host64(x["S0"][b:b + 1, h:h + 1].contiguous())
    return oracle.forward(q, k, v, gg, beta, S0, want_o=want_o, col_block=col_block)
