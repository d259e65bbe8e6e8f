"""Seeded synthetic inputs for Kimi Delta Attention (KDA).

This module draws the random tensors that both the HIP path and the fp64 oracle
consume.  It holds none of the method's arithmetic: it never evaluates the gate,
the decay, the delta rule or an output.  It only draws values with the
distributions of the workloads below, L2-normalises q and k per token (the
caller's job: the library applies no normalisation or scaling) and rounds to
the input dtype.

Page context: "Kimi K3 internal structure analysis" (molayo1419.me), section
"Sequence mixing: 3 KDA layers per global MLA layer", describes KDA as a
recurrent linear attention with a fixed-size state, a channel-wise retention
factor and the gate parameters (A, z).  The pages give no shapes, seeds or
distributions; the workload table below states them.

Draw order inside one generator: q, k, v, beta-logit, z, A, S0.
Normal distributions are written N(mean, std) (std, not variance).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

__all__ = [
    "Workload",
    "WORKLOADS",
    "make_prefill_inputs",
    "make_decode_state",
    "make_decode_step_inputs",
    "decode_step_seed",
]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int          # batch (prefill) or number of independent sequences (decode)
    H: int
    T: int          # tokens per sequence (prefill); 1 for decode
    dk: int
    dv: int
    dtype: torch.dtype
    seed: int
    s0_std: float = 0.0          # 0 means a zero initial state
    stress_heads_mean: Optional[float] = None  # z mean for heads h >= H/2
    decode_steps: int = 0
    note: str = ""


# Every workload's q, k ~ N(0,1) L2-normalised per token, v ~ N(0,1),
# beta = sigmoid(N(0,1)), z ~ N(0,1) per token/head/channel, A ~ N(0, 0.5)
# per head and key channel.
WORKLOADS = {
    "small_f32": Workload(
        "small_f32", B=1, H=1, T=128, dk=32, dv=32, dtype=torch.float32, seed=1000,
        note="B1 H1 T128 d32 fp32, zero initial state"),
    "prefill_h8_t4k": Workload(
        "prefill_h8_t4k", B=1, H=8, T=4096, dk=128, dv=128, dtype=torch.bfloat16, seed=1001,
        note="B1 H8 T4096 d128 bf16, zero initial state"),
    "prefill_b4_h32_t32k": Workload(
        "prefill_b4_h32_t32k", B=4, H=32, T=32768, dk=128, dv=128, dtype=torch.bfloat16,
        seed=1002, stress_heads_mean=3.0,
        note="B4 H32 T32768 d128 bf16; heads 16..31 draw z ~ N(3,1) so the gate sits "
             "near its floor (decay-range stress)"),
    "prefill_h32_t1m": Workload(
        "prefill_h32_t1m", B=1, H=32, T=1 << 20, dk=128, dv=128, dtype=torch.bfloat16,
        seed=1003, s0_std=0.02,
        note="B1 H32 T1048576 d128 bf16, initial state ~ N(0, 0.02)"),
    "decode_256x32": Workload(
        "decode_256x32", B=256, H=32, T=1, dk=128, dv=128, dtype=torch.bfloat16,
        seed=1004, s0_std=0.02, decode_steps=1000,
        note="256 sequences x H32, d128, one bf16 token per step, fp32 state ~ N(0,0.02) "
             "updated in place, fresh seeded inputs each step"),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    """L2-normalise along the last axis (fp32)."""
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def make_prefill_inputs(B: int, T: int, H: int, dk: int, dv: int, dtype: torch.dtype,
                        seed: int, device="cpu", s0_std: float = 0.0,
                        stress_heads_mean: Optional[float] = None) -> dict:
    """Draw one prefill problem.

    Returns a dict with q, k [B,T,H,dk], v [B,T,H,dv], beta [B,T,H] and z
    [B,T,H,dk] in `dtype`; A [H,dk] fp32; S0 [B,H,dk,dv] fp32 or None.
    Values are generated in fp32 and rounded once to `dtype` (RNE).
    """
    gen = _gen(seed, device)
    f32 = torch.float32
    q = _unit_rows(torch.randn(B, T, H, dk, generator=gen, device=device, dtype=f32))
    q = q.to(dtype)
    k = _unit_rows(torch.randn(B, T, H, dk, generator=gen, device=device, dtype=f32))
    k = k.to(dtype)
    v = torch.randn(B, T, H, dv, generator=gen, device=device, dtype=f32).to(dtype)
    beta = torch.sigmoid(torch.randn(B, T, H, generator=gen, device=device, dtype=f32)).to(dtype)
    z = torch.randn(B, T, H, dk, generator=gen, device=device, dtype=f32)
    if stress_heads_mean is not None:
        z[:, :, H // 2:, :] += stress_heads_mean
    z = z.to(dtype)
    A = torch.randn(H, dk, generator=gen, device=device, dtype=f32) * 0.5
    S0 = None
    if s0_std > 0.0:
        S0 = torch.randn(B, H, dk, dv, generator=gen, device=device, dtype=f32) * s0_std
    return dict(q=q, k=k, v=v, beta=beta, z=z, A=A, S0=S0)


def workload_prefill_inputs(w: Workload, device="cpu", T: Optional[int] = None,
                            B: Optional[int] = None, H: Optional[int] = None) -> dict:
    """Prefill inputs of a named workload (optionally with fewer tokens/batch/heads)."""
    return make_prefill_inputs(B or w.B, T or w.T, H or w.H, w.dk, w.dv, w.dtype, w.seed,
                               device=device, s0_std=w.s0_std,
                               stress_heads_mean=w.stress_heads_mean)


def make_decode_state(N: int, H: int, dk: int, dv: int, seed: int, device="cpu",
                      s0_std: float = 0.02) -> dict:
    """The decode state [N,H,dk,dv] fp32 ~ N(0, s0_std) and the gate parameter A [H,dk]."""
    gen = _gen(seed, device)
    A = torch.randn(H, dk, generator=gen, device=device, dtype=torch.float32) * 0.5
    S = torch.randn(N, H, dk, dv, generator=gen, device=device, dtype=torch.float32) * s0_std
    return dict(A=A, S=S)


def decode_step_seed(base_seed: int, step: int) -> int:
    return base_seed + 7919 * (step + 1)


def make_decode_step_inputs(N: int, H: int, dk: int, dv: int, dtype: torch.dtype,
                            base_seed: int, step: int, device="cpu") -> dict:
    """Fresh per-step q, k [N,H,dk], v [N,H,dv], beta [N,H], z [N,H,dk]."""
    gen = _gen(decode_step_seed(base_seed, step), device)
    f32 = torch.float32
    q = _unit_rows(torch.randn(N, H, dk, generator=gen, device=device, dtype=f32)).to(dtype)
    k = _unit_rows(torch.randn(N, H, dk, generator=gen, device=device, dtype=f32)).to(dtype)
    v = torch.randn(N, H, dv, generator=gen, device=device, dtype=f32).to(dtype)
    beta = torch.sigmoid(torch.randn(N, H, generator=gen, device=device, dtype=f32)).to(dtype)
    z = torch.randn(N, H, dk, generator=gen, device=device, dtype=f32).to(dtype)
    return dict(q=q, k=k, v=v, beta=beta, z=z)
