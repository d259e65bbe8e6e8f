"""GPU parity of kda_gate_bwd (reverse mode of the gate) against the oracle's
fp64 reverse mode on the same inputs: fp32 and bf16 z, every dk, row counts
that do not divide into the row ranges, saturated gate inputs, and the
backward benchmark's full size (dA summed over 16384 rows per column)."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_gate_amd import kda_gate_bwd
from kda_testutil import GRAD_TOL, prefill_device, rho, say

pytestmark = pytest.mark.gpu


def _check(z, A, dg, dtype):
    out = kda_gate_bwd(z, A, dg)
    torch.cuda.synchronize()
    ref = oracle.gate_backward_np(z, A, dg)
    r = {"dz": rho(out["dz"], ref["dz"]), "dA": rho(out["dA"], ref["dA"])}
    print("    " + " ".join(f"{k}={v:.1e}" for k, v in r.items()), flush=True)
    for k, v in r.items():
        assert np.isfinite(out[k].cpu().numpy()).all(), k
        assert v <= GRAD_TOL, (k, v)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,T,H,dk", [(2, 37, 3, 32), (1, 5, 2, 64), (2, 300, 4, 128), (1, 1, 1, 32)])
def test_gate_backward(dtype, B, T, H, dk):
    say("gate backward", dtype, B, T, H, dk)
    x = prefill_device(B, T, H, dk, dk, dtype, 800 + T, stress=3.0)
    gen = torch.Generator(device="cuda").manual_seed(801 + T)
    dg = torch.randn(B, T, H, dk, device="cuda", generator=gen)
    _check(x["z"], x["A"], dg, dtype)


def test_gate_backward_saturated_inputs():
    """|exp(A) z| up to ~1e3: sigmoid' underflows to 0 without NaN."""
    say("gate backward, saturated inputs")
    gen = torch.Generator(device="cuda").manual_seed(810)
    z = 200.0 * torch.randn(2, 16, 2, 32, device="cuda", generator=gen)
    A = torch.randn(2, 32, device="cuda", generator=gen)
    dg = torch.randn(2, 16, 2, 32, device="cuda", generator=gen)
    _check(z, A, dg, torch.float32)


def test_gate_backward_benchmark_size():
    say("gate backward B4 T4096 H32 d128 bf16")
    x = prefill_device(4, 4096, 32, 128, 128, torch.bfloat16, 820, stress=3.0)
    gen = torch.Generator(device="cuda").manual_seed(821)
    dg = torch.randn(4, 4096, 32, 128, device="cuda", generator=gen)
    _check(x["z"], x["A"], dg, torch.bfloat16)
