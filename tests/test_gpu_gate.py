"""GPU parity of kda_gate against the oracle's gate (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_gate_amd import inputs, kda_gate
from kda_testutil import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", [(1, 1, 1, 32), (2, 37, 3, 64), (1, 129, 4, 128)])
def test_gate_matches_oracle(dtype, shape):
    B, T, H, dk = shape
    say("gate", dtype, shape)
    x = inputs.make_prefill_inputs(B, T, H, dk, dk, dtype, 11, device="cuda", stress_heads_mean=3.0)
    z = (x["z"].float() * 4.0).to(dtype)          # widen the argument range
    g = kda_gate(z, x["A"])
    torch.cuda.synchronize()
    ref = oracle.gate(z, x["A"])
    got = g.double().cpu().numpy()
    # fp32 evaluation of exp / sigmoid: a few ulp of |g| <= 5
    np.testing.assert_allclose(got, ref, rtol=0, atol=2e-6)
    assert np.all(got <= 0.0) and np.all(got >= -5.0)


def test_gate_extremes():
    say("gate extremes")
    z = torch.tensor([0.0, 1e-30, -1e-30, 60.0, -60.0, 1e4, -1e4, 3.0], dtype=torch.float32)
    z = z.repeat(4).reshape(1, 1, 1, 32).cuda()
    A = torch.zeros(1, 32, device="cuda")
    g = kda_gate(z, A)
    torch.cuda.synchronize()
    got = g.double().cpu().numpy().ravel()
    ref = oracle.gate(z, A).ravel()
    np.testing.assert_allclose(got, ref, rtol=0, atol=2e-6)
    assert got[0] == -2.5
    assert got[5] == -5.0 and got[6] > -1e-30


def test_gate_full_size_sampled():
    """B4 H32 T32768 d128 bf16 (the decay-stress workload) in the launch the
    benchmark times; 2^20 sampled elements checked one by one against the
    oracle (each sample laid out as its own head with its own A entry)."""
    w = inputs.WORKLOADS["prefill_b4_h32_t32k"]
    say("gate full size", w.name)
    x = inputs.workload_prefill_inputs(w, device="cuda")
    g = kda_gate(x["z"], x["A"])
    torch.cuda.synchronize()
    idx = torch.randint(0, g.numel(), (1 << 20,), generator=torch.Generator().manual_seed(5))
    idx_d = idx.cuda()
    zs = x["z"].reshape(-1)[idx_d].double().cpu().numpy()
    As = x["A"].reshape(-1)[(idx_d % (w.H * w.dk))].double().cpu().numpy()
    got = g.reshape(-1)[idx_d].double().cpu().numpy()
    ref = oracle.gate(zs.reshape(1, 1, -1, 1), As.reshape(-1, 1)).reshape(-1)
    np.testing.assert_allclose(got, ref, rtol=0, atol=2e-6)
    sums = oracle.tile_log_decay_sums(g[:, :4096].cpu())
    assert sums.min() >= -80.0 and sums.max() <= 0.0
    del x, g
    torch.cuda.empty_cache()
