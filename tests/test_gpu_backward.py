"""GPU parity of kda_chunk_bwd (reverse mode of the recurrence) against the
oracle's reverse mode on the same inputs, for both paths (16-token chunks on
the matrix cores, and token by token): fp32 and bf16, every (dk, dv) family,
T around the 8-token checkpoint and 16-token chunk spacings, with and without
the initial state and the final-state gradient, the decay at the gate's
floor, and (token path) with the floor removed.  The gradients are fp32
arithmetic for either input dtype (the oracle reads the same rounded inputs),
so every case is held to 1e-4."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_gate_amd import KdaError, kda_chunk_bwd, kda_chunk_bwd_workspace_size_flags
from linear_attention_sequence_gate_amd._lib import KDA_FLAG_CHECK_RANGE, KDA_FLAG_TOKEN_BACKWARD
from kda_testutil import GRAD_TOL, oracle_gate_f32, prefill_device, rho, say

pytestmark = pytest.mark.gpu

PATHS = {"chunked": 0, "token": KDA_FLAG_TOKEN_BACKWARD}


def _run(dtype, B, T, H, dk, dv, seed, s0=True, dst=True, g=None, path="chunked"):
    x = prefill_device(B, T, H, dk, dv, dtype, seed, s0_std=0.3 if s0 else 0.0)
    g_f32 = oracle_gate_f32(x["z"], x["A"]) if g is None else g
    gen = torch.Generator(device="cuda").manual_seed(seed + 1)
    d_o = torch.randn(B, T, H, dv, device="cuda", generator=gen).to(dtype)
    dST = torch.randn(B, H, dk, dv, device="cuda", generator=gen) if dst else None
    out = kda_chunk_bwd(x["q"], x["k"], x["v"], g_f32.cuda(), x["beta"], x["S0"], d_o, dST,
                        flags=PATHS[path])
    torch.cuda.synchronize()
    ref = oracle.backward_np(x["q"], x["k"], x["v"], g_f32, x["beta"], x["S0"], d_o, dST)
    res = {}
    for name, rname in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dg", "dg"), ("dbeta", "dbeta"),
                        ("d_initial_state", "dS0")):
        r = rho(out[name], ref[rname])
        res[name] = r
        assert np.isfinite(out[name].cpu().numpy()).all(), name
    print("    " + " ".join(f"{k}={v:.1e}" for k, v in res.items()), flush=True)
    for name, r in res.items():
        assert r <= GRAD_TOL, (name, r)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T", [1, 8, 9, 16, 17, 37])
def test_backward_f32_small(T, path):
    say("backward f32", path, T)
    _run(torch.float32, 2, T, 2, 32, 32, 700 + T, path=path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dk,dv,T", [(64, 128, 20), (128, 64, 17), (32, 64, 24), (128, 128, 48)])
def test_backward_f32_shapes(dk, dv, T, path):
    say("backward f32", path, dk, dv, T)
    _run(torch.float32, 1, T, 2, dk, dv, 710 + T, s0=False, path=path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dk,dv,T", [(128, 128, 70), (32, 64, 13), (64, 32, 33), (32, 128, 40)])
def test_backward_bf16(dk, dv, T, path):
    say("backward bf16", path, dk, dv, T)
    _run(torch.bfloat16, 1, T, 3, dk, dv, 720 + T, dst=False, path=path)


def test_backward_chunked_many_chunks():
    """Several chains of many 16-token chunks and a ragged tail, bf16, d = 128,
    in the launch shape of the benchmark (chains a multiple of 8)."""
    say("backward chunked B2 H4 T301 d128")
    _run(torch.bfloat16, 2, 301, 4, 128, 128, 740)


@pytest.mark.parametrize("path", PATHS)
def test_backward_decay_at_the_floor(path):
    """g = -5 everywhere: every 16-token chunk's decay sum is exactly -80, the
    largest range the chunked path's mid-chunk reference has to cover."""
    say("backward at the floor", path)
    T, H, d = 50, 2, 64
    g = torch.full((1, T, H, d), -5.0)
    _run(torch.float32, 1, T, H, d, d, 750, g=g, path=path)


def test_backward_without_the_floor():
    """The token-level reverse mode assumes nothing about the decay range."""
    say("backward without the floor")
    T, H, d = 40, 2, 64
    g = -20.0 * torch.rand(1, T, H, d, generator=torch.Generator().manual_seed(731))
    _run(torch.float32, 1, T, H, d, d, 730, g=g, path="token")


def test_backward_range_check():
    """The chunked path's range check rejects g below the floor (KDA_ERR_RANGE)."""
    say("backward range check")
    x = prefill_device(1, 32, 2, 32, 32, torch.float32, 760)
    g = torch.full((1, 32, 2, 32), -6.0, device="cuda")
    d_o = torch.ones(1, 32, 2, 32, device="cuda")
    with pytest.raises(KdaError) as err:
        kda_chunk_bwd(x["q"], x["k"], x["v"], g, x["beta"], None, d_o, flags=KDA_FLAG_CHECK_RANGE)
    assert err.value.code == -4
    g.fill_(-1.0)
    out = kda_chunk_bwd(x["q"], x["k"], x["v"], g, x["beta"], None, d_o, flags=KDA_FLAG_CHECK_RANGE)
    torch.cuda.synchronize()
    assert torch.isfinite(out["dq"]).all()


def test_backward_benchmark_shape_sampled_chains():
    """The benchmark's backward workload (B4 H32 T4096 d128 bf16, heads 16-31
    decay-stress), one call in the benchmark's launch configuration; one
    ordinary and one decay-stress chain compared in full with the oracle."""
    say("backward chunked B4 H32 T4096 d128 (two chains against the oracle)")
    B, T, H, d = 4, 4096, 32, 128
    x = prefill_device(B, T, H, d, d, torch.bfloat16, 4243, s0_std=0.02, stress=3.0)
    g = oracle_gate_f32(x["z"], x["A"])
    gen = torch.Generator(device="cuda").manual_seed(4244)
    d_o = torch.randn(B, T, H, d, device="cuda", generator=gen).to(torch.bfloat16)
    dST = torch.randn(B, H, d, d, device="cuda", generator=gen)
    out = kda_chunk_bwd(x["q"], x["k"], x["v"], g.cuda(), x["beta"], x["S0"], d_o, dST)
    torch.cuda.synchronize()
    for b, h in ((0, 3), (3, 29)):
        chain = lambda t: t[b:b + 1, :, h:h + 1].contiguous()
        ref = oracle.backward_np(chain(x["q"]), chain(x["k"]), chain(x["v"]), chain(g),
                                 chain(x["beta"]), x["S0"][b:b + 1, h:h + 1].contiguous(),
                                 chain(d_o), dST[b:b + 1, h:h + 1].contiguous())
        res = {name: rho(chain(out[name]), ref[rname])
               for name, rname in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dg", "dg"),
                                   ("dbeta", "dbeta"))}
        res["d_initial_state"] = rho(out["d_initial_state"][b:b + 1, h:h + 1], ref["dS0"])
        print(f"    b{b} h{h} " + " ".join(f"{k}={v:.1e}" for k, v in res.items()), flush=True)
        for name, r in res.items():
            assert r <= GRAD_TOL, (b, h, name, r)


# --------------------------------------------------------------------------
# Segmented chunked reverse mode (workspace smaller than the whole sequence)
# --------------------------------------------------------------------------

GRADS = (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dg", "dg"), ("dbeta", "dbeta"),
         ("d_initial_state", "dS0"))


@pytest.mark.parametrize("dtype,B,T,H,dk,dv,seg,slow", [
    (torch.bfloat16, 2, 301, 4, 128, 128, 64, False),   # 5 segments, ragged last one
    (torch.float32, 1, 100, 2, 64, 32, 32, False),      # 4 segments, a 4-token last one
    (torch.float32, 1, 200, 2, 32, 32, 32, True),       # slow decay: gradients cross 7 segments
    (torch.bfloat16, 1, 130, 2, 128, 64, 32, True),
])
def test_backward_segmented_matches_oracle_and_one_segment(dtype, B, T, H, dk, dv, seg, slow):
    say("backward segmented", dtype, B, T, H, dk, dv, "segments of", seg, "slow" if slow else "")
    x = prefill_device(B, T, H, dk, dv, dtype, 770 + T, s0_std=0.3)
    # slow: z - 6 puts g near -0.01, so a state gradient survives hundreds of tokens
    g = oracle_gate_f32(x["z"].float() - 6.0 if slow else x["z"], x["A"])
    gen = torch.Generator(device="cuda").manual_seed(771 + T)
    d_o = torch.randn(B, T, H, dv, device="cuda", generator=gen).to(dtype)
    dST = torch.randn(B, H, dk, dv, device="cuda", generator=gen)
    args = (x["q"], x["k"], x["v"], g.cuda(), x["beta"], x["S0"], d_o, dST)
    one = kda_chunk_bwd(*args)
    seg_out = kda_chunk_bwd(*args, segment_tokens=seg)
    torch.cuda.synchronize()
    ref = oracle.backward_np(x["q"], x["k"], x["v"], g, x["beta"], x["S0"], d_o, dST)
    res = {name: rho(seg_out[name], ref[rname]) for name, rname in GRADS}
    same = {name: bool(torch.equal(seg_out[name], one[name])) for name, _ in GRADS}
    print("    " + " ".join(f"{k}={v:.1e}" for k, v in res.items()), "bit-equal to one segment:",
          all(same.values()), flush=True)
    for name, _ in GRADS:
        assert torch.isfinite(seg_out[name]).all(), name
        assert res[name] <= GRAD_TOL, (name, res[name])
        assert rho(seg_out[name], one[name]) <= 1e-6, name


@pytest.mark.timeout(900)
def test_backward_t1m_within_a_bounded_workspace():
    """B1 H32 T1M d128 bf16: about 230 GB of workspace in one segment, run in
    32768-token segments (under 8 GB).  Two chains are checked against the
    oracle on three windows: the first 4096 tokens, 4096 tokens around the
    first segment boundary, and the last 4096.  The gate g = -5 U(0, 1)
    decays every channel by about e^-2.5 a token, so a state gradient from 512
    tokens further on is exactly zero in fp64 (e^-1280): each window's oracle
    runs the forward recurrence from the sequence start (C oracle) and the
    reverse mode over the window plus 512 tokens, whose final state gradient
    is then zero (the true one for the last window)."""
    B, T, H, d = 1, 1 << 20, 32, 128
    seg = 32768
    say("backward B1 H32 T1M in 32768-token segments")
    x = prefill_device(B, T, H, d, d, torch.bfloat16, 4343, s0_std=0.02)
    del x["z"]
    gen = torch.Generator(device="cuda").manual_seed(4344)
    g = -5.0 * torch.rand(B, T, H, d, device="cuda", generator=gen)
    d_o = torch.randn(B, T, H, d, device="cuda", generator=gen).to(torch.bfloat16)
    dST = torch.randn(B, H, d, d, device="cuda", generator=gen)
    ws_bytes = kda_chunk_bwd_workspace_size_flags(B, T, H, d, d, 1, 0, seg)
    assert ws_bytes < 8e9
    out = kda_chunk_bwd(x["q"], x["k"], x["v"], g, x["beta"], x["S0"], d_o, dST, segment_tokens=seg)
    torch.cuda.synchronize()
    for name, _ in GRADS:
        assert torch.isfinite(out[name]).all(), name
    margin = 512
    for h in (3, 29):
        chain = lambda t, a, b: t[:, a:b, h:h + 1].contiguous()
        for (t0, t1) in ((0, 4096), (seg - 2048, seg + 2048), (T - 4096, T)):
            say("  chain", h, "window", t0, t1)
            S_start = x["S0"][:, h:h + 1].contiguous()
            if t0 > 0:
                _, S_start = oracle.forward(chain(x["q"], 0, t0), chain(x["k"], 0, t0),
                                            chain(x["v"], 0, t0), chain(g, 0, t0),
                                            chain(x["beta"], 0, t0), S_start, want_o=False,
                                            col_block=8)
            t2 = min(t1 + margin, T)
            dS_end = dST[:, h:h + 1].contiguous() if t2 == T else None
            ref = oracle.backward_np(chain(x["q"], t0, t2), chain(x["k"], t0, t2),
                                     chain(x["v"], t0, t2), chain(g, t0, t2),
                                     chain(x["beta"], t0, t2), S_start, chain(d_o, t0, t2), dS_end)
            n = t1 - t0
            res = {name: rho(chain(out[name], t0, t1), ref[rname][:, :n])
                   for name, rname in GRADS[:-1]}
            if t0 == 0:
                res["d_initial_state"] = rho(out["d_initial_state"][:, h:h + 1], ref["dS0"])
            print(f"    h{h} [{t0}, {t1}) " + " ".join(f"{k}={v:.1e}" for k, v in res.items()),
                  flush=True)
            for name, r in res.items():
                assert r <= GRAD_TOL, (h, t0, name, r)
    del x, g, d_o, out
    torch.cuda.empty_cache()
