#!/usr/bin/env python3
"""KDA hot-path benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A timed step is one pass of the prefill hot path over the synthetic batch
B4 H32 T32768 d128 bf16 (half of the heads with the gate near its floor):
kda_gate (z -> g) followed by kda_chunk_fwd (q, k, v, g, beta -> o, final
state).  The decode step (256 sequences x H32, d128, fp32 state of 512 MiB
updated in place) is timed in the same run over 1000 consecutive steps with
fresh pre-generated inputs, and reported in the same JSON line.

value   = prefill tokens/s (B*T tokens, all 32 heads, per wall-clock step)
roofline= the chunked-prefill kernel against HBM (its arithmetic intensity,
          ~99 flop/B, is below the MI355X ridge of ~312 flop/B)
cpu_baseline = the fp64 oracle timed on this host on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from linear_attention_sequence_gate_amd import _lib, inputs  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure

PREFILL = inputs.WORKLOADS["prefill_b4_h32_t32k"]
DECODE = inputs.WORKLOADS["decode_256x32"]


def prefill_work(w, B=None, T=None, H=None):
    """Algorithmic bytes and flops of one kda_chunk_fwd call (and of the gate)."""
    B, T, H = B or w.B, T or w.T, H or w.H
    dk, dv = w.dk, w.dv
    e = 2 if w.dtype == torch.bfloat16 else 4
    ht = B * T * H                                   # head-tokens
    chunk_bytes = ht * ((2 * dk + dv) * e + dk * 4 + e + dv * e)   # q,k,v + g + beta + o
    chunk_bytes += B * H * dk * dv * 4 * (2 if w.s0_std > 0 else 1)  # state out (and in)
    Lbar = (64 + 16) / 2                             # mean causal length with dense diagonal tiles
    flops_per_ht = 6 * dk * dv + 2 * 2 * Lbar * dk + 2 * 2 * Lbar * dv + 2 * Lbar * dv
    # = 6 d^2 (W S, Q S, K^T U) + A, P (2 L d each) + W, U' (2 L d each) + P U (2 L d);
    # plus the UT inverse (~ C^2 * 16 / 3 per chunk ~ 1.4k per head-token at C=64)
    flops_per_ht += 64 * 64 * 16 / 3 / 64 * 4
    gate_bytes = ht * dk * (e + 4)
    return dict(head_tokens=ht, chunk_bytes=chunk_bytes, chunk_flops=flops_per_ht * ht,
                gate_bytes=gate_bytes)


def decode_bytes(w):
    N, H, dk, dv = w.B, w.H, w.dk, w.dv
    e = 2
    return N * H * (2 * dk * dv * 4 + (3 * dk + dv) * e + e + dv * e) + H * dk * 4


def time_prefill(steps, warmup):
    w = PREFILL
    dev = torch.device("cuda")
    x = inputs.workload_prefill_inputs(w, device=dev)
    g = torch.empty(x["z"].shape, device=dev, dtype=torch.float32)
    o = torch.empty(w.B, w.T, w.H, w.dv, device=dev, dtype=w.dtype)
    ST = torch.empty(w.B, w.H, w.dk, w.dv, device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream()

    def step(evs=None):
        if evs: evs[0].record(stream)
        _lib.kda_gate(x["z"], x["A"], g, stream=stream)
        if evs: evs[1].record(stream)
        _lib.kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], x["S0"], final_state=ST, o=o,
                           stream=stream)
        if evs: evs[2].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gate_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    chunk_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    return dict(x=x, g=g, o=o, ST=ST, wall_s=wall, gate_ms=gate_ms, chunk_ms=chunk_ms)


def time_decode(nsteps=1000, warmup=20):
    w = DECODE
    dev = torch.device("cuda")
    st = inputs.make_decode_state(w.B, w.H, w.dk, w.dv, w.seed, device=dev, s0_std=w.s0_std)
    S = st["S"]
    # fresh seeded inputs for every timed step, generated before timing
    xs = [inputs.make_decode_step_inputs(w.B, w.H, w.dk, w.dv, w.dtype, w.seed, t, device=dev)
          for t in range(nsteps)]
    o = torch.empty(w.B, w.H, w.dv, device=dev, dtype=w.dtype)
    stream = torch.cuda.current_stream()
    for t in range(warmup):
        x = xs[t % nsteps]
        _lib.kda_decode_step(x["q"], x["k"], x["v"], x["z"], st["A"], x["beta"], S, o, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for t in range(nsteps):
        x = xs[t]
        _lib.kda_decode_step(x["q"], x["k"], x["v"], x["z"], st["A"], x["beta"], S, o, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / nsteps
    del xs
    return dict(us_per_step=us, steps=nsteps)


def parity_sample(res, n_tokens=2048):
    """rho of sampled chains of the last timed prefill output against the oracle
    (first n_tokens of one ordinary head and one decay-stress head)."""
    import oracle
    x, w = res["x"], PREFILL
    out = {}
    for (b, h) in ((0, 3), (3, 29)):
        sl = lambda a: a[b:b + 1, :n_tokens, h:h + 1].contiguous()
        g_ref = oracle.gate(sl(x["z"]), x["A"][h:h + 1])
        o_ref, _ = oracle.forward(sl(x["q"]), sl(x["k"]), sl(x["v"]), g_ref,
                                  x["beta"][b:b + 1, :n_tokens, h:h + 1].contiguous(), None,
                                  col_block=8)
        out[f"rho_o_b{b}h{h}_first{n_tokens}"] = oracle.rho(sl(res["o"]), o_ref)
    return out


def cpu_baseline(chains=8, tokens=4096):
    """The fp64 oracle (as it stands) on a bounded sample of the prefill workload."""
    import oracle
    w = PREFILL
    x = inputs.make_prefill_inputs(1, tokens, chains, w.dk, w.dv, w.dtype, w.seed,
                                   stress_heads_mean=w.stress_heads_mean)
    threads = min(os.cpu_count() or 1, 16)
    t0 = time.perf_counter()
    g = oracle.gate(x["z"], x["A"])
    oracle.forward(x["q"], x["k"], x["v"], g, x["beta"], None, col_block=w.dv // 8,
                   nthreads=threads)
    dt = time.perf_counter() - t0
    head_tokens = chains * tokens
    return {"value": head_tokens / w.H / dt, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"gate + token recurrence in fp64 on {chains} heads x {tokens} tokens "
                      f"of the B4 H32 T32768 d128 workload ({head_tokens} head-tokens, "
                      f"{dt:.1f} s); tokens/s = head-tokens/s / 32 heads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the (batch, head) chains shard across GPUs without communication, so the "
              "per-GPU figure at --gpus 1 is the per-GPU throughput).", file=sys.stderr)
        sys.exit(2)
    _lib.load_library()
    torch.cuda.init()

    res = time_prefill(args.steps, args.warmup)
    w = PREFILL
    work = prefill_work(w)
    ms_per_step = res["wall_s"] * 1e3 / args.steps
    tokens = w.B * w.T
    value = tokens / (ms_per_step / 1e3)
    chunk_s = res["chunk_ms"] / 1e3
    gate_ms = res["gate_ms"]
    chunk_gbs = work["chunk_bytes"] / chunk_s / 1e9
    chunk_tflops = work["chunk_flops"] / chunk_s / 1e12

    dec = time_decode(args.decode_steps)
    dbytes = decode_bytes(DECODE)
    dec_gbs = dbytes / (dec["us_per_step"] * 1e-6) / 1e9

    parity = {} if args.no_parity else parity_sample(res)
    del res
    torch.cuda.empty_cache()
    cpu = None if args.no_cpu_baseline else cpu_baseline()

    line = {
        "metric": "KDA chunkwise prefill tokens/s + decode-step HBM GB/s, % of roofline",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "KDA prefill B4 H32 T32768 d128 bf16, heads 16-31 decay-stress "
                               "(gate + chunked prefill per step); decode 256x32 d128 fp32 state",
                   "global_batch": w.B, "seq_len": w.T, "heads": w.H, "dk": w.dk, "dv": w.dv,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": chunk_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": chunk_gbs / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "chunk_fwd_kernel<bf16,128,64>",
                     "bytes_per_launch": work["chunk_bytes"], "avg_ms": chunk_s * 1e3},
        "prefill": {"gate_ms": gate_ms, "chunk_ms": chunk_s * 1e3,
                    "gate_gbs": work["gate_bytes"] / (gate_ms / 1e3) / 1e9,
                    "chunk_alg_tflops": chunk_tflops,
                    "mfma_frac_of_bf16_peak": chunk_tflops / BF16_PEAK_TFLOPS,
                    "head_tokens": work["head_tokens"]},
        "decode": {"us_per_step": dec["us_per_step"], "steps": dec["steps"],
                   "tokens_per_s": DECODE.B / (dec["us_per_step"] * 1e-6),
                   "roofline": {"bound": "hbm", "achieved": dec_gbs, "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": dec_gbs / HBM_PEAK_GBS, "traffic": None,
                                "kernel": "decode_step_kernel<bf16,128,128>",
                                "bytes_per_launch": dbytes}},
        "parity": parity,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
