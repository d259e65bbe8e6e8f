#!/usr/bin/env python3
"""KDA hot-path benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A timed step is one pass of the prefill hot path over the synthetic batch
B4 H32 T32768 d128 bf16 (heads 16..31 with the gate near its floor):
kda_chunk_fwd_gated (q, k, v, z, A, beta -> o, final state), the gate
evaluated inside the chunk kernel, in the plan the library picks for these
sizes: two segments per sequence, one workgroup per chain, guarded (four
launches of chunk32_kernel: a probe of the second segment's transitions, the
split's first and last phases, and a one-pass launch that returns at once
when every transition vanished in the probe).  The two-kernel form of the same step
(kda_gate z -> g, then kda_chunk_fwd) is timed beside it.  The decode step (256 sequences x H32, d128, fp32 state of 512 MiB
updated in place) is timed in the same run over 1000 consecutive steps with
fresh pre-generated inputs, and reported in the same JSON line.

value        prefill tokens/s (B*T tokens, all 32 heads, per wall-clock step)
roofline     the step's launches (chunk32_kernel with the gate fused) against
             HBM: the algorithm's bytes over the step's time; its arithmetic
             intensity (~96 flop/B) is below the MI355X ridge (~312 flop/B)
cpu_baseline the fp64 oracle timed on this host on a bounded sample of the same
             workload (a reported baseline, not a target)

    python bench.py --ingest-pmc FETCH_DIR WRITE_DIR

reads the counter CSVs of two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE`
runs of this script, scales each kernel's counters by what they read for the
plain 1 GiB device copy the script times, and writes profiles/hbm_traffic_*.md;
later runs report those bytes as `traffic` while the kernel sources still hash
to the recorded values.

    python bench.py --ingest-trace TRACE_DIR

summarises the kernel_trace.csv of a `rocprofv3 --kernel-trace --stats` run of
this script into profiles/kernel_trace_*.md.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from linear_attention_sequence_gate_amd import _lib, inputs  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure
COPY_BYTES = 1 << 30           # calibration copy: 1 GiB read + 1 GiB written

PREFILL = inputs.WORKLOADS["prefill_b4_h32_t32k"]
DECODE = inputs.WORKLOADS["decode_256x32"]

CSRC = os.path.join(ROOT, "linear_attention_sequence_gate_amd", "csrc")
PROFILE_TAG = "prefill_b4h32t32k_decode256x32"
TRAFFIC_MD = os.path.join(ROOT, "profiles", f"hbm_traffic_{PROFILE_TAG}.md")
TRACE_MD = os.path.join(ROOT, "profiles", f"kernel_trace_{PROFILE_TAG}.md")
# kernel -> (name fragments in a profiler trace, sources that define it).  A
# step's launches: every instance of the pipelined kernel with the gate fused
# (one pass, or a split's first and last phases; the split of this workload
# has two segments, so no chaining launch), and the same with g read.
KERNELS = {
    "fused_fwd": (("chunk32_kernel<128, true,", "chunk32_kernelILi128ELb1E"),
                  ("kda_chunk.hip", "kda_device.h")),
    "chunk_fwd": (("chunk32_kernel<128, false,", "chunk32_kernelILi128ELb0E", "chunk_fwd_kernel"),
                  ("kda_chunk.hip", "kda_device.h")),
    "decode_step": (("decode_step_kernel",), ("kda_decode.hip", "kda_device.h")),
    "gate": (("gate_kernel",), ("kda_gate.hip", "kda_device.h")),
}


def _matches(name, frags):
    return any(f in name for f in frags)


def step_groups(named):
    """[(kernel name, value)] of one kernel group in launch order -> the
    launches of each step: a step makes the same sequence of launches (one
    pass; or a guarded split's probe, first phase, last phase and the
    fallback that returns at once), so the least launched instance appears
    once per step."""
    names = {}
    for n, _ in named:
        names[n] = names.get(n, 0) + 1
    steps = min(names.values()) if names else 0
    if steps == 0 or len(named) % steps:
        raise SystemExit(f"launches {len(named)} do not form steps: {names}")
    k = len(named) // steps
    groups = [named[i * k:(i + 1) * k] for i in range(steps)]
    if any([n for n, _ in g] != [n for n, _ in groups[0]] for g in groups):
        raise SystemExit(f"the steps do not launch the same sequence: {names}")
    return groups


def per_step(named):
    """(steps, per-step sums) of step_groups."""
    groups = step_groups(named)
    return len(groups), [sum(v for _, v in g) for g in groups]


def headline_plan():
    """(segments, one workgroup per chain, guarded) the library picks for the step."""
    w = PREFILL
    return _lib.kda_chunk_fwd_plan(w.B, w.T, w.H, w.dk, w.dv, _lib.KDA_BF16, with_guard=True)


def plan_text(P, wide, guarded):
    lay = "one workgroup per chain" if wide else "64-column slices"
    if P < 2:
        return f"one pass, {lay}"
    if guarded:
        return (f"{P} segments per sequence, {lay}, guarded: a probe of the second segment's "
                "transitions, the split's two phases, and a one-pass launch in 64-column slices "
                "that runs only if some transition had not vanished (it returns at once here)")
    return f"{P} segments per sequence, {lay}"


def headline_main_instance():
    """Name fragments of the step's dominant launch (the split's first phase,
    or the one pass), its v workgroups and their 32-token periods each."""
    w = PREFILL
    P, wide, guarded = _lib.kda_chunk_fwd_plan(w.B, w.T, w.H, w.dk, w.dv, _lib.KDA_BF16, with_guard=True)
    tr = P >= 2 and not guarded        # a guarded split's first phase runs without transitions
    frag = (f"chunk32_kernel<128, true, {str(tr).lower()}, {str(wide).lower()}>",
            f"chunk32_kernelILi128ELb1ELb{int(tr)}ELb{int(wide)}E")
    per = -(-w.T // P)
    seg_len = -(-per // 32) * 32
    wgs = w.B * w.H * (w.dv // (128 if wide else 64)) * P
    return frag, wgs, seg_len // 32 + 2

# UT inverse of one 64-token chunk, per head-token (block substitution over
# 16x16 blocks; the same constant as the flop model of the scope table).
INV_FLOPS_PER_HT = 2218
# the same count for 32-token chunks: the substitution's work per chunk grows
# as the cube of the chunk length, per token as its square, so a quarter
INV_FLOPS_PER_HT_C32 = 554


def prefill_work(w, B=None, T=None, H=None):
    """Algorithmic bytes and flops of one kda_chunk_fwd call (and of the gate,
    and of the fused call kda_chunk_fwd_gated).

    Bytes: q, k, v, beta and o once in the input dtype, g once in fp32, the
    final state (and the initial one when given) in fp32.  The fused call reads
    z in the input dtype instead of g, and the [H, dk] table A.
    Flops per head-token of the benchmarked kernel (C = 32-token chunks of two
    dense 16-token subtiles, mean causal length Lbar = (32 + 16) / 2 = 24):
    6 dk dv for K~ S, Q~ S and K^T U; 2 Lbar dk each for A and P; 2 Lbar dv
    each for T (V - K~ S) and P U (W = T K~ is never formed); the UT inverse.
    The scope table's count for 64-token chunks (Lbar = 40, with W) is
    reported beside it."""
    B, T, H = B or w.B, T or w.T, H or w.H
    dk, dv = w.dk, w.dv
    e = 2 if w.dtype == torch.bfloat16 else 4
    ht = B * T * H                                   # head-tokens
    chunk_bytes = ht * ((2 * dk + dv) * e + dk * 4 + e + dv * e)
    chunk_bytes += B * H * dk * dv * 4 * (2 if w.s0_std > 0 else 1)
    lbar32, lbar64 = (32 + 16) / 2, (64 + 16) / 2
    flops_per_ht = 6 * dk * dv + 2 * lbar32 * (2 * dk + 2 * dv) + INV_FLOPS_PER_HT_C32
    flops_c64 = 6 * dk * dv + 2 * lbar64 * (3 * dk + 2 * dv) + INV_FLOPS_PER_HT
    gate_bytes = ht * dk * (e + 4)
    fused_bytes = chunk_bytes - ht * dk * (4 - e) + H * dk * 4
    return dict(head_tokens=ht, chunk_bytes=chunk_bytes, chunk_flops=flops_per_ht * ht,
                flops_per_head_token=flops_per_ht, flops_per_head_token_c64=flops_c64,
                gate_bytes=gate_bytes, fused_bytes=fused_bytes)


def decode_bytes(w):
    """State read + written once, q/k/v/z/beta read, o written, A read."""
    N, H, dk, dv = w.B, w.H, w.dk, w.dv
    e = 2
    return N * H * (2 * dk * dv * 4 + (3 * dk + dv) * e + e + dv * e) + H * dk * 4


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """Per-launch HBM bytes from the recorded counter summary for kernels whose
    sources are unchanged since the counters were taken (else None)."""
    out = {k: None for k in KERNELS}
    try:
        text = open(TRAFFIC_MD).read()
    except OSError:
        return out
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return out
    rec = json.loads(m.group(1))
    for k, (_, srcs) in KERNELS.items():
        r = rec.get("kernels", {}).get(k)
        if r and r.get("source_sha256") == source_hash(srcs):
            out[k] = r["traffic_bytes"]
    return out


def time_copy(reps=5):
    """Plain device copy of 1 GiB (the HBM calibration kernel for the counters)."""
    src = torch.empty(COPY_BYTES // 4, device="cuda", dtype=torch.float32).normal_()
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) / 1e3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * COPY_BYTES / s / 1e9


def time_prefill(steps, warmup):
    """The timed step, kda_chunk_fwd_gated: one launch of the chunk kernel with
    the gate fused (HIP events around each launch on its stream)."""
    w = PREFILL
    dev = torch.device("cuda")
    x = inputs.workload_prefill_inputs(w, device=dev)
    o = torch.empty(w.B, w.T, w.H, w.dv, device=dev, dtype=w.dtype)
    ST = torch.empty(w.B, w.H, w.dk, w.dv, device=dev, dtype=torch.float32)
    ws = torch.empty(max(_lib.kda_chunk_fwd_gated_workspace_size(w.B, w.T, w.H, w.dk, w.dv, 1), 256),
                     device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream()     # the kernel is launched on it

    def step(evs=None):
        if evs: evs[0].record(stream)
        _lib.kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"], x["S0"],
                                 final_state=ST, o=o, workspace=ws, stream=stream)
        if evs: evs[1].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fused_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    return dict(x=x, o=o, ST=ST, wall_s=wall, fused_ms=fused_ms)


def time_two_kernel(x, steps, warmup=2):
    """The same step as two launches, kda_gate (z -> g in HBM) then
    kda_chunk_fwd, each bracketed by HIP events on the launch stream."""
    w = PREFILL
    dev = torch.device("cuda")
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
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    gate_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    chunk_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    del g, o, ST
    torch.cuda.empty_cache()
    return dict(gate_ms=gate_ms, chunk_ms=chunk_ms)


def time_prefill_plans(reps=10, warmup=5):
    """The step's sizes in other plans, each call bracketed by HIP events:
    one pass in 64-column slices (what the library ran before it weighed one
    workgroup per chain; independent of the gates), and the library's plan and
    that one pass with gates that keep memory (z - 12 everywhere: no
    transition vanishes, so the split's last phase reruns whole segments and
    its transitions run whole after the segments' workgroups)."""
    w = PREFILL
    dev = torch.device("cuda")
    x = inputs.workload_prefill_inputs(w, device=dev)
    o = torch.empty(w.B, w.T, w.H, w.dv, device=dev, dtype=w.dtype)
    ST = torch.empty(w.B, w.H, w.dk, w.dv, device=dev, dtype=torch.float32)
    ws = torch.empty(max(_lib.kda_chunk_fwd_gated_workspace_size(w.B, w.T, w.H, w.dk, w.dv, 1), 256),
                     device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream()
    one = _lib.KDA_FLAG_WORKGROUP_PER_SLICE | _lib.kda_flag_segments(1)

    def timed(z, flags):
        run = lambda: _lib.kda_chunk_fwd_gated(x["q"], x["k"], x["v"], z, x["A"], x["beta"], x["S0"],
                                               final_state=ST, o=o, workspace=ws, flags=flags,
                                               stream=stream)
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    P, wide, guarded = headline_plan()
    out = {"one_pass_slices_ms": timed(x["z"], one)}
    zk = (x["z"].float() - 12.0).to(x["z"].dtype)
    out["gates_keep_memory"] = {"plan_ms": timed(zk, 0), "one_pass_slices_ms": timed(zk, one),
                                "inputs": "z - 12 everywhere (g about -3e-5 per token)"}
    out["plan"] = {"segments": P, "workgroup_per_chain": wide, "guarded": guarded}
    del x, o, ST, ws, zk
    torch.cuda.empty_cache()
    return out


LONG = inputs.WORKLOADS["prefill_h32_t1m"]


def time_long_prefill(reps=3):
    """kda_chunk_fwd_gated (gate and chunked prefill, as the main step) on the
    few-chain long workload (B1 H32 T1M: 64 workgroups in one pass) in one
    pass, with the library's sequence split, and with the split whose last
    phase reruns whole segments (KDA_FLAG_SPLIT_FULL_RERUN), in that order."""
    w = LONG
    dev = torch.device("cuda")
    x = inputs.workload_prefill_inputs(w, device=dev)
    o = torch.empty(w.B, w.T, w.H, w.dv, device=dev, dtype=w.dtype)
    ST = torch.empty(w.B, w.H, w.dk, w.dv, device=dev, dtype=torch.float32)
    nseg = _lib.kda_chunk_fwd_auto_segments(w.B, w.T, w.H, w.dk, w.dv, 1)
    ws = torch.empty(_lib.kda_chunk_fwd_gated_workspace_size(w.B, w.T, w.H, w.dk, w.dv, 1),
                     device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream()
    out = {}
    for label, fl in (("one_pass", _lib.kda_flag_segments(1)), ("split", 0),
                      ("split_full_rerun", _lib.KDA_FLAG_SPLIT_FULL_RERUN)):
        def run():
            _lib.kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"], x["S0"],
                                     final_state=ST, o=o, workspace=ws, flags=fl, stream=stream)
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        out[label + "_ms"] = e0.elapsed_time(e1) / reps
    work = prefill_work(w)
    s_ = out["split_ms"] / 1e3
    plan = _lib.kda_chunk_fwd_plan(w.B, w.T, w.H, w.dk, w.dv, 1)
    plan_rr = _lib.kda_chunk_fwd_plan(w.B, w.T, w.H, w.dk, w.dv, 1, _lib.KDA_FLAG_SPLIT_FULL_RERUN)
    out.update(segments=nseg, workgroup_per_chain=plan[1],
               full_rerun_plan={"segments": plan_rr[0], "workgroup_per_chain": plan_rr[1]},
               speedup=out["one_pass_ms"] / out["split_ms"],
               tokens_per_s=w.B * w.T / s_,
               hbm_frac_of_roofline=work["fused_bytes"] / s_ / 1e9 / HBM_PEAK_GBS,
               workload=w.note + "; gate fused (kda_chunk_fwd_gated)")
    del x, o, ST, ws
    torch.cuda.empty_cache()
    return out


SMALL = inputs.WORKLOADS["prefill_h8_t4k"]


def time_small_prefill(reps=20, copies=5, warmup=10, windows=5):
    """kda_chunk_fwd_gated on the few-chain short workload (B1 H8 T4096 d128
    bf16: 8 chains, 16 workgroups in one pass), with the segment count the
    library picks.  Its 56 MiB of inputs and outputs would stay in the 256 MB
    last-level cache across repetitions, so the calls rotate over `copies`
    independent sets of inputs and outputs.  A call takes about 60 us, little
    more than the host needs to issue it, so a pause of the host thread
    leaves the GPU idle inside a timed window: the median of `windows`
    windows of `reps` calls is reported."""
    w = SMALL
    dev = torch.device("cuda")
    xs = [inputs.make_prefill_inputs(w.B, w.T, w.H, w.dk, w.dv, w.dtype, w.seed + 97 * i,
                                     device=dev, s0_std=w.s0_std,
                                     stress_heads_mean=w.stress_heads_mean)
          for i in range(copies)]
    os_ = [torch.empty(w.B, w.T, w.H, w.dv, device=dev, dtype=w.dtype) for _ in range(copies)]
    Ss = [torch.empty(w.B, w.H, w.dk, w.dv, device=dev, dtype=torch.float32) for _ in range(copies)]
    nseg = _lib.kda_chunk_fwd_auto_segments(w.B, w.T, w.H, w.dk, w.dv, 1)
    ws = torch.empty(max(_lib.kda_chunk_fwd_gated_workspace_size(w.B, w.T, w.H, w.dk, w.dv, 1), 256),
                     device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream()

    def run(i):
        x = xs[i % copies]
        _lib.kda_chunk_fwd_gated(x["q"], x["k"], x["v"], x["z"], x["A"], x["beta"], x["S0"],
                                 final_state=Ss[i % copies], o=os_[i % copies], workspace=ws,
                                 stream=stream)

    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    per_window = []
    for _ in range(windows):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            run(i)
        e1.record(stream)
        torch.cuda.synchronize()
        per_window.append(e0.elapsed_time(e1) / reps)
    ms = sorted(per_window)[windows // 2]
    work = prefill_work(w)
    s_ = ms / 1e3
    out = {"ms": ms, "ms_windows": per_window, "segments": nseg, "tokens_per_s": w.B * w.T / s_,
           "head_tokens_per_s": work["head_tokens"] / s_,
           "hbm_frac_of_roofline": work["fused_bytes"] / s_ / 1e9 / HBM_PEAK_GBS,
           "bytes_per_call": work["fused_bytes"],
           "workload": w.note + "; gate fused (kda_chunk_fwd_gated); inputs rotated over "
                                f"{copies} copies"}
    del xs, os_, Ss, ws
    torch.cuda.empty_cache()
    return out


def time_pairwise_diagonal(reps=5):
    """kda_chunk_fwd on the benchmark's prefill workload with the dense MFMA
    diagonal tiles (what the gate floor allows) and with the position-pair
    diagonal path the floor made unnecessary, in the same kernel."""
    w = PREFILL
    dev = torch.device("cuda")
    x = inputs.workload_prefill_inputs(w, device=dev)
    g = _lib.kda_gate(x["z"], x["A"])
    o = torch.empty(w.B, w.T, w.H, w.dv, device=dev, dtype=w.dtype)
    ST = torch.empty(w.B, w.H, w.dk, w.dv, device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream()
    out = {}
    # the same plan for both: one pass of 64-column slices (the position-pair
    # path's layout)
    for label, fl in (("dense_ms", _lib.KDA_FLAG_WORKGROUP_PER_SLICE),
                      ("pairwise_ms", _lib.KDA_FLAG_PAIRWISE_DIAGONAL)):
        def run():
            _lib.kda_chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], x["S0"], final_state=ST, o=o,
                               flags=fl, stream=stream)
        for _ in range(5):         # past the first launches' clock ramp
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        out[label] = e0.elapsed_time(e1) / reps
    out.update(pairwise_over_dense=out["pairwise_ms"] / out["dense_ms"],
               workload=w.note.split(";")[0])
    del x, g, o, ST
    torch.cuda.empty_cache()
    return out


FP32_PEAK_TFLOPS = 157.3      # MI355X fp32 (matrix and vector), vendor figure
BWD_CHUNK = 16
# chunked reverse mode, flops per head-token with every product counted once
# (C = 16-token chunks, d = dk = dv):
#   d^2 terms: forward state pass K~S, K^T U (4); reverse pass K^ dN, Q~^T dO,
#              K~^T dW (6); dQ~ = dO S^T, dK~ = dW S^T, dK^ = U dN^T (6)
#   C d terms: At, P (4); U, dU's P^T dO, dW (6); dT, dP (4); pair terms dQ',
#              dK', dK" (two) (8)
def bwd_chunk_flops(d):
    return 16 * d * d + 22 * BWD_CHUNK * d


def time_backward(reps=5):
    """kda_chunk_bwd on B4 H32 T32768 d128 bf16 (the prefill workload's
    chains and length; heads 16-31 decay-stress), chunked path: with the
    whole-sequence workspace (one segment) and with a workspace for
    4096-token segments (the forward state pass then runs twice); the
    token-level path and the gate's reverse mode timed beside it."""
    B, T, H, d = 4, 32768, 32, 128
    seg = 4096
    dev = torch.device("cuda")
    x = inputs.make_prefill_inputs(B, T, H, d, d, torch.bfloat16, 4242, device=dev, s0_std=0.02,
                                   stress_heads_mean=3.0)
    g = _lib.kda_gate(x["z"], x["A"])
    d_o = torch.randn(B, T, H, d, device=dev).to(torch.bfloat16)
    ws_whole = _lib.kda_chunk_bwd_workspace_size_flags(B, T, H, d, d, 1, 0, 0)
    ws_seg = _lib.kda_chunk_bwd_workspace_size_flags(B, T, H, d, d, 1, 0, seg)
    ws = torch.empty(ws_whole, device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream()

    def timed(flags, n, warm, nbytes):
        wsv = ws[:nbytes]
        run = lambda: _lib.kda_chunk_bwd(x["q"], x["k"], x["v"], g, x["beta"], x["S0"], d_o, None,
                                         workspace=wsv, flags=flags, stream=stream)
        for _ in range(warm):      # past the first launches' clock ramp
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms = timed(0, reps, 3, ws_whole)
    ms_seg = timed(0, reps, 2, ws_seg)
    del ws
    torch.cuda.empty_cache()
    tok_bytes = _lib.kda_chunk_bwd_workspace_size_flags(B, T, H, d, d, 1, _lib.KDA_FLAG_TOKEN_BACKWARD, 0)
    ws = torch.empty(tok_bytes, device=dev, dtype=torch.uint8)
    ms_token = timed(_lib.KDA_FLAG_TOKEN_BACKWARD, 1, 1, tok_bytes)
    del ws
    torch.cuda.empty_cache()
    # the gate's reverse mode on the same rows (dz, dA from a dg of that shape)
    dg = torch.randn(B, T, H, d, device=dev)
    gws = torch.empty(max(_lib.kda_gate_bwd_workspace_size(B, T, H, d), 256), device=dev,
                      dtype=torch.uint8)
    for _ in range(3):
        _lib.kda_gate_bwd(x["z"], x["A"], dg, workspace=gws, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        _lib.kda_gate_bwd(x["z"], x["A"], dg, workspace=gws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    gate_ms = e0.elapsed_time(e1) / reps
    gate_bytes = B * T * H * d * (2 + 4 + 4)             # z (bf16), dg, dz
    del dg, gws
    ht = B * T * H
    tflops = bwd_chunk_flops(d) * ht / (ms / 1e3) / 1e12
    del x, g, d_o
    torch.cuda.empty_cache()
    return {"ms": ms, "workload": f"B{B} H{H} T{T} d{d} bf16, heads 16-31 decay-stress (gradients fp32)",
            "head_tokens_per_s": ht / (ms / 1e3), "workspace_bytes": ws_whole,
            "segmented": {"segment_tokens": seg, "ms": ms_seg, "workspace_bytes": ws_seg,
                          "over_one_segment": ms_seg / ms},
            "token_path_ms": ms_token,
            "gate_bwd_ms": gate_ms, "gate_bwd_gbs": gate_bytes / (gate_ms / 1e3) / 1e9,
            "roofline": {"bound": "mfma", "achieved": tflops, "peak": FP32_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": tflops / FP32_PEAK_TFLOPS,
                         "flops_per_head_token": bwd_chunk_flops(d),
                         "scope": "whole call (four launches), fp32 matrix-core peak"}}


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
    x = res["x"]
    out = {}
    for (b, h) in ((0, 3), (3, 29)):
        sl = lambda a: a[b:b + 1, :n_tokens, h:h + 1].contiguous()
        g_ref = oracle.gate(sl(x["z"]), x["A"][h:h + 1])
        o_ref, _ = oracle.forward(sl(x["q"]), sl(x["k"]), sl(x["v"]), g_ref,
                                  x["beta"][b:b + 1, :n_tokens, h:h + 1].contiguous(), None,
                                  col_block=8)
        out[f"rho_o_b{b}h{h}_first{n_tokens}"] = oracle.rho(sl(res["o"]), o_ref)
    return out


def cpu_baseline(x, budget_s=15.0, window=4096):
    """The fp64 oracle (as it stands: gate, then the token recurrence with o) on
    the workload's own inputs, all B*H chains, over successive token windows
    (each window starts from the state the previous one ended in), until about
    budget_s seconds of oracle time are spent.  Host copies are made outside
    the timed region."""
    import oracle
    w = PREFILL
    threads = min(os.cpu_count() or 1, 16)
    A = x["A"].double().cpu()
    S, spent, done, t_end = None, 0.0, 0, 0
    for t0 in range(0, w.T, window):
        sl = slice(t0, min(t0 + window, w.T))
        h64 = {n: x[n][:, sl].double().cpu().numpy() for n in ("q", "k", "v", "z", "beta")}
        t = time.perf_counter()
        g = oracle.gate(h64["z"], A)
        _, S = oracle.forward(h64["q"], h64["k"], h64["v"], g, h64["beta"], S,
                              col_block=w.dv // 8, nthreads=threads)
        spent += time.perf_counter() - t
        done += w.B * w.H * (sl.stop - sl.start)
        t_end = sl.stop
        del h64, g
        if spent >= budget_s:
            break
    return {"value": done / spent / w.H, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 gate + token recurrence (with outputs) over tokens 0..{t_end} of all "
                      f"{w.B * w.H} chains of B4 H32 T32768 d128 ({done} head-tokens, "
                      f"{spent:.1f} s on {threads} threads); tokens/s = head-tokens/s / 32"}


# ---------------------------------------------------------------------------
# counter ingestion (CPU only)
# ---------------------------------------------------------------------------
def _pmc_rows(d, counter):
    """(kernel name, value) per dispatch from a rocprofv3 counter_collection.csv."""
    rows = []
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") != counter:
                    continue
                key = (f, r.get("Dispatch_Id", r.get("Correlation_Id")))
                rows.append((key, r["Kernel_Name"], float(r["Counter_Value"])))
    # sum the per-instance values of one dispatch; dispatches in launch order
    agg = {}
    for key, name, val in rows:
        n, v = agg.get(key, (name, 0.0))
        agg[key] = (n, v + val)

    def order(key):
        try:
            return (key[0], int(key[1]))
        except (TypeError, ValueError):
            return (key[0], 0)
    return [agg[k] for k in sorted(agg, key=order)]


def ingest_pmc(fetch_dir, write_dir):
    cal = {}
    per = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _pmc_rows(d, counter)                 # values in KiB
        # the 1 GiB device-to-device copies are the runtime's largest copyBuffer
        # dispatches in the run
        cb = [v * 1024 for n, v in rows if "copyBuffer" in n]
        copies = [v for v in cb if v >= 0.9 * max(cb, default=0.0)]
        if not copies or max(copies) < 0.25 * COPY_BYTES:
            raise SystemExit(f"{counter}: no 1 GiB copy dispatch found in {d}")
        cal[counter] = COPY_BYTES / (sum(copies) / len(copies))
        for k, (frag, _) in KERNELS.items():
            named = [(n, v * 1024) for n, v in rows if _matches(n, frag)]
            if named:
                steps, sums = per_step(named)
                per.setdefault(k, {})[counter] = (sum(sums) / steps, steps)
    rec = {"copy_factor": {"fetch": cal["FETCH_SIZE"], "write": cal["WRITE_SIZE"]}, "kernels": {}}
    for k, (_, srcs) in KERNELS.items():
        if k not in per or len(per[k]) < 2:
            continue
        f = per[k]["FETCH_SIZE"][0] * cal["FETCH_SIZE"]
        wb = per[k]["WRITE_SIZE"][0] * cal["WRITE_SIZE"]
        rec["kernels"][k] = {"fetch_bytes": round(f), "write_bytes": round(wb),
                             "traffic_bytes": round(f + wb),
                             "dispatches": per[k]["FETCH_SIZE"][1],
                             "source_sha256": source_hash(srcs)}
    w = PREFILL
    work = prefill_work(w)
    alg = {"fused_fwd": work["fused_bytes"], "chunk_fwd": work["chunk_bytes"],
           "decode_step": decode_bytes(DECODE), "gate": work["gate_bytes"]}
    P, wide, guarded = headline_plan()
    lines = ["# HBM traffic per step (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
             "Workloads: prefill B4 H32 T32768 d128 bf16 (the fused step, then gate + chunk),",
             f"decode 256x32 d128.  The prefill steps run the library's plan ({plan_text(P, wide, guarded)});",
             "a step's figure sums its launches of the kernel.",
             "Each counter is scaled by the factor that maps its reading for a plain",
             "1 GiB device copy (torch `copy_` -> the runtime's copyBuffer kernel, timed",
             "in the same script) to 1 GiB.", "",
             "Commands (from the repository root):", "",
             "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -- "
             "python3 -u bench.py --steps 2 --warmup 1 --decode-steps 20 --no-cpu-baseline --no-parity --no-extras",
             "    rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -- "
             "python3 -u bench.py --steps 2 --warmup 1 --decode-steps 20 --no-cpu-baseline --no-parity --no-extras",
             "    python3 bench.py --ingest-pmc gpurun_out/pmc_fetch gpurun_out/pmc_write", "",
             f"Copy factors: FETCH {cal['FETCH_SIZE']:.4f}, WRITE {cal['WRITE_SIZE']:.4f}", "",
             "| kernel (per step) | fetch (MB) | write (MB) | traffic (MB) | algorithmic (MB) | traffic / algorithmic |",
             "|---|---|---|---|---|---|"]
    for k, r in rec["kernels"].items():
        lines.append(f"| {KERNELS[k][0][0]} | {r['fetch_bytes'] / 1e6:.1f} | {r['write_bytes'] / 1e6:.1f} "
                     f"| {r['traffic_bytes'] / 1e6:.1f} | {alg[k] / 1e6:.1f} "
                     f"| {r['traffic_bytes'] / alg[k]:.3f} |")
    lines += ["", "Machine-readable record (read by bench.py; a kernel's entry is used only",
              "while its sources hash to `source_sha256`):", "", "```json",
              json.dumps(rec, indent=1), "```", ""]
    os.makedirs(os.path.dirname(TRAFFIC_MD), exist_ok=True)
    with open(TRAFFIC_MD, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


TRACE_STEPS, TRACE_WARMUP, TRACE_DECODE = 20, 20, 200
TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/ktrace -o bench -- "
             f"python3 -u bench.py --steps {TRACE_STEPS} --warmup {TRACE_WARMUP} "
             f"--decode-steps {TRACE_DECODE} --no-cpu-baseline --no-parity --no-extras")
EXTRA_TRACES = {
    # name: (bench.py --only value, profile file, what the run holds)
    "long": ("long", "kernel_trace_prefill_b1h32t1m_split.md",
             "kda_chunk_fwd_gated (the gate fused into the chunk kernel) on B1 H32 T1048576 "
             "d128 bf16 in one pass (64-column slices; 1 warm-up + 3 timed calls), with the "
             "library's sequence split (the same; P = 8, one workgroup per chain), and with "
             "KDA_FLAG_SPLIT_FULL_RERUN (the same; P = 9, one workgroup per chain). The stopping "
             "split's segment workgroups fill the GPU, so its transitions run first in a launch of "
             "their own (64-column slices); otherwise a split call "
             "is three launches: chunk32_kernel phase 1 (the segments "
             "from their start states, the transitions of segments 1..P-1; the full rerun "
             "leaves the last segment out), seg_chain_kernel, and chunk32_kernel phase 3 "
             "(segments 1..P-1: up to where their transitions vanished, or whole with the "
             "full rerun); the mode and the workgroup count tell the launches apart."),
    "backward": ("backward", "kernel_trace_backward_b4h32t32k.md",
                 "kda_gate once, then kda_chunk_bwd on B4 H32 T32768 d128 bf16 (heads 16-31 "
                 "decay-stress): the chunked path with the whole-sequence workspace (3 warm-up + 5 "
                 "timed calls; per call cb_prep_kernel (X, P, At per 16-token chunk), cb_fwd_kernel "
                 "(state entering each even chunk), cb_bwd_kernel (gradient leaving each odd chunk) "
                 "and cb_grad_kernel (token gradients, one workgroup per chunk pair)); the same "
                 "with a workspace for 4096-token segments (2 + 5 calls; per call a forward sweep of "
                 "cb_prep_kernel and cb_fwd_kernel over segments 0..6, then the four kernels per "
                 "segment in reverse; rows labelled by the call their prep launch belongs to); "
                 "then the token-level path (1 warm-up + 1 timed call; "
                 "bwd_ckpt_kernel, bwd_kernel, bwd_sum_kernel) and kda_gate_bwd."),
    "small": ("small", "kernel_trace_prefill_b1h8t4096_split.md",
              "kda_chunk_fwd_gated on B1 H8 T4096 d128 bf16 with the library's automatic "
              "sequence split (10 segments of 416 tokens), inputs rotated over five copies (10 "
              "warm-up + 5 windows of 20 timed calls).  A call is three launches: chunk32_kernel phase 1 "
              "(segment 0 from the initial state, segments 1..9 from zero, and their "
              "transitions), seg_chain_kernel (serial chaining), chunk32_kernel phase 3 "
              "(segments 1..9 up to where their transitions vanished); the workgroup count "
              "tells the phases apart."),
    "pairwise": ("pairwise", "kernel_trace_prefill_b4h32t32k_pairwise_diagonal.md",
                 "kda_gate once, then kda_chunk_fwd on B4 H32 T32768 d128 bf16 in one pass of "
                 "64-column slices (the position-pair path's plan) with the dense "
                 "MFMA diagonal tiles (5 warm-up + 5 timed calls) and with the position-pair "
                 "diagonal path (the same), in that order."),
}


def extra_trace_cmd(name):
    return (f"rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/ktrace_{name} "
            f"-o {name} -- python3 -u bench.py --only {EXTRA_TRACES[name][0]}")


def ingest_trace(d):
    """Summarise the kernel trace of TRACE_CMD.  Per kernel: every call, and
    the calls the benchmark times (the last `steps` launches, after the
    warm-up whose first launches run while the clocks ramp).  The fused
    kernel's HBM fraction is computed from the timed calls, as bench.py's
    `roofline` is."""
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {d}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    P, wide, guarded = headline_plan()
    lines = ["# Kernel durations (rocprofv3 kernel trace)", "",
             f"Workloads: prefill B4 H32 T32768 d128 bf16 (the fused step: {TRACE_WARMUP} warm-up "
             f"and {TRACE_STEPS} timed steps; then gate + chunk as two kernels: 2 warm-up and "
             f"{TRACE_STEPS} timed steps), decode 256x32 d128 (20 warm-up + {TRACE_DECODE} steps), "
             "plus the 1 GiB calibration copy.  The prefill steps run the library's plan for "
             f"these sizes: {plan_text(P, wide, guarded)}.  Durations from the trace's start/end timestamps; "
             "'timed' is the last steps, the ones the benchmark times, and a step's time sums "
             "its launches.", "",
             "Command (from the repository root):", "", "    " + TRACE_CMD,
             "    python3 bench.py --ingest-trace gpurun_out/ktrace", "",
             "| kernel | launches | steps | avg per step (us) | min (us) | max (us) | timed steps | "
             "timed avg per step (us) |",
             "|---|---|---|---|---|---|---|---|"]
    frags = dict((k, v[0]) for k, v in KERNELS.items())
    frags["copy (calibration)"] = ("copyBuffer",)
    timed_n = {"fused_fwd": TRACE_STEPS, "chunk_fwd": TRACE_STEPS, "gate": TRACE_STEPS,
               "decode_step": TRACE_DECODE}
    rec = {}
    inst = []
    for label, frag in frags.items():
        named = [(r["Kernel_Name"], (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
                 for r in rows if _matches(r["Kernel_Name"], frag)]
        if not named:
            continue
        steps, us = per_step(named)
        k = len(named) // steps
        n = min(timed_n.get(label, steps), steps)
        timed = us[-n:]
        rec[label] = sum(timed) / len(timed)
        lines.append(f"| {label}: {k} instance(s) | {len(named)} | {steps} | {sum(us) / steps:.1f} "
                     f"| {min(us):.1f} | {max(us):.1f} | {n} | {rec[label]:.1f} |")
        groups = step_groups(named)[-n:]
        for j in range(k):
            t = [g[j][1] for g in groups]
            inst.append(f"| {label} | {j + 1} of {k} | `{groups[0][j][0].split('(')[0][:70]}` | "
                        f"{len(t)} | {sum(t) / len(t):.1f} |")
    lines += ["", "Launches of a step, over the timed steps:", "",
              "| kernel | launch | instance | timed launches | avg (us) |", "|---|---|---|---|---|"] + inst
    if "fused_fwd" in rec:
        fb = prefill_work(PREFILL)["fused_bytes"]
        frac = fb / (rec["fused_fwd"] * 1e-6) / 1e9 / HBM_PEAK_GBS
        lines += ["", f"Fused step, timed steps: {fb} algorithmic bytes per step / "
                      f"{rec['fused_fwd']:.1f} us = {fb / (rec['fused_fwd'] * 1e-6) / 1e9:.0f} GB/s, "
                      f"{frac:.4f} of 8 TB/s."]
    if "decode_step" in rec:
        db = decode_bytes(DECODE)
        lines += ["", f"Decode, timed launches: {db} bytes per step / {rec['decode_step']:.1f} us = "
                      f"{db / (rec['decode_step'] * 1e-6) / 1e9:.0f} GB/s, "
                      f"{db / (rec['decode_step'] * 1e-6) / 1e9 / HBM_PEAK_GBS:.4f} of 8 TB/s."]
    lines.append("")
    os.makedirs(os.path.dirname(TRACE_MD), exist_ok=True)
    with open(TRACE_MD, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def ingest_trace_extra(name, d):
    """Kernel durations of one extra run (bench.py --only NAME).  chunk32_kernel
    launches are grouped by workgroup count, and in the position-pair run by
    mode (its first half of launches is the dense path, the second the
    position-pair path)."""
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {d}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    rows = [r for r in rows if _matches(r["Kernel_Name"], ("chunk32_kernel", "seg_chain_kernel",
                                                           "seg_scan_kernel", "seg_apply_kernel",
                                                           "gate_kernel",
                                                           "bwd_ckpt_kernel", "bwd_kernel", "bwd_sum_kernel",
                                                           "cb_prep_kernel", "cb_fwd_kernel", "cb_bwd_kernel",
                                                           "cb_grad_kernel"))]
    chunk_rows = [r for r in rows if "chunk32_kernel" in r["Kernel_Name"]]
    groups = {}
    prep_wgs = None
    for r in rows:
        kname = r["Kernel_Name"].split("(")[0].replace("void ", "")[:40]
        wgs = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
        label = ""
        if name == "pairwise" and r in chunk_rows:
            label = "dense" if chunk_rows.index(r) < len(chunk_rows) // 2 else "position pairs"
        if name == "long":
            # one pass first (the first launch's grid), then the stopping
            # split's calls, then the full rerun's, whose first phase is the
            # only launch of the per-chain instance with transition columns
            first = int(chunk_rows[0]["Grid_Size_X"])
            split_rows = [x for x in rows if int(x["Grid_Size_X"]) != first
                          or "chunk32_kernel" not in x["Kernel_Name"]]
            rr = next((i for i, x in enumerate(split_rows)
                       if "chunk32_kernel<128, true, true, true>" in x["Kernel_Name"]), len(split_rows))
            if r not in split_rows:
                label = "one pass"
            else:
                label = "stopping split" if split_rows.index(r) < rr else "full rerun"
        if name == "backward" and "cb_" in kname:
            # the chunked path's launches belong to the call (whole sequence or
            # one segment) whose prep launch, with one workgroup per chunk,
            # precedes them
            if "cb_prep" in kname:
                prep_wgs = wgs
            label = "whole sequence" if prep_wgs == max(
                int(x["Grid_Size_X"]) // max(1, int(x["Workgroup_Size_X"]))
                for x in rows if "cb_prep" in x["Kernel_Name"]) else "segment"
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups.setdefault((kname, label, wgs), []).append(us)
    only, fname, what = EXTRA_TRACES[name]
    lines = [f"# Kernel durations, `bench.py --only {only}` (rocprofv3 kernel trace)", "",
             what, "", "Command (from the repository root):", "", "    " + extra_trace_cmd(name),
             f"    python3 bench.py --ingest-trace-extra {name} gpurun_out/ktrace_{name}", "",
             "| kernel | mode | workgroups | calls | avg (ms) | min (ms) | max (ms) |",
             "|---|---|---|---|---|---|---|"]
    for (kname, label, wgs), us in groups.items():
        lines.append(f"| `{kname}` | {label} | {wgs} | {len(us)} | {sum(us) / len(us) / 1e3:.3f} "
                     f"| {min(us) / 1e3:.3f} | {max(us) / 1e3:.3f} |")
    lines.append("")
    with open(os.path.join(ROOT, "profiles", fname), "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


SQ_PASSES = (
    "SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_LDS SQ_ACTIVE_INST_VALU "
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_ANY",
    "SQ_LDS_BANK_CONFLICT SQ_LDS_ADDR_CONFLICT SQ_WAIT_INST_LDS SQ_WAIT_ANY SQ_ACTIVE_INST_LDS "
    "SQ_ACTIVE_INST_SCA SQ_ACTIVE_INST_VMEM SQ_INST_LEVEL_LDS",
)
SQ_MD = os.path.join(ROOT, "profiles", "sq_counters_chunk32_b4h32t32k.md")
N_SE, N_SIMD = 32, 1024        # MI355X: 8 XCDs x 4 shader engines; 256 CUs x 4 SIMDs


def recorded_sq():
    """The fused kernel's recorded SQ figures (MFMA busy, VALU active and their
    sum, the issue share), while its sources are unchanged since they were
    taken (else an empty dict)."""
    try:
        text = open(SQ_MD).read()
    except OSError:
        return {}
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return {}
    rec = json.loads(m.group(1))
    if rec.get("source_sha256") != source_hash(KERNELS["fused_fwd"][1]):
        return {}
    return rec


def recorded_mfma_busy():
    return recorded_sq().get("mfma_busy_frac")


SQ_STEPS, SQ_WARMUP = 5, 20


def sq_cmd(i):
    return (f"rocprofv3 --pmc {SQ_PASSES[i]} --output-format csv -d gpurun_out/sq{i} -- "
            f"python3 -u bench.py --steps {SQ_STEPS} --warmup {SQ_WARMUP} --decode-steps 20 "
            "--no-cpu-baseline --no-parity --no-extras")


BWD_COUNTERS_MD = os.path.join(ROOT, "profiles", "counters_backward_b4h32t32k.md")
BWD_PMC_PASSES = SQ_PASSES + ("FETCH_SIZE", "WRITE_SIZE")
BWD_LAUNCHES = (("prep", "cb_prep_kernel"), ("forward pass", "cb_fwd_kernel"),
                ("reverse pass", "cb_bwd_kernel"), ("gradients", "cb_grad_kernel"))


def bwd_pmc_cmd(i):
    return (f"rocprofv3 --pmc {BWD_PMC_PASSES[i]} --output-format csv -d gpurun_out/bwd_pmc{i} -- "
            "python3 -u bench.py --only backward")


def _copy_factors():
    """FETCH_SIZE / WRITE_SIZE scale factors recorded with the HBM traffic profile."""
    m = re.search(r"```json\n(.*?)\n```", open(TRAFFIC_MD).read(), re.S)
    cf = json.loads(m.group(1))["copy_factor"]
    return {"FETCH_SIZE": cf["fetch"], "WRITE_SIZE": cf["write"]}


def ingest_backward_counters(dirs):
    """Counters of the chunked backward's four launches (bench.py --only
    backward).  Its first calls use the whole-sequence workspace (3 warm-up,
    5 timed); each launch's first 8 dispatches are those calls, and the last
    5 of them are averaged."""
    cal = _copy_factors()
    vals = {}
    for d in dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        rows = {}
        for f in files:
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    key = (f, int(r["Dispatch_Id"]))
                    ent = rows.setdefault(key, {"name": r["Kernel_Name"], "t": int(r["Start_Timestamp"]), "c": {}})
                    ent["c"][r["Counter_Name"]] = ent["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        disp = sorted(rows.values(), key=lambda e: e["t"])
        for label, frag in BWD_LAUNCHES:
            mine = [e for e in disp if frag in e["name"]][:8][-5:]
            for e in mine:
                for ctr, v in e["c"].items():
                    vals.setdefault(label, {}).setdefault(ctr, []).append(v)
    avg = {l: {c: sum(v) / len(v) for c, v in cs.items()} for l, cs in vals.items()}
    lines = ["# Counters of the chunked backward's launches (rocprofv3 --pmc)", "",
             "Workload: kda_chunk_bwd on B4 H32 T32768 d128 bf16 (heads 16-31 decay-stress), "
             "whole-sequence workspace; per launch, the average of the 5 timed calls after 3 "
             "warm-up ones.  FETCH_SIZE and WRITE_SIZE are scaled by the copy calibration of "
             f"the HBM traffic profile (fetch {cal['FETCH_SIZE']:.4f}, write {cal['WRITE_SIZE']:.4f}).  "
             f"Shares are of every SIMD's cycles ({N_SIMD} SIMDs; kernel cycles = "
             f"SQ_BUSY_CYCLES / {N_SE} shader engines).", "",
             "Commands (from the repository root):", ""]
    lines += ["    " + bwd_pmc_cmd(i) for i in range(len(BWD_PMC_PASSES))]
    lines += ["    python3 bench.py --ingest-backward-counters " +
              " ".join(f"gpurun_out/bwd_pmc{i}" for i in range(len(BWD_PMC_PASSES))), "",
              "| launch | fetch (GB) | write (GB) | kernel cycles | VALU active | MFMA busy | "
              "wave time waiting | LDS bank-conflict cycles per LDS instruction |",
              "|---|---|---|---|---|---|---|---|"]
    for label, _ in BWD_LAUNCHES:
        c = avg.get(label, {})
        f = c.get("FETCH_SIZE", float("nan")) * 1024 * cal["FETCH_SIZE"] / 1e9
        w = c.get("WRITE_SIZE", float("nan")) * 1024 * cal["WRITE_SIZE"] / 1e9
        cyc = c.get("SQ_BUSY_CYCLES", float("nan")) / N_SE
        va = 4 * c.get("SQ_ACTIVE_INST_VALU", float("nan")) / (cyc * N_SIMD)
        mb = c.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / (cyc * N_SIMD)
        wt = c.get("SQ_WAIT_ANY", float("nan")) / c.get("SQ_WAVE_CYCLES", float("nan"))
        bc = c.get("SQ_LDS_BANK_CONFLICT", float("nan")) / c.get("SQ_INSTS_LDS", float("nan"))
        lines.append(f"| {label} | {f:.2f} | {w:.2f} | {cyc:.4g} | {va:.3f} | {mb:.3f} | {wt:.3f} | {bc:.2f} |")
    lines.append("")
    os.makedirs(os.path.dirname(BWD_COUNTERS_MD), exist_ok=True)
    with open(BWD_COUNTERS_MD, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def ingest_sq(dirs):
    """Shader-sequencer counters of chunk32_kernel on the benchmark workload,
    averaged per dispatch, and unit-free figures per SIMD and 32-token period."""
    vals = {}
    counters = [c for ps in SQ_PASSES for c in ps.split()]
    for d in dirs:
        for ctr in counters:
            try:
                rows = _pmc_rows(d, ctr)
            except SystemExit:
                continue
            # the timed steps only: the last SQ_STEPS, after the warm-up; of
            # each step's launches the split's first phase (every counter is
            # largest there)
            named = [(n, x) for n, x in rows if _matches(n, KERNELS["fused_fwd"][0])]
            v = [max(x for _, x in g) for g in step_groups(named)][-SQ_STEPS:] if named else []
            if v:
                vals[ctr] = sum(v) / len(v)
    frag, wgs, periods = headline_main_instance()
    P, wide, guarded = headline_plan()
    simd_periods = wgs * 4 * periods
    lines = ["# Shader-sequencer counters, chunk32_kernel with the gate fused (rocprofv3 --pmc)", "",
             f"Workload: prefill B4 H32 T32768 d128 bf16 in the library's plan ({plan_text(P, wide, guarded)}); "
             f"the counters are those of the step's main launch `{frag[0]}` (the split's first phase): "
             f"{wgs} segment workgroups of 12 waves, "
             f"{periods} periods of 32 tokens each.  Averaged over the {SQ_STEPS} timed steps "
             f"after {SQ_WARMUP} warm-up ones.", "",
             "Commands (from the repository root):", ""]
    lines += ["    " + sq_cmd(i) for i in range(len(SQ_PASSES))]
    lines += ["    python3 bench.py --ingest-sq " + " ".join(f"gpurun_out/sq{i}" for i in range(len(SQ_PASSES))), "",
              "| counter | per dispatch |", "|---|---|"]
    for k in sorted(vals):
        lines.append(f"| {k} | {vals[k]:.4g} |")
    derived = []
    if "SQ_INSTS_VALU" in vals:
        derived.append(f"| VALU instructions per SIMD per period (MFMA included) | {vals['SQ_INSTS_VALU'] / simd_periods:.0f} |")
    if "SQ_INSTS_LDS" in vals:
        derived.append(f"| LDS instructions per SIMD per period | {vals['SQ_INSTS_LDS'] / simd_periods:.0f} |")
    if "SQ_LDS_BANK_CONFLICT" in vals and "SQ_INSTS_LDS" in vals:
        derived.append(f"| LDS bank-conflict cycles per LDS instruction | "
                       f"{vals['SQ_LDS_BANK_CONFLICT'] / vals['SQ_INSTS_LDS']:.2f} |")
    if "SQ_WAIT_ANY" in vals and "SQ_WAVE_CYCLES" in vals:
        derived.append(f"| share of wave time waiting (any) | {vals['SQ_WAIT_ANY'] / vals['SQ_WAVE_CYCLES']:.2f} |")
    if "SQ_ACTIVE_INST_ANY" in vals and "SQ_WAVE_CYCLES" in vals:
        derived.append(f"| share of wave time issuing | {vals['SQ_ACTIVE_INST_ANY'] / vals['SQ_WAVE_CYCLES']:.2f} |")
    rec = {}
    if "SQ_VALU_MFMA_BUSY_CYCLES" in vals and "SQ_BUSY_CYCLES" in vals:
        # SQ_BUSY_CYCLES is summed over the shader engines, so per engine it is
        # the kernel's duration in cycles; the MFMA busy cycles are summed over
        # every SIMD
        cycles = vals["SQ_BUSY_CYCLES"] / N_SE
        rec["mfma_busy_frac"] = vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * N_SIMD)
        derived.append(f"| kernel cycles (SQ_BUSY_CYCLES / {N_SE} shader engines) | {cycles:.4g} |")
        derived.append(f"| MFMA busy share of every SIMD's cycles (SQ_VALU_MFMA_BUSY_CYCLES / "
                       f"(cycles x {N_SIMD} SIMDs)) | {rec['mfma_busy_frac']:.3f} |")
        if "SQ_ACTIVE_INST_VALU" in vals:
            # SQ_ACTIVE_INST_VALU counts in units of 4 cycles (as SQ_WAVE_CYCLES,
            # whose per-wave sum is the kernel's cycles / 4 here)
            rec["valu_active_frac"] = 4 * vals["SQ_ACTIVE_INST_VALU"] / (cycles * N_SIMD)
            rec["issue_frac"] = rec["valu_active_frac"] + rec["mfma_busy_frac"]
            if "SQ_INSTS_VALU" in vals:
                rec["cycles_per_valu_inst"] = 4 * vals["SQ_ACTIVE_INST_VALU"] / vals["SQ_INSTS_VALU"]
                derived.append(f"| cycles per VALU instruction (4 SQ_ACTIVE_INST_VALU / SQ_INSTS_VALU) | "
                               f"{rec['cycles_per_valu_inst']:.2f} |")
            derived.append(f"| VALU-active share of every SIMD's cycles (4 SQ_ACTIVE_INST_VALU / "
                           f"(cycles x {N_SIMD} SIMDs)) | {rec['valu_active_frac']:.3f} |")
            derived.append(f"| issue share: VALU active + MFMA busy | {rec['issue_frac']:.3f} |")
    if derived:
        lines += ["", "Derived (counts are summed over waves; the shares divide counters kept in "
                  "the same unit):", "", "| figure | value |", "|---|---|"] + derived
    if rec:
        rec["source_sha256"] = source_hash(KERNELS["fused_fwd"][1])
        lines += ["", "Machine-readable record (read by bench.py while the kernel's sources hash "
                  "to `source_sha256`):", "", "```json", json.dumps(rec, indent=1), "```"]
    lines.append("")
    with open(SQ_MD, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # as many timed steps as the committed kernel trace takes (TRACE_STEPS)
    ap.add_argument("--steps", type=int, default=20)
    # the first ~10 launches of a fresh process run up to 30% slower (clocks
    # ramping; visible in a kernel trace), so the default warm-up covers them
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the extra lines (few-chain long prefill, position-pair diagonal)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--ingest-trace", metavar="TRACE_DIR")
    ap.add_argument("--ingest-trace-extra", nargs=2, metavar=("NAME", "TRACE_DIR"))
    ap.add_argument("--ingest-sq", nargs="+", metavar="PMC_DIR")
    ap.add_argument("--ingest-backward-counters", nargs="+", metavar="PMC_DIR")
    ap.add_argument("--only", choices=("long", "pairwise", "backward", "small"),
                    help="time only one extra line and print its record")
    args = ap.parse_args()
    if args.ingest_pmc:
        ingest_pmc(*args.ingest_pmc)
        return
    if args.ingest_trace:
        ingest_trace(args.ingest_trace)
        return
    if args.ingest_trace_extra:
        ingest_trace_extra(*args.ingest_trace_extra)
        return
    if args.ingest_sq:
        ingest_sq(args.ingest_sq)
        return
    if args.ingest_backward_counters:
        ingest_backward_counters(args.ingest_backward_counters)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the (batch, head) chains shard across GPUs without communication, so the "
              "per-GPU figure at --gpus 1 is the per-GPU throughput).", file=sys.stderr)
        sys.exit(2)
    _lib.load_library()
    torch.cuda.init()
    if args.only:
        rec = {"long": time_long_prefill, "pairwise": time_pairwise_diagonal,
               "backward": time_backward, "small": time_small_prefill}[args.only]()
        print(json.dumps(rec), flush=True)
        return

    copy_gbs = time_copy()
    res = time_prefill(args.steps, args.warmup)
    two = time_two_kernel(res["x"], args.steps)
    P, wide, guarded = headline_plan()
    w = PREFILL
    work = prefill_work(w)
    ms_per_step = res["wall_s"] * 1e3 / args.steps
    tokens = w.B * w.T
    value = tokens / (ms_per_step / 1e3)
    fused_s = res["fused_ms"] / 1e3
    fused_gbs = work["fused_bytes"] / fused_s / 1e9
    fused_tflops = work["chunk_flops"] / fused_s / 1e12
    ai = work["chunk_flops"] / work["fused_bytes"]
    attainable_tflops = min(BF16_PEAK_TFLOPS, ai * HBM_PEAK_GBS / 1e3)
    chunk_s = two["chunk_ms"] / 1e3
    gate_ms = two["gate_ms"]
    chunk_gbs = work["chunk_bytes"] / chunk_s / 1e9

    parity = {} if args.no_parity else parity_sample(res)
    cpu = None if args.no_cpu_baseline else cpu_baseline(res["x"], budget_s=args.cpu_budget)
    del res
    torch.cuda.empty_cache()

    plans_res = None if args.no_extras else time_prefill_plans()
    small_res = None if args.no_extras else time_small_prefill()
    long_res = None if args.no_extras else time_long_prefill()
    pair_res = None if args.no_extras else time_pairwise_diagonal()
    bwd_res = None if args.no_extras else time_backward()
    dec = time_decode(args.decode_steps)
    dbytes = decode_bytes(DECODE)
    dec_gbs = dbytes / (dec["us_per_step"] * 1e-6) / 1e9
    traffic = recorded_traffic()

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
                               f"(gate + chunked prefill per step, gate fused; the library's plan: "
                               f"{plan_text(P, wide, guarded)}); "
                               "decode 256x32 d128 fp32 state",
                   "global_batch": w.B, "seq_len": w.T, "heads": w.H, "dk": w.dk, "dv": w.dv,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": fused_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": fused_gbs / HBM_PEAK_GBS, "traffic": traffic["fused_fwd"],
                     "kernel": f"chunk32_kernel<128, true, ...> (gate fused; {plan_text(P, wide, guarded)})",
                     "bytes_per_step": work["fused_bytes"], "avg_ms": fused_s * 1e3,
                     "scope": "the whole step (every launch), HIP events on the launch stream"},
        "prefill": {"fused_ms": fused_s * 1e3,
                    "plan": {"segments": P, "workgroup_per_chain": wide, "guarded": guarded},
                    "other_plans": plans_res,
                    "alg_tflops": fused_tflops,
                    "flops_per_head_token": work["flops_per_head_token"],
                    "flops_per_head_token_c64_model": work["flops_per_head_token_c64"],
                    "arith_intensity": ai,
                    "mfma_frac_of_bf16_peak": fused_tflops / BF16_PEAK_TFLOPS,
                    "rocprof_mfma_busy_frac": recorded_mfma_busy(),
                    "rocprof_valu_active_frac": recorded_sq().get("valu_active_frac"),
                    "rocprof_issue_frac": recorded_sq().get("issue_frac"),
                    "roofline_frac_of_attainable": fused_tflops / attainable_tflops,
                    "head_tokens": work["head_tokens"],
                    "two_kernel": {"gate_ms": gate_ms, "chunk_ms": chunk_s * 1e3,
                                   "step_ms": gate_ms + chunk_s * 1e3,
                                   "gate_gbs": work["gate_bytes"] / (gate_ms / 1e3) / 1e9,
                                   "gate_traffic": traffic["gate"],
                                   "chunk_gbs": chunk_gbs,
                                   "chunk_hbm_frac": chunk_gbs / HBM_PEAK_GBS,
                                   "chunk_bytes_per_launch": work["chunk_bytes"],
                                   "chunk_traffic": traffic["chunk_fwd"]}},
        "prefill_h8_t4k": small_res,
        "prefill_long": long_res,
        "prefill_pairwise_diagonal": pair_res,
        "prefill_backward": bwd_res,
        "decode": {"us_per_step": dec["us_per_step"], "steps": dec["steps"],
                   "tokens_per_s": DECODE.B / (dec["us_per_step"] * 1e-6),
                   "roofline": {"bound": "hbm", "achieved": dec_gbs, "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": dec_gbs / HBM_PEAK_GBS,
                                "traffic": traffic["decode_step"],
                                "kernel": "decode_step_kernel<bf16,128,128>",
                                "bytes_per_launch": dbytes}},
        "hbm_copy_gbs": copy_gbs,
        "parity": parity,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
