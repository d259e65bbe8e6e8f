"""The Python binding rejects mismatched tensors before calling the library.

The C ABI takes bare pointers, so a k of the wrong dtype or a state of the
wrong shape would make a kernel read or write outside its buffer.  Every
wrapper therefore checks shapes, dtypes and devices first.  These tests run on
the CPU: `load_library` is replaced by a function that fails the test, so a
check that let a bad call through would be caught before any device work.
Correctly shaped CPU tensors must get as far as the device check.
"""
import pytest
import torch

import linear_attention_sequence_gate_amd._lib as L

B, T, H, DK, DV = 2, 5, 3, 32, 64
BF, F32 = torch.bfloat16, torch.float32


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def fail(*a, **k):
        raise AssertionError("the library was reached with invalid arguments")
    monkeypatch.setattr(L, "load_library", fail)


def prefill(dt=BF):
    return dict(q=torch.zeros(B, T, H, DK, dtype=dt), k=torch.zeros(B, T, H, DK, dtype=dt),
                v=torch.zeros(B, T, H, DV, dtype=dt), g=torch.zeros(B, T, H, DK, dtype=F32),
                beta=torch.zeros(B, T, H, dtype=dt))


def gated(dt=BF):
    a = prefill(dt)
    del a["g"]
    a["z"] = torch.zeros(B, T, H, DK, dtype=dt)
    a["A"] = torch.zeros(H, DK, dtype=F32)
    return a


def decode(dt=BF, N=4):
    return dict(q=torch.zeros(N, H, DK, dtype=dt), k=torch.zeros(N, H, DK, dtype=dt),
                v=torch.zeros(N, H, DV, dtype=dt), z=torch.zeros(N, H, DK, dtype=dt),
                A=torch.zeros(H, DK, dtype=F32), beta=torch.zeros(N, H, dtype=dt),
                state=torch.zeros(N, H, DK, DV, dtype=F32))


def _raises(fn, match, **kw):
    with pytest.raises(ValueError, match=match):
        fn(**kw)


# (argument, replacement, expected message) for kda_chunk_fwd
PREFILL_BAD = [
    ("k", torch.zeros(B, T, H, DK, dtype=F32), "k has dtype"),            # fp32 k with bf16 q
    ("k", torch.zeros(B, T, H, DK + 1, dtype=BF), "k has shape"),
    ("v", torch.zeros(B, T + 1, H, DV, dtype=BF), "v has shape"),
    ("v", torch.zeros(B, T, H, DV, dtype=F32), "v has dtype"),
    ("g", torch.zeros(B, T, H, DK, dtype=BF), "g has dtype"),
    ("g", torch.zeros(B, T, H, DV, dtype=F32), "g has shape"),
    ("beta", torch.zeros(B, T, H, dtype=F32), "beta has dtype"),         # fp32 beta with bf16 q
    ("beta", torch.zeros(B, T, dtype=BF), "beta has shape"),
    ("initial_state", torch.zeros(1, 1, DK, DV, dtype=F32), "initial_state has shape"),
    ("initial_state", torch.zeros(B, H, DK, DV, dtype=BF), "initial_state has dtype"),
    ("final_state", torch.zeros(B, H, DV, DK, dtype=F32), "final_state has shape"),
    ("o", torch.zeros(B, T, H, DV + 32, dtype=BF), "o has shape"),
    ("o", torch.zeros(B, T, H, DV, dtype=F32), "o has dtype"),
    ("workspace", torch.zeros(64, dtype=F32), "workspace must be a uint8"),
]


@pytest.mark.parametrize("name,bad,msg", PREFILL_BAD, ids=[c[2] for c in PREFILL_BAD])
def test_chunk_fwd_rejects(name, bad, msg):
    a = prefill()
    a[name] = bad
    _raises(L.kda_chunk_fwd, msg, **a)


def test_chunk_fwd_rejects_q_rank_and_dtype():
    a = prefill()
    a["q"] = torch.zeros(B, T, H * DK, dtype=BF)
    _raises(L.kda_chunk_fwd, "q must have 4 dimensions", **a)
    a = prefill()
    a["q"] = torch.zeros(B, T, H, DK, dtype=torch.float16)
    _raises(L.kda_chunk_fwd, "q has dtype", **a)


@pytest.mark.parametrize("dt", [BF, F32])
def test_chunk_fwd_valid_reaches_device_check(dt):
    a = prefill(dt)
    a["initial_state"] = torch.zeros(B, H, DK, DV, dtype=F32)
    a["o"] = torch.zeros(B, T, H, DV, dtype=dt)
    _raises(L.kda_chunk_fwd, "device tensors only", **a)


GATED_BAD = [
    ("z", torch.zeros(B, T, H, DK, dtype=F32), "z has dtype"),
    ("z", torch.zeros(B, T, H, DV, dtype=BF), "z has shape"),
    ("A", torch.zeros(DK, dtype=F32), "A has shape"),
    ("A", torch.zeros(H, DK, dtype=BF), "A has dtype"),
    ("A", None, "z and A are required"),
    ("beta", torch.zeros(B, T, H, dtype=F32), "beta has dtype"),
    ("initial_state", torch.zeros(B, H, DK, DK, dtype=F32), "initial_state has shape"),
]


@pytest.mark.parametrize("name,bad,msg", GATED_BAD, ids=[c[2] for c in GATED_BAD])
def test_chunk_fwd_gated_rejects(name, bad, msg):
    a = gated()
    a[name] = bad
    _raises(L.kda_chunk_fwd_gated, msg, **a)


def test_chunk_fwd_gated_valid_reaches_device_check():
    _raises(L.kda_chunk_fwd_gated, "device tensors only", **gated())


def test_gate_rejects():
    z = torch.zeros(B, T, H, DK, dtype=BF)
    A = torch.zeros(H, DK, dtype=F32)
    _raises(L.kda_gate, "A has shape", z=z, A=torch.zeros(H + 1, DK, dtype=F32))
    _raises(L.kda_gate, "A has dtype", z=z, A=A.double())
    _raises(L.kda_gate, "g has dtype", z=z, A=A, g=torch.zeros(B, T, H, DK, dtype=BF))
    _raises(L.kda_gate, "g has shape", z=z, A=A, g=torch.zeros(B, T, H, DK // 2, dtype=F32))
    _raises(L.kda_gate, "z has dtype", z=z.double(), A=A)
    _raises(L.kda_gate, "device tensors only", z=z, A=A)


DECODE_BAD = [
    ("k", torch.zeros(4, H, DK, dtype=F32), "k has dtype"),
    ("k", torch.zeros(5, H, DK, dtype=BF), "k has shape"),
    ("v", torch.zeros(4, H, DV, dtype=F32), "v has dtype"),
    ("z", torch.zeros(4, H, DV, dtype=BF), "z has shape"),
    ("A", torch.zeros(H, DV, dtype=F32), "A has shape"),
    ("A", None, "A is required"),
    ("beta", torch.zeros(4, H, dtype=F32), "beta has dtype"),
    ("state", torch.zeros(1, 1, DK, DV, dtype=F32), "state has shape"),
    ("state", torch.zeros(4, H, DK, DV, dtype=BF), "state has dtype"),
    ("o", torch.zeros(4, H, DK, dtype=BF), "o has shape"),
]


@pytest.mark.parametrize("name,bad,msg", DECODE_BAD, ids=[c[2] for c in DECODE_BAD])
def test_decode_rejects(name, bad, msg):
    a = decode()
    a[name] = bad
    _raises(L.kda_decode_step, msg, **a)


def test_decode_valid_reaches_device_check():
    _raises(L.kda_decode_step, "device tensors only", **decode())


def test_decode_pooled_rejects():
    a = decode()
    del a["state"]
    pool = torch.zeros(7, H, DK, DV, dtype=F32)
    slots = torch.zeros(4, dtype=torch.int32)
    _raises(L.kda_decode_step_pooled, "state_pool has shape", state_pool=torch.zeros(
        7, H, DV, DK, dtype=F32), slots=slots, **a)
    _raises(L.kda_decode_step_pooled, "state_pool has dtype", state_pool=pool.to(BF),
            slots=slots, **a)
    _raises(L.kda_decode_step_pooled, "device tensors only", state_pool=pool, slots=slots, **a)


def test_chunk_fwd_pooled_rejects():
    a = prefill()
    pool = torch.zeros(9, H, DK, DV, dtype=F32)
    slots = torch.zeros(B, dtype=torch.int32)
    _raises(L.kda_chunk_fwd_pooled, "initial_state has shape",
            state_pool=torch.zeros(9, H, DK, DK, dtype=F32), slots=slots, **a)
    _raises(L.kda_chunk_fwd_pooled, "initial_state has dtype", state_pool=pool.to(BF),
            slots=slots, **a)
    _raises(L.kda_chunk_fwd_pooled, "device tensors only", state_pool=pool, slots=slots, **a)


def test_varlen_rejects():
    total = 11
    q = torch.zeros(total, H, DK, dtype=BF)
    args = dict(q=q, k=q.clone(), v=torch.zeros(total, H, DV, dtype=BF),
                g=torch.zeros(total, H, DK, dtype=F32), beta=torch.zeros(total, H, dtype=BF),
                state_pool=torch.zeros(4, H, DK, DV, dtype=F32),
                slots=torch.zeros(2, dtype=torch.int32),
                cu_seqlens=torch.tensor([0, 5, 11], dtype=torch.int64))
    bad = dict(args, v=torch.zeros(total - 1, H, DV, dtype=BF))
    _raises(L.kda_chunk_fwd_varlen_pooled, "v has shape", **bad)
    bad = dict(args, slots=torch.zeros(3, dtype=torch.int32))
    _raises(L.kda_chunk_fwd_varlen_pooled, "slots has shape", **bad)
    bad = dict(args, g=torch.zeros(total, H, DK, dtype=BF))
    _raises(L.kda_chunk_fwd_varlen_pooled, "g has dtype", **bad)
    _raises(L.kda_chunk_fwd_varlen_pooled, "device tensors only", **args)
    ga = dict(args)
    del ga["g"]
    ga.update(z=torch.zeros(total, H, DK, dtype=F32), A=torch.zeros(H, DK, dtype=F32))
    _raises(L.kda_chunk_fwd_varlen_pooled_gated, "z has dtype", **ga)
    ga.update(z=torch.zeros(total, H, DK, dtype=BF))
    _raises(L.kda_chunk_fwd_varlen_pooled_gated, "device tensors only", **ga)


def test_chunk_bwd_rejects():
    a = prefill()
    d_o = torch.zeros(B, T, H, DV, dtype=BF)
    _raises(L.kda_chunk_bwd, "d_o has dtype", initial_state=None, d_o=d_o.float(), **a)
    _raises(L.kda_chunk_bwd, "d_o has shape", initial_state=None,
            d_o=torch.zeros(B, T, H, DK, dtype=BF), **a)
    _raises(L.kda_chunk_bwd, "d_final_state has shape", initial_state=None, d_o=d_o,
            d_final_state=torch.zeros(B, H, DK, DK, dtype=F32), **a)
    _raises(L.kda_chunk_bwd, "g and d_o are required", initial_state=None, d_o=None, **a)
    _raises(L.kda_chunk_bwd, "device tensors only", initial_state=None, d_o=d_o, **a)


def test_gate_bwd_rejects():
    z = torch.zeros(B, T, H, DK, dtype=BF)
    A = torch.zeros(H, DK, dtype=F32)
    dg = torch.zeros(B, T, H, DK, dtype=F32)
    _raises(L.kda_gate_bwd, "dg has dtype", z=z, A=A, dg=dg.to(BF))
    _raises(L.kda_gate_bwd, "dg has shape", z=z, A=A, dg=dg[:, :1])
    _raises(L.kda_gate_bwd, "device tensors only", z=z, A=A, dg=dg)
