"""Thin ctypes binding of libkda.so (see include/kda.h for the contract).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libkda.so.  PyTorch supplies device memory and the current stream.
There is no fallback: if the library is missing or a call fails, an exception
is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
KDA_OK = 0
KDA_ERR_INVALID_ARGUMENT = -1
KDA_ERR_UNSUPPORTED = -2
KDA_ERR_HIP = -3
KDA_ERR_RANGE = -4
KDA_FLAG_CHECK_RANGE = 1
KDA_FLAG_PAIRWISE_DIAGONAL = 2
KDA_FLAG_SEGMENTS_SHIFT = 8
KDA_FLAG_SEGMENTS_MASK = 0xFF00
KDA_FLAG_TOKEN_BACKWARD = 0x10000
KDA_FLAG_SPLIT_FULL_RERUN = 0x20000
KDA_FLAG_WORKGROUP_PER_CHAIN = 0x40000
KDA_FLAG_WORKGROUP_PER_SLICE = 0x80000


def kda_flag_segments(n: int) -> int:
    """Flag bits that request n segments per sequence (0 = library's choice, 1 = no split)."""
    return (int(n) << KDA_FLAG_SEGMENTS_SHIFT) & KDA_FLAG_SEGMENTS_MASK

EXPORTED = ("kda_gate", "kda_chunk_fwd", "kda_chunk_fwd_workspace_size",
            "kda_chunk_fwd_workspace_size_segments", "kda_chunk_fwd_auto_segments",
            "kda_chunk_fwd_plan", "kda_decode_step", "kda_state_pool_reset", "kda_chunk_fwd_pooled",
            "kda_chunk_fwd_varlen_pooled", "kda_decode_step_pooled", "kda_chunk_bwd",
            "kda_chunk_bwd_workspace_size", "kda_gate_bwd", "kda_gate_bwd_workspace_size",
            "kda_chunk_fwd_gated", "kda_chunk_fwd_gated_workspace_size",
            "kda_chunk_fwd_varlen_pooled_gated", "kda_chunk_fwd_gated_noalloc",
            "kda_chunk_bwd_workspace_size_flags", "kda_last_error", "kda_version")


class KdaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libkda error {code}: {msg}")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkda.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m linear_attention_sequence_gate_amd.build`")
    L = ctypes.CDLL(path)
    vp, i64, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.kda_gate.argtypes = [vp, vp, vp, i64, i64, i64, i64, c_int, vp]
    L.kda_gate.restype = c_int
    L.kda_chunk_fwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, c_int]
    L.kda_chunk_fwd_workspace_size.restype = ctypes.c_size_t
    L.kda_chunk_fwd_workspace_size_segments.argtypes = [i64, i64, i64, i64, i64, c_int, c_int]
    L.kda_chunk_fwd_workspace_size_segments.restype = ctypes.c_size_t
    L.kda_chunk_fwd_auto_segments.argtypes = [i64, i64, i64, i64, i64, c_int]
    L.kda_chunk_fwd_auto_segments.restype = c_int
    L.kda_chunk_fwd_plan.argtypes = [i64, i64, i64, i64, i64, c_int, ctypes.c_uint,
                                     ctypes.POINTER(c_int), ctypes.POINTER(c_int), ctypes.POINTER(c_int)]
    L.kda_chunk_fwd_plan.restype = c_int
    L.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                i64, i64, i64, i64, i64, c_int, ctypes.c_uint, vp]
    L.kda_chunk_fwd.restype = c_int
    L.kda_chunk_fwd_gated_workspace_size.argtypes = [i64, i64, i64, i64, i64, c_int]
    L.kda_chunk_fwd_gated_workspace_size.restype = ctypes.c_size_t
    L.kda_chunk_fwd_gated.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                      i64, i64, i64, i64, i64, c_int, ctypes.c_uint, vp]
    L.kda_chunk_fwd_gated.restype = c_int
    L.kda_chunk_fwd_gated_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                              i64, i64, i64, i64, i64, c_int, ctypes.c_uint, vp]
    L.kda_chunk_fwd_gated_noalloc.restype = c_int
    L.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, c_int, vp]
    L.kda_decode_step.restype = c_int
    L.kda_state_pool_reset.argtypes = [vp, vp, i64, i64, i64, i64, i64, vp]
    L.kda_state_pool_reset.restype = c_int
    L.kda_chunk_fwd_pooled.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                       i64, i64, i64, i64, i64, i64, c_int, ctypes.c_uint, vp]
    L.kda_chunk_fwd_pooled.restype = c_int
    L.kda_decode_step_pooled.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                         i64, c_int, vp]
    L.kda_chunk_fwd_varlen_pooled.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64,
                                              i64, i64, i64, c_int, ctypes.c_uint, vp]
    L.kda_chunk_fwd_varlen_pooled.restype = c_int
    L.kda_chunk_fwd_varlen_pooled_gated.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64,
                                                    i64, i64, i64, i64, i64, c_int, ctypes.c_uint, vp]
    L.kda_chunk_fwd_varlen_pooled_gated.restype = c_int
    L.kda_chunk_bwd_workspace_size.argtypes = [i64, i64, i64, i64, i64, c_int]
    L.kda_chunk_bwd_workspace_size.restype = ctypes.c_size_t
    L.kda_chunk_bwd_workspace_size_flags.argtypes = [i64, i64, i64, i64, i64, c_int, ctypes.c_uint,
                                                     i64]
    L.kda_chunk_bwd_workspace_size_flags.restype = ctypes.c_size_t
    L.kda_chunk_bwd.argtypes = [vp] * 15 + [ctypes.c_size_t, i64, i64, i64, i64, i64, c_int,
                                            ctypes.c_uint, vp]
    L.kda_chunk_bwd.restype = c_int
    L.kda_gate_bwd_workspace_size.argtypes = [i64, i64, i64, i64]
    L.kda_gate_bwd_workspace_size.restype = ctypes.c_size_t
    L.kda_gate_bwd.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i64, i64, i64, i64, c_int, vp]
    L.kda_gate_bwd.restype = c_int
    L.kda_decode_step_pooled.restype = c_int
    L.kda_last_error.argtypes = []
    L.kda_last_error.restype = ctypes.c_char_p
    L.kda_version.argtypes = []
    L.kda_version.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(code: int):
    if code != KDA_OK:
        raise KdaError(code, load_library().kda_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("libkda takes device tensors only")
            if not t.is_contiguous():
                raise ValueError("libkda takes contiguous tensors only")


_IN_DTYPES = (torch.bfloat16, torch.float32)


def _expect(name: str, t: Optional[torch.Tensor], shape, dtype=None) -> None:
    """Raise ValueError unless `t` (when given) has exactly `shape` and `dtype`.

    The C ABI receives bare pointers and cannot tell a wrong-sized or
    wrong-typed buffer from a right one, so every wrapper checks each tensor
    here, before the library is called."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(int(s) for s in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _in_dtype(name: str, t: torch.Tensor) -> torch.dtype:
    if t.dtype not in _IN_DTYPES:
        raise ValueError(f"{name} has dtype {t.dtype}; bfloat16 or float32 expected")
    return t.dtype


def _same_device(*ts) -> None:
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors on different devices: {sorted(str(d) for d in devs)}")


def _rank(name: str, t: torch.Tensor, n: int) -> None:
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, got shape {tuple(t.shape)}")


def _workspace(t: Optional[torch.Tensor]) -> None:
    if t is not None and t.dtype != torch.uint8:
        raise ValueError(f"workspace must be a uint8 tensor, got {t.dtype}")


def kda_version() -> str:
    return load_library().kda_version().decode()


def kda_last_error() -> str:
    return load_library().kda_last_error().decode()


def kda_gate(z: torch.Tensor, A: torch.Tensor, g: Optional[torch.Tensor] = None,
             stream=None) -> torch.Tensor:
    """g = -5 * sigmoid(exp(A) * z).  z [B,T,H,dk] (bf16/fp32), A [H,dk] fp32 -> g fp32."""
    _rank("z", z, 4)
    B, T, H, dk = z.shape
    _in_dtype("z", z)
    _expect("A", A, (H, dk), torch.float32)
    _expect("g", g, (B, T, H, dk), torch.float32)
    _same_device(z, A, g)
    _dev(z, A, g)
    if g is None:
        g = torch.empty(z.shape, device=z.device, dtype=torch.float32)
    _check(load_library().kda_gate(_ptr(z), _ptr(A), _ptr(g), B, T, H, dk, _dtype_code(z),
                                   _stream(stream)))
    return g


def _check_prefill(q, k, v, beta, initial_state, final_state, o, workspace, g=None, z=None,
                   A=None, d_o=None, d_final_state=None, state_rows=None):
    """Shapes and dtypes of a prefill-type call: q, k (and z) [B,T,H,dk], v
    and o [B,T,H,dv], beta [B,T,H], all in q's dtype; g [B,T,H,dk], A [H,dk]
    and the states [B,H,dk,dv] (or [state_rows,H,dk,dv]) in fp32.  Returns
    (B, T, H, dk, dv)."""
    _rank("q", q, 4)
    B, T, H, dk = q.shape
    dt = _in_dtype("q", q)
    _rank("v", v, 4)
    dv = v.shape[-1]
    _expect("k", k, (B, T, H, dk), dt)
    _expect("v", v, (B, T, H, dv), dt)
    _expect("beta", beta, (B, T, H), dt)
    _expect("z", z, (B, T, H, dk), dt)
    _expect("o", o, (B, T, H, dv), dt)
    _expect("d_o", d_o, (B, T, H, dv), dt)
    _expect("g", g, (B, T, H, dk), torch.float32)
    _expect("A", A, (H, dk), torch.float32)
    rows = B if state_rows is None else state_rows
    _expect("initial_state", initial_state, (rows, H, dk, dv), torch.float32)
    _expect("final_state", final_state, (rows, H, dk, dv), torch.float32)
    _expect("d_final_state", d_final_state, (B, H, dk, dv), torch.float32)
    _workspace(workspace)
    _same_device(q, k, v, beta, z, o, d_o, g, A, initial_state, final_state, d_final_state,
                 workspace)
    return B, T, H, dk, dv


def kda_chunk_fwd_workspace_size(B: int, T: int, H: int, dk: int, dv: int, dtype: int,
                                 nseg: Optional[int] = None) -> int:
    """Workspace bytes for these sizes; nseg is an explicit segment count (None: the library's)."""
    L = load_library()
    if nseg is None:
        return int(L.kda_chunk_fwd_workspace_size(B, T, H, dk, dv, dtype))
    return int(L.kda_chunk_fwd_workspace_size_segments(B, T, H, dk, dv, dtype, nseg))


def kda_chunk_fwd_auto_segments(B: int, T: int, H: int, dk: int, dv: int, dtype: int) -> int:
    """Segments per sequence the library picks for these sizes (1 = one pass)."""
    return int(load_library().kda_chunk_fwd_auto_segments(B, T, H, dk, dv, dtype))


def kda_chunk_fwd_plan(B: int, T: int, H: int, dk: int, dv: int, dtype: int,
                       flags: int = 0, with_guard: bool = False):
    """(segments per sequence, one workgroup per chain?) that kda_chunk_fwd
    follows for these sizes and flags given the workspace the library asks
    for; with_guard adds whether a two-segment split is guarded (a probe picks
    it or the one pass on the device)."""
    seg, per_chain, guarded = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    _check(load_library().kda_chunk_fwd_plan(B, T, H, dk, dv, dtype, flags, ctypes.byref(seg),
                                             ctypes.byref(per_chain), ctypes.byref(guarded)))
    if with_guard:
        return seg.value, bool(per_chain.value), bool(guarded.value)
    return seg.value, bool(per_chain.value)


def kda_chunk_fwd(q, k, v, g, beta, initial_state=None, final_state=None, o=None,
                  want_final_state: bool = True, flags: int = 0, workspace=None,
                  stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise prefill.  Returns (o [B,T,H,dv], final_state [B,H,dk,dv] fp32 or None)."""
    B, T, H, dk, dv = _check_prefill(q, k, v, beta, initial_state, final_state, o, workspace,
                                     g=g)
    _dev(q, k, v, g, beta, initial_state, final_state, o, workspace)
    dt = _dtype_code(q)
    if o is None:
        o = torch.empty((B, T, H, dv), device=q.device, dtype=q.dtype)
    if final_state is None and want_final_state:
        final_state = torch.empty((B, H, dk, dv), device=q.device, dtype=torch.float32)
    if workspace is None:
        # the range-check counter and, when the sizes take the sequence-split
        # path, its per-segment states
        nseg = (flags & KDA_FLAG_SEGMENTS_MASK) >> KDA_FLAG_SEGMENTS_SHIFT
        ws_bytes = kda_chunk_fwd_workspace_size(B, T, H, dk, dv, dt, nseg)
        workspace = torch.empty(max(ws_bytes, 256), device=q.device, dtype=torch.uint8)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().kda_chunk_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(final_state),
        _ptr(o), _ptr(workspace), ws_bytes, B, T, H, dk, dv, dt, flags, _stream(stream)))
    return o, final_state


def kda_chunk_fwd_gated_workspace_size(B: int, T: int, H: int, dk: int, dv: int, dtype: int,
                                       nseg: Optional[int] = None) -> int:
    """Workspace bytes for kda_chunk_fwd_gated (nseg: an explicit segment count)."""
    L = load_library()
    gated = int(L.kda_chunk_fwd_gated_workspace_size(B, T, H, dk, dv, dtype))
    return max(gated, kda_chunk_fwd_workspace_size(B, T, H, dk, dv, dtype, nseg))


def kda_chunk_fwd_gated(q, k, v, z, A, beta, initial_state=None, final_state=None, o=None,
                        want_final_state: bool = True, flags: int = 0, workspace=None,
                        stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Gate and chunkwise prefill in one call (g from z and A inside it).
    Returns (o [B,T,H,dv], final_state [B,H,dk,dv] fp32 or None)."""
    B, T, H, dk, dv = _check_prefill(q, k, v, beta, initial_state, final_state, o, workspace,
                                     z=z, A=A)
    if z is None or A is None:
        raise ValueError("z and A are required")
    _dev(q, k, v, z, A, beta, initial_state, final_state, o, workspace)
    dt = _dtype_code(q)
    if o is None:
        o = torch.empty((B, T, H, dv), device=q.device, dtype=q.dtype)
    if final_state is None and want_final_state:
        final_state = torch.empty((B, H, dk, dv), device=q.device, dtype=torch.float32)
    if workspace is None:
        nseg = (flags & KDA_FLAG_SEGMENTS_MASK) >> KDA_FLAG_SEGMENTS_SHIFT
        ws_bytes = kda_chunk_fwd_gated_workspace_size(B, T, H, dk, dv, dt, nseg)
        workspace = torch.empty(max(ws_bytes, 256), device=q.device, dtype=torch.uint8)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().kda_chunk_fwd_gated(
        _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A), _ptr(beta), _ptr(initial_state),
        _ptr(final_state), _ptr(o), _ptr(workspace), ws_bytes, B, T, H, dk, dv, dt, flags,
        _stream(stream)))
    return o, final_state


KDA_NOALLOC_SCRATCH_BYTES = 32 << 20


def kda_chunk_fwd_gated_noalloc(q, k, v, z, A, beta, initial_state=None, final_state=None,
                                o=None, flags: int = 0,
                                stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """kda_chunk_fwd_gated with the library's fixed device scratch instead of a
    workspace (the C call allocates nothing; pass `o` and `final_state` to make
    the whole call allocation-free here too).  Returns (o, final_state)."""
    B, T, H, dk, dv = _check_prefill(q, k, v, beta, initial_state, final_state, o, None,
                                     z=z, A=A)
    if z is None or A is None:
        raise ValueError("z and A are required")
    _dev(q, k, v, z, A, beta, initial_state, final_state, o)
    dt = _dtype_code(q)
    if o is None:
        o = torch.empty((B, T, H, dv), device=q.device, dtype=q.dtype)
    _check(load_library().kda_chunk_fwd_gated_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A), _ptr(beta), _ptr(initial_state),
        _ptr(final_state), _ptr(o), B, T, H, dk, dv, dt, flags, _stream(stream)))
    return o, final_state


def _check_decode(q, k, v, z, A, beta, o, state=None, pool=None):
    """Shapes and dtypes of a decode call: q, k, z [N,H,dk], v and o [N,H,dv],
    beta [N,H], all in q's dtype; A [H,dk] and the state [N,H,dk,dv] (or a
    pool [n_slots,H,dk,dv]) in fp32.  Returns (N, H, dk, dv)."""
    _rank("q", q, 3)
    N, H, dk = q.shape
    dt = _in_dtype("q", q)
    _rank("v", v, 3)
    dv = v.shape[-1]
    _expect("k", k, (N, H, dk), dt)
    _expect("z", z, (N, H, dk), dt)
    _expect("v", v, (N, H, dv), dt)
    _expect("beta", beta, (N, H), dt)
    _expect("o", o, (N, H, dv), dt)
    _expect("A", A, (H, dk), torch.float32)
    if state is not None:
        _expect("state", state, (N, H, dk, dv), torch.float32)
    if pool is not None:
        _rank("state_pool", pool, 4)
        _expect("state_pool", pool, (pool.shape[0], H, dk, dv), torch.float32)
    for name, t in (("z", z), ("A", A), ("beta", beta)):
        if t is None:
            raise ValueError(f"{name} is required")
    _same_device(q, k, v, z, A, beta, o, state, pool)
    return N, H, dk, dv


def kda_decode_step(q, k, v, z, A, beta, state, o=None, stream=None) -> torch.Tensor:
    """One decode step; `state` [N,H,dk,dv] fp32 is updated in place.  Returns o [N,H,dv]."""
    N, H, dk, dv = _check_decode(q, k, v, z, A, beta, o, state=state)
    _dev(q, k, v, z, A, beta, state, o)
    if o is None:
        o = torch.empty((N, H, dv), device=q.device, dtype=q.dtype)
    _check(load_library().kda_decode_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A), _ptr(beta), _ptr(state), _ptr(o),
        N, H, dk, dv, _dtype_code(q), _stream(stream)))
    return o


def _slots(slots: torch.Tensor) -> torch.Tensor:
    if slots.dtype != torch.int32 or not slots.is_cuda or not slots.is_contiguous():
        raise ValueError("slots must be a contiguous int32 CUDA tensor")
    return slots


def kda_state_pool_reset(state_pool, slots, stream=None) -> None:
    """Zero the listed slots of a state pool [n_slots, H, dk, dv] fp32."""
    _rank("state_pool", state_pool, 4)
    if state_pool.dtype != torch.float32:
        raise ValueError(f"state_pool has dtype {state_pool.dtype}, expected torch.float32")
    _dev(state_pool)
    slots = _slots(slots)
    _same_device(state_pool, slots)
    n_slots, H, dk, dv = state_pool.shape
    _check(load_library().kda_state_pool_reset(
        _ptr(state_pool), _ptr(slots), slots.numel(), n_slots, H, dk, dv, _stream(stream)))


def kda_chunk_fwd_pooled(q, k, v, g, beta, state_pool, slots, o=None, flags: int = 0,
                         workspace=None, stream=None) -> torch.Tensor:
    """Chunkwise prefill of B sequences whose states live in `state_pool`
    [n_slots, H, dk, dv] fp32 at `slots` [B] int32 (read, then overwritten
    with the final states).  Returns o [B,T,H,dv]."""
    _rank("state_pool", state_pool, 4)
    B, T, H, dk, dv = _check_prefill(q, k, v, beta, state_pool, None, o, workspace, g=g,
                                     state_rows=state_pool.shape[0])
    _dev(q, k, v, g, beta, state_pool, o, workspace)
    slots = _slots(slots)
    _expect("slots", slots, (B,))
    _same_device(q, slots)
    n_slots = state_pool.shape[0]
    dt = _dtype_code(q)
    if o is None:
        o = torch.empty((B, T, H, dv), device=q.device, dtype=q.dtype)
    if workspace is None:
        nseg = (flags & KDA_FLAG_SEGMENTS_MASK) >> KDA_FLAG_SEGMENTS_SHIFT
        ws_bytes = kda_chunk_fwd_workspace_size(B, T, H, dk, dv, dt, nseg)
        workspace = torch.empty(max(ws_bytes, 256), device=q.device, dtype=torch.uint8)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load_library().kda_chunk_fwd_pooled(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool), _ptr(slots), _ptr(o),
        _ptr(workspace), ws_bytes, B, T, n_slots, H, dk, dv, dt, flags, _stream(stream)))
    return o


def kda_decode_step_pooled(q, k, v, z, A, beta, state_pool, slots, o=None,
                           stream=None) -> torch.Tensor:
    """One decode step for N sequences whose states live in `state_pool`
    [n_slots, H, dk, dv] fp32 at `slots` [N] int32, updated in place.
    Returns o [N,H,dv]."""
    N, H, dk, dv = _check_decode(q, k, v, z, A, beta, o, pool=state_pool)
    _dev(q, k, v, z, A, beta, state_pool, o)
    slots = _slots(slots)
    _expect("slots", slots, (N,))
    _same_device(q, slots)
    if o is None:
        o = torch.empty((N, H, dv), device=q.device, dtype=q.dtype)
    _check(load_library().kda_decode_step_pooled(
        _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A), _ptr(beta), _ptr(state_pool), _ptr(slots),
        _ptr(o), N, state_pool.shape[0], H, dk, dv, _dtype_code(q), _stream(stream)))
    return o


def _check_varlen(q, k, v, beta, state_pool, slots, cu_seqlens, o, g=None, z=None, A=None):
    """Shapes and dtypes of a packed (variable-length) prefill: q, k (and z)
    [total,H,dk], v and o [total,H,dv], beta [total,H] in q's dtype; g
    [total,H,dk], A [H,dk] and the pool [n_slots,H,dk,dv] fp32; slots [B]
    int32 and cu_seqlens [B+1] int64.  Returns (total, H, dk, dv, B)."""
    _rank("q", q, 3)
    total, H, dk = q.shape
    dt = _in_dtype("q", q)
    _rank("v", v, 3)
    dv = v.shape[-1]
    _expect("k", k, (total, H, dk), dt)
    _expect("z", z, (total, H, dk), dt)
    _expect("v", v, (total, H, dv), dt)
    _expect("beta", beta, (total, H), dt)
    _expect("o", o, (total, H, dv), dt)
    _expect("g", g, (total, H, dk), torch.float32)
    _expect("A", A, (H, dk), torch.float32)
    _rank("state_pool", state_pool, 4)
    _expect("state_pool", state_pool, (state_pool.shape[0], H, dk, dv), torch.float32)
    _rank("cu_seqlens", cu_seqlens, 1)
    B = cu_seqlens.numel() - 1
    _expect("slots", slots, (B,))
    _same_device(q, k, v, beta, z, g, A, o, state_pool, slots, cu_seqlens)
    return total, H, dk, dv, B


def kda_chunk_fwd_varlen_pooled(q, k, v, g, beta, state_pool, slots, cu_seqlens, o=None,
                                flags: int = 0, stream=None) -> torch.Tensor:
    """Prefill of B sequences of different lengths packed along the token axis
    (q, k, g [total,H,dk], v [total,H,dv], beta [total,H]; sequence b is rows
    cu_seqlens[b] .. cu_seqlens[b+1]-1, cu_seqlens int64 [B+1] on the device),
    with states in `state_pool` at `slots` [B].  Returns o [total,H,dv]."""
    total, H, dk, dv, B = _check_varlen(q, k, v, beta, state_pool, slots, cu_seqlens, o, g=g)
    _dev(q, k, v, g, beta, state_pool, o)
    slots = _slots(slots)
    if cu_seqlens.dtype != torch.int64 or not cu_seqlens.is_cuda or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int64 CUDA tensor")
    if o is None:
        o = torch.empty((total, H, dv), device=q.device, dtype=q.dtype)
    _check(load_library().kda_chunk_fwd_varlen_pooled(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool), _ptr(slots),
        _ptr(cu_seqlens), _ptr(o), B, total, state_pool.shape[0], H, dk, dv, _dtype_code(q), flags,
        _stream(stream)))
    return o


def kda_chunk_fwd_varlen_pooled_gated(q, k, v, z, A, beta, state_pool, slots, cu_seqlens, o=None,
                                      flags: int = 0, stream=None) -> torch.Tensor:
    """kda_chunk_fwd_varlen_pooled with the gate inside the chunk kernel: z
    [total,H,dk] and A [H,dk] instead of g.  Returns o [total,H,dv]."""
    total, H, dk, dv, B = _check_varlen(q, k, v, beta, state_pool, slots, cu_seqlens, o, z=z,
                                        A=A)
    if z is None or A is None:
        raise ValueError("z and A are required")
    _dev(q, k, v, z, A, beta, state_pool, o)
    slots = _slots(slots)
    if cu_seqlens.dtype != torch.int64 or not cu_seqlens.is_cuda or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int64 CUDA tensor")
    if o is None:
        o = torch.empty((total, H, dv), device=q.device, dtype=q.dtype)
    _check(load_library().kda_chunk_fwd_varlen_pooled_gated(
        _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A), _ptr(beta), _ptr(state_pool), _ptr(slots),
        _ptr(cu_seqlens), _ptr(o), B, total, state_pool.shape[0], H, dk, dv, _dtype_code(q), flags,
        _stream(stream)))
    return o


def kda_chunk_bwd_workspace_size(B: int, T: int, H: int, dk: int, dv: int, dtype: int) -> int:
    return int(load_library().kda_chunk_bwd_workspace_size(B, T, H, dk, dv, dtype))


KDA_BWD_SEGMENTS_MIN_WORKSPACE = -1


def kda_chunk_bwd_workspace_size_flags(B: int, T: int, H: int, dk: int, dv: int, dtype: int,
                                       flags: int = 0, segment_tokens: int = 0) -> int:
    """Workspace bytes of the backward path `flags` selects: segment_tokens 0 =
    the whole sequence in one segment, n > 0 = segments of n tokens (chunked
    path), KDA_BWD_SEGMENTS_MIN_WORKSPACE = the least kda_chunk_bwd accepts."""
    return int(load_library().kda_chunk_bwd_workspace_size_flags(B, T, H, dk, dv, dtype, flags,
                                                                 segment_tokens))


def kda_chunk_bwd(q, k, v, g, beta, initial_state, d_o, d_final_state=None,
                  want_d_initial_state: bool = True, workspace=None, flags: int = 0,
                  segment_tokens: Optional[int] = None, stream=None) -> dict:
    """Gradients of <o, d_o> + <S_T, d_final_state> through kda_chunk_fwd's
    recurrence.  Returns dict dq, dk, dg [B,T,H,dk], dv [B,T,H,dv], dbeta
    [B,T,H] and d_initial_state [B,H,dk,dv] (fp32; the last None if not wanted).
    flags: KDA_FLAG_CHECK_RANGE, KDA_FLAG_TOKEN_BACKWARD (token-level path).
    Without a workspace one is allocated: for segments of `segment_tokens`
    tokens when given (chunked path; the call then runs the sequence in
    segments), else for the whole sequence."""
    B, T, H, dk, dv = _check_prefill(q, k, v, beta, initial_state, None, None, workspace, g=g,
                                     d_o=d_o, d_final_state=d_final_state)
    if g is None or d_o is None:
        raise ValueError("g and d_o are required")
    _dev(q, k, v, g, beta, initial_state, d_o, d_final_state, workspace)
    dt = _dtype_code(q)
    f32 = dict(device=q.device, dtype=torch.float32)
    out = dict(dq=torch.empty(B, T, H, dk, **f32), dk=torch.empty(B, T, H, dk, **f32),
               dv=torch.empty(B, T, H, dv, **f32), dg=torch.empty(B, T, H, dk, **f32),
               dbeta=torch.empty(B, T, H, **f32),
               d_initial_state=torch.empty(B, H, dk, dv, **f32) if want_d_initial_state else None)
    if workspace is None:
        ws_bytes = (kda_chunk_bwd_workspace_size(B, T, H, dk, dv, dt) if segment_tokens is None
                    else kda_chunk_bwd_workspace_size_flags(B, T, H, dk, dv, dt, flags,
                                                            segment_tokens))
        workspace = torch.empty(max(ws_bytes, 256), device=q.device, dtype=torch.uint8)
    _check(load_library().kda_chunk_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(d_o),
        _ptr(d_final_state), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
        _ptr(out["dbeta"]), _ptr(out["d_initial_state"]), _ptr(workspace),
        workspace.numel() * workspace.element_size(), B, T, H, dk, dv, dt, flags,
        _stream(stream)))
    return out


def kda_gate_bwd_workspace_size(B: int, T: int, H: int, dk: int) -> int:
    return int(load_library().kda_gate_bwd_workspace_size(B, T, H, dk))


def kda_gate_bwd(z, A, dg, workspace=None, stream=None) -> dict:
    """Reverse mode of kda_gate: dz [B,T,H,dk] and dA [H,dk] (fp32) of <g, dg>."""
    _rank("z", z, 4)
    B, T, H, dk = z.shape
    _in_dtype("z", z)
    _expect("A", A, (H, dk), torch.float32)
    _expect("dg", dg, (B, T, H, dk), torch.float32)
    _workspace(workspace)
    _same_device(z, A, dg, workspace)
    _dev(z, A, dg, workspace)
    f32 = dict(device=z.device, dtype=torch.float32)
    out = dict(dz=torch.empty(B, T, H, dk, **f32), dA=torch.empty(H, dk, **f32))
    if workspace is None:
        workspace = torch.empty(max(kda_gate_bwd_workspace_size(B, T, H, dk), 256),
                                device=z.device, dtype=torch.uint8)
    _check(load_library().kda_gate_bwd(
        _ptr(z), _ptr(A), _ptr(dg), _ptr(out["dz"]), _ptr(out["dA"]), _ptr(workspace),
        workspace.numel() * workspace.element_size(), B, T, H, dk, _dtype_code(z),
        _stream(stream)))
    return out
