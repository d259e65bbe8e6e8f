"""C-ABI checks that need no GPU: the library loads, exports every function
include/kda.h declares, and host-side validation rejects bad calls with the
documented codes before any HIP call is made (only fake, never-dereferenced
pointers are passed, and every call here fails validation)."""
import ctypes
import os
import re
import subprocess

import pytest

from linear_attention_sequence_gate_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

P = ctypes.c_void_p(0x100000)      # 16-byte aligned fake device addresses
P2 = ctypes.c_void_p(0x200000)
P3 = ctypes.c_void_p(0x300000)
BAD = ctypes.c_void_p(0x100008)    # misaligned
NULL = None


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return _lib.load_library()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("kda_gate", "kda_chunk_fwd", "kda_chunk_fwd_workspace_size",
              "kda_chunk_fwd_workspace_size_segments", "kda_chunk_fwd_auto_segments",
              "kda_chunk_fwd_plan", "kda_decode_step", "kda_state_pool_reset", "kda_chunk_fwd_pooled",
              "kda_chunk_fwd_varlen_pooled", "kda_decode_step_pooled", "kda_chunk_bwd",
              "kda_chunk_bwd_workspace_size", "kda_gate_bwd", "kda_gate_bwd_workspace_size",
              "kda_chunk_fwd_gated", "kda_chunk_fwd_gated_workspace_size",
              "kda_chunk_fwd_varlen_pooled_gated", "kda_chunk_fwd_gated_noalloc",
              "kda_chunk_bwd_workspace_size_flags", "kda_last_error", "kda_version"):
        assert n in names
    assert set(names) == set(_lib.EXPORTED)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (kda_\w+)$", out, flags=re.M))
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(L, n)


def test_version(L):
    assert "gfx950" in _lib.kda_version()


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.load_library(str(tmp_path / "nope.so"))


def chunk(L, q=P, k=P, v=P, g=P, beta=P, S0=NULL, ST=NULL, o=P2, ws=NULL, wsb=0,
          B=1, T=64, H=1, dk=32, dv=32, dt=1, flags=0):
    return L.kda_chunk_fwd(q, k, v, g, beta, S0, ST, o, ws, wsb, B, T, H, dk, dv, dt, flags, None)


def test_chunk_validation(L):
    E = _lib
    assert chunk(L, q=NULL) == E.KDA_ERR_INVALID_ARGUMENT
    assert "null" in _lib.kda_last_error()
    assert chunk(L, o=NULL) == E.KDA_ERR_INVALID_ARGUMENT
    assert chunk(L, T=0) == E.KDA_ERR_INVALID_ARGUMENT
    assert chunk(L, B=-1) == E.KDA_ERR_INVALID_ARGUMENT
    assert chunk(L, dk=48) == E.KDA_ERR_UNSUPPORTED
    assert chunk(L, dv=256) == E.KDA_ERR_UNSUPPORTED
    assert chunk(L, dt=7) == E.KDA_ERR_UNSUPPORTED
    # fp32 with dk = 128: the fp32 16-token path, which needs its per-chunk
    # buffers in the workspace
    assert chunk(L, dt=0, dk=128) == E.KDA_ERR_INVALID_ARGUMENT
    assert "workspace" in _lib.kda_last_error()
    need = L.kda_chunk_fwd_workspace_size(1, 64, 1, 128, 32, 0)
    assert chunk(L, dt=0, dk=128, ws=P3, wsb=need - 1) == E.KDA_ERR_INVALID_ARGUMENT
    assert chunk(L, B=1 << 30, T=1 << 30) == E.KDA_ERR_INVALID_ARGUMENT   # overflow
    assert chunk(L, k=BAD) == E.KDA_ERR_INVALID_ARGUMENT          # misaligned
    assert chunk(L, o=P) == E.KDA_ERR_INVALID_ARGUMENT            # o aliases q
    assert chunk(L, flags=4) == E.KDA_ERR_INVALID_ARGUMENT        # unknown flag
    assert chunk(L, flags=E.KDA_FLAG_WORKGROUP_PER_SLICE << 1) == E.KDA_ERR_INVALID_ARGUMENT
    # one workgroup per chain: the pipelined path at dk = dv = 128 only, not
    # with the position-pair path, and not together with the per-slice layout
    both = E.KDA_FLAG_WORKGROUP_PER_CHAIN | E.KDA_FLAG_WORKGROUP_PER_SLICE
    assert chunk(L, flags=both) == E.KDA_ERR_INVALID_ARGUMENT
    assert "exclude" in _lib.kda_last_error()
    assert chunk(L, flags=E.KDA_FLAG_WORKGROUP_PER_CHAIN) == E.KDA_ERR_UNSUPPORTED   # dk = 32
    assert "per chain" in _lib.kda_last_error()
    assert chunk(L, dk=128, dv=64, flags=E.KDA_FLAG_WORKGROUP_PER_CHAIN) == E.KDA_ERR_UNSUPPORTED
    assert chunk(L, dk=128, dv=128, flags=E.KDA_FLAG_WORKGROUP_PER_CHAIN |
                 E.KDA_FLAG_PAIRWISE_DIAGONAL) == E.KDA_ERR_UNSUPPORTED
    assert chunk(L, dt=0, dk=128, dv=128, ws=P3,
                 flags=E.KDA_FLAG_WORKGROUP_PER_CHAIN) == E.KDA_ERR_UNSUPPORTED   # fp32
    assert chunk(L, flags=E.KDA_FLAG_TOKEN_BACKWARD) == E.KDA_ERR_INVALID_ARGUMENT   # backward only
    assert chunk(L, flags=E.KDA_FLAG_PAIRWISE_DIAGONAL) == E.KDA_ERR_UNSUPPORTED   # dk = 32
    assert "position-pair" in _lib.kda_last_error()
    assert chunk(L, dk=128, dv=128, flags=E.KDA_FLAG_PAIRWISE_DIAGONAL | E.KDA_FLAG_CHECK_RANGE,
                 ws=P3, wsb=4096) == E.KDA_ERR_INVALID_ARGUMENT
    assert chunk(L, flags=1) == E.KDA_ERR_INVALID_ARGUMENT        # range check needs workspace
    assert chunk(L, flags=1, ws=P3, wsb=8) == E.KDA_ERR_INVALID_ARGUMENT  # too small
    assert "workspace" in _lib.kda_last_error()


def test_workspace_query(L):
    assert L.kda_chunk_fwd_workspace_size(1, 64, 1, 32, 32, 1) >= 4
    # fp32 at dk = 128: the counter, then X, P, At (3 x 16 x 16) and the
    # decayed operands (49 dk) of each 16-token chunk, fp32, each rounded
    # up to 256 bytes
    for B, T, H, dv in ((1, 64, 1, 128), (2, 1000, 3, 32)):
        n = B * H * -(-T // 16)
        r256 = lambda x: -(-x // 256) * 256
        want = 256 + r256(n * 768 * 4) + r256(n * 49 * 128 * 4)
        assert L.kda_chunk_fwd_workspace_size(B, T, H, 128, dv, 0) == want
        assert L.kda_chunk_fwd_workspace_size_segments(B, T, H, 128, dv, 0, 1) == want
        assert L.kda_chunk_fwd_gated_workspace_size(B, T, H, 128, dv, 0) == want + r256(B * T * H * 128 * 4)
    assert L.kda_chunk_fwd_workspace_size(1, 64, 1, 48, 32, 1) == 0
    assert L.kda_chunk_fwd_workspace_size(0, 64, 1, 32, 32, 1) == 0
    assert L.kda_chunk_fwd_workspace_size(1, 64, 1, 32, 32, 5) == 0


def test_sequence_split_workspace_and_policy(L):
    ws = L.kda_chunk_fwd_workspace_size
    wss = L.kda_chunk_fwd_workspace_size_segments
    auto = L.kda_chunk_fwd_auto_segments

    def split_bytes(B, H, dv, P, scan=False):
        # (P-1) initial states, (P-1) zero-start states, (P-2) transitions,
        # with the log-depth chaining a second buffer of (P-2) transitions,
        # then one int per (segment after the first, chain, 64 transition
        # columns) rounded up to 256 bytes
        vsz, msz = B * H * 128 * dv * 4, B * H * 128 * 128 * 4
        zc = -(-(P - 1) * B * H * 2 * 4 // 256) * 256
        return 256 + 2 * (P - 1) * vsz + (P - 2) * msz + (P - 2) * msz * scan + zc

    # B8 H32 T32K: 256 chains, one workgroup each, fill the GPU in one pass
    assert auto(8, 32768, 32, 128, 128, 1) == 1
    assert ws(8, 32768, 32, 128, 128, 1) == 256
    # B4 H32 T32K: 128 chains; two segments of each fill the GPU with one
    # workgroup per chain and segment (cheaper than 256 workgroups of 64
    # columns in one pass, which form every chunk's operands twice)
    assert auto(4, 32768, 32, 128, 128, 1) == 2
    assert ws(4, 32768, 32, 128, 128, 1) == split_bytes(4, 32, 128, 2)
    # B1 H32 T1M: 32 chains; the split takes eight segments (the stopping
    # split: the v workgroups of all segments in one round)
    P = auto(1, 1 << 20, 32, 128, 128, 1)
    assert P == 8, P
    # the automatic workspace covers the count of either scheme and layout
    assert ws(1, 1 << 20, 32, 128, 128, 1) >= split_bytes(1, 32, 128, P)
    assert ws(1, 1 << 20, 32, 128, 128, 1) in [split_bytes(1, 32, 128, n) for n in range(P, 17)]
    assert wss(1, 1 << 20, 32, 128, 128, 1, 0) == ws(1, 1 << 20, 32, 128, 128, 1)
    assert wss(1, 1 << 20, 32, 128, 128, 1, P) == split_bytes(1, 32, 128, P)
    # one chain: many more segments
    P1 = auto(1, 1 << 20, 1, 128, 128, 1)
    assert P1 > 4 * P, (P1, P)
    assert ws(1, 1 << 20, 1, 128, 128, 1) >= wss(1, 1 << 20, 1, 128, 128, 1, P1)
    # 129 segments of one chain are chained by the log-depth scan, which
    # takes a second buffer of transitions; 9 segments serially
    assert wss(1, 1 << 20, 1, 128, 128, 1, 129) == split_bytes(1, 1, 128, 129, scan=True)
    assert wss(1, 1 << 20, 1, 128, 128, 1, 9) == split_bytes(1, 1, 128, 9)
    # few chains of a short sequence split too (segments of >= 128 tokens):
    # B1 H8 T4096 runs 16 workgroups in one pass
    P8 = auto(1, 4096, 8, 128, 128, 1)
    assert 3 <= P8 <= 32, P8
    assert wss(1, 4096, 8, 128, 128, 1, P8) == split_bytes(1, 8, 128, P8)
    assert ws(1, 4096, 8, 128, 128, 1) >= split_bytes(1, 8, 128, P8)
    # 64 and 128 chains: four and two segments fill the GPU
    assert auto(8, 4096, 8, 128, 128, 1) == 4
    assert auto(16, 4096, 8, 128, 128, 1) == 2
    # enough chains to fill the GPU, or too short to split: one pass
    assert auto(32, 4096, 8, 128, 128, 1) == 1
    assert auto(1, 383, 1, 128, 128, 1) == 1 and ws(1, 383, 1, 128, 128, 1) == 256
    # shapes without the pipelined kernel run in one pass
    assert auto(1, 1 << 20, 1, 64, 64, 1) == 1
    assert auto(1, 1 << 20, 1, 32, 32, 0) == 1
    assert auto(0, 64, 1, 128, 128, 1) == 0
    assert wss(1, 4096, 2, 32, 32, 0, 4) == 256           # fp32: no split path
    assert wss(1, 4096, 2, 128, 128, 1, 1) == 256         # 1 = never split
    # explicit counts: the 32-token-aligned segment length decides how many
    assert wss(1, 1000, 2, 128, 64, 1, 3) == split_bytes(1, 2, 64, 3)   # 352 + 352 + 296
    assert wss(1, 64, 2, 128, 64, 1, 3) == split_bytes(1, 2, 64, 2)     # two 32-token segments
    assert wss(1, 1000, 2, 128, 64, 1, 256) == 0


def test_sequence_split_validation(L):
    E = _lib
    seg3 = _lib.kda_flag_segments(3)
    # fp32 or dk != 128 have no split path
    assert chunk(L, flags=seg3) == E.KDA_ERR_UNSUPPORTED
    assert "split" in _lib.kda_last_error()
    # an explicit split needs its workspace
    assert chunk(L, dk=128, dv=128, T=4096, flags=seg3) == E.KDA_ERR_INVALID_ARGUMENT
    assert "workspace" in _lib.kda_last_error()
    assert chunk(L, dk=128, dv=128, T=4096, flags=seg3, ws=P3, wsb=256) == E.KDA_ERR_INVALID_ARGUMENT


def test_gate_validation(L):
    E = _lib
    assert L.kda_gate(NULL, P, P2, 1, 1, 1, 32, 1, None) == E.KDA_ERR_INVALID_ARGUMENT
    assert L.kda_gate(P, P3, P2, 1, 1, 1, 40, 1, None) == E.KDA_ERR_UNSUPPORTED
    assert L.kda_gate(P, P3, P2, 1, 0, 1, 32, 1, None) == E.KDA_ERR_INVALID_ARGUMENT
    assert L.kda_gate(P, P3, P2, 1, 1, 1, 32, 9, None) == E.KDA_ERR_UNSUPPORTED
    assert L.kda_gate(P, P3, P, 1, 1, 1, 32, 1, None) == E.KDA_ERR_INVALID_ARGUMENT   # g aliases z
    assert L.kda_gate(BAD, P3, P2, 1, 1, 1, 32, 1, None) == E.KDA_ERR_INVALID_ARGUMENT


def test_decode_validation(L):
    E = _lib

    def dec(q=P, k=P, v=P, z=P, A=P3, beta=P, S=P3, o=P2, N=4, H=2, dk=32, dv=32, dt=1):
        return L.kda_decode_step(q, k, v, z, A, beta, S, o, N, H, dk, dv, dt, None)

    assert dec(S=NULL) == E.KDA_ERR_INVALID_ARGUMENT
    assert dec(N=0) == E.KDA_ERR_INVALID_ARGUMENT
    assert dec(dv=96) == E.KDA_ERR_UNSUPPORTED
    assert dec(dt=3) == E.KDA_ERR_UNSUPPORTED
    assert dec(o=P) == E.KDA_ERR_INVALID_ARGUMENT
    assert dec(z=BAD) == E.KDA_ERR_INVALID_ARGUMENT
    assert dec(N=1 << 40, H=1 << 30) == E.KDA_ERR_INVALID_ARGUMENT


def test_pool_validation(L):
    E = _lib
    S4 = ctypes.c_void_p(0x10004)          # 4-byte aligned, not 16
    reset = lambda pool=P, slots=P3, n=2, ns=4, H=1, dk=32, dv=32: L.kda_state_pool_reset(
        pool, slots, n, ns, H, dk, dv, None)
    assert reset(pool=NULL) == E.KDA_ERR_INVALID_ARGUMENT
    assert reset(slots=NULL) == E.KDA_ERR_INVALID_ARGUMENT
    assert reset(ns=0) == E.KDA_ERR_INVALID_ARGUMENT
    assert reset(n=0) == E.KDA_ERR_INVALID_ARGUMENT
    assert reset(dk=48) == E.KDA_ERR_UNSUPPORTED
    assert reset(pool=BAD) == E.KDA_ERR_INVALID_ARGUMENT
    assert reset(slots=ctypes.c_void_p(0x10002)) == E.KDA_ERR_INVALID_ARGUMENT
    assert reset(ns=1 << 40, H=1 << 20) == E.KDA_ERR_INVALID_ARGUMENT   # overflow
    dec = lambda pool=P, slots=S4, o=P2, N=2, ns=4: L.kda_decode_step_pooled(
        P, P, P, P, P, P, pool, slots, o, N, ns, 1, 32, 32, 1, None)
    assert dec(pool=NULL) == E.KDA_ERR_INVALID_ARGUMENT
    assert dec(ns=-1) == E.KDA_ERR_INVALID_ARGUMENT
    assert dec(o=S4) == E.KDA_ERR_INVALID_ARGUMENT                        # o aliases slots
    ch = lambda pool=P, slots=S4, o=P2, ns=4: L.kda_chunk_fwd_pooled(
        P, P, P, P, P, pool, slots, o, NULL, 0, 1, 64, ns, 1, 32, 32, 1, 0, None)
    assert ch(slots=NULL) == E.KDA_ERR_INVALID_ARGUMENT
    assert ch(ns=0) == E.KDA_ERR_INVALID_ARGUMENT
    assert ch(o=P) == E.KDA_ERR_INVALID_ARGUMENT                          # o aliases the pool
    # fp32 at dk = 128 (the fp32 16-token path) needs its workspace here too;
    # the packed call does not take it
    assert L.kda_chunk_fwd_pooled(P, P, P, P, P, P3, S4, P2, NULL, 0, 1, 64, 4, 1, 128, 32, 0, 0,
                                  None) == E.KDA_ERR_INVALID_ARGUMENT
    assert "workspace" in _lib.kda_last_error()

    vl = lambda cu=P3, dk=128, dv=128, dt=1, flags=0, pool=P, o=P2: L.kda_chunk_fwd_varlen_pooled(
        P, P, P, P, P, pool, S4, cu, o, 2, 100, 4, 1, dk, dv, dt, flags, None)
    assert vl(cu=NULL) == E.KDA_ERR_INVALID_ARGUMENT
    assert vl(cu=ctypes.c_void_p(0x300004)) == E.KDA_ERR_INVALID_ARGUMENT   # not 8-byte aligned
    assert vl(dk=64) == E.KDA_ERR_UNSUPPORTED
    assert vl(dt=0, dv=32) == E.KDA_ERR_UNSUPPORTED                       # fp32, dk = 128
    assert vl(dt=0) == E.KDA_ERR_UNSUPPORTED
    assert vl(flags=E.KDA_FLAG_CHECK_RANGE) == E.KDA_ERR_INVALID_ARGUMENT
    assert vl(flags=_lib.kda_flag_segments(3)) == E.KDA_ERR_INVALID_ARGUMENT
    assert vl(o=P) == E.KDA_ERR_INVALID_ARGUMENT                           # o aliases the pool


def test_backward_validation(L):
    E = _lib
    # the range-check counter, then the larger of the two paths' buffers:
    # token path = state checkpoints every 8 tokens per 32-column slice plus,
    # with several slices, their partial row gradients (dq, dk, dg, dbeta);
    # chunked path = the state entering each even 16-token chunk and the
    # gradient leaving each odd (or last) one, three 16x16 matrices and the
    # decayed operands (81 dk floats) per chunk, and W, dU per token
    def chunked(nbh, T, dk, dv):
        r = lambda x: (x + 255) // 256 * 256
        nc = (T + 15) // 16
        npair = (nc + 1) // 2
        return (2 * r(nbh * npair * dk * dv * 4) + r(nbh * nc * 768 * 4) + 2 * r(nbh * nc * 16 * dv * 4)
                + r(nbh * nc * 49 * dk * 4))
    assert chunked(1, 64, 32, 32) > 8 * 32 * 32 * 4
    assert L.kda_chunk_bwd_workspace_size(1, 64, 1, 32, 32, 1) == 256 + chunked(1, 64, 32, 32)
    token = 2 * 3 * 2 * 128 * 64 * 4 + 2 * (2 * 9 * 3) * (3 * 128 + 1) * 4
    assert L.kda_chunk_bwd_workspace_size(2, 9, 3, 128, 64, 0) == 256 + max(token, chunked(6, 9, 128, 64))
    assert L.kda_chunk_bwd_workspace_size(1, 64, 1, 48, 32, 1) == 0
    Q = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(16)]
    bwd = lambda ws=Q[14], wsb=1 << 20, dq=Q[8], T=64, dk=32, dt=1, S0=None, flags=0: L.kda_chunk_bwd(
        Q[0], Q[1], Q[2], Q[3], Q[4], S0, Q[6], None, dq, Q[9], Q[10], Q[11], Q[12], None,
        ws, wsb, 1, T, 1, dk, 32, dt, flags, None)
    assert bwd(flags=4) == E.KDA_ERR_INVALID_ARGUMENT
    assert bwd(flags=E.KDA_FLAG_SPLIT_FULL_RERUN) == E.KDA_ERR_INVALID_ARGUMENT   # prefill only
    assert "flag" in _lib.kda_last_error()
    assert bwd(flags=E.KDA_FLAG_TOKEN_BACKWARD | E.KDA_FLAG_CHECK_RANGE) == E.KDA_ERR_INVALID_ARGUMENT
    assert bwd(dq=NULL) == E.KDA_ERR_INVALID_ARGUMENT
    assert bwd(ws=NULL) == E.KDA_ERR_INVALID_ARGUMENT
    assert bwd(wsb=100) == E.KDA_ERR_INVALID_ARGUMENT
    assert "workspace" in _lib.kda_last_error()
    assert bwd(dk=48) == E.KDA_ERR_UNSUPPORTED
    assert bwd(dt=5) == E.KDA_ERR_UNSUPPORTED
    assert bwd(T=0) == E.KDA_ERR_INVALID_ARGUMENT
    assert bwd(dq=Q[0]) == E.KDA_ERR_INVALID_ARGUMENT         # output aliases q
    assert bwd(S0=BAD) == E.KDA_ERR_INVALID_ARGUMENT          # misaligned


def test_backward_segmented_workspace(L):
    """The chunked reverse mode runs in segments when the workspace holds less
    than the whole sequence: one segment's buffers plus the states entering
    segments 1 .. n-1 and two gradient carries, [B*H, dk, dv] fp32 each."""
    E = _lib
    r = lambda x: (x + 255) // 256 * 256

    def seg_bytes(nbh, T, dk, dv):
        nc = (T + 15) // 16
        npair = (nc + 1) // 2
        return (2 * r(nbh * npair * dk * dv * 4) + r(nbh * nc * 768 * 4) + 2 * r(nbh * nc * 16 * dv * 4)
                + r(nbh * nc * 49 * dk * 4))

    q = L.kda_chunk_bwd_workspace_size_flags
    B, T, H, dk, dv = 2, 1000, 3, 64, 32
    nbh, state = B * H, B * H * dk * dv * 4
    whole = q(B, T, H, dk, dv, 1, 0, 0)
    assert whole == 256 + seg_bytes(nbh, T, dk, dv)
    for seg, nseg in ((64, 16), (100, 8), (500, 2), (992, 2)):       # rounded up to 32 tokens
        s32 = (seg + 31) // 32 * 32
        assert q(B, T, H, dk, dv, 1, 0, seg) == 256 + seg_bytes(nbh, s32, dk, dv) + (nseg - 1 + 2) * state
    assert q(B, T, H, dk, dv, 1, 0, 1000) == whole                   # one segment
    mn = q(B, T, H, dk, dv, 1, 0, E.KDA_BWD_SEGMENTS_MIN_WORKSPACE)
    assert mn < whole
    assert all(mn <= q(B, T, H, dk, dv, 1, 0, 32 * u) for u in range(1, 32))
    # the token path ignores the segment length and takes its whole-sequence size
    tok = q(B, T, H, dk, dv, 1, E.KDA_FLAG_TOKEN_BACKWARD, 0)
    assert tok == q(B, T, H, dk, dv, 1, E.KDA_FLAG_TOKEN_BACKWARD, 64)
    assert L.kda_chunk_bwd_workspace_size(B, T, H, dk, dv, 1) == max(tok, whole)
    assert q(B, T, H, dk, dv, 1, 0, -2) == 0
    # B1 H32 T1M d128: about 230 GB in one segment, under 8 GB in 32768-token ones
    assert q(1, 1 << 20, 32, 128, 128, 1, 0, 0) > 200e9
    assert q(1, 1 << 20, 32, 128, 128, 1, 0, 32768) < 8e9
    assert q(1, 1 << 20, 32, 128, 128, 1, 0, E.KDA_BWD_SEGMENTS_MIN_WORKSPACE) < 2e9
    # kda_chunk_bwd rejects less than the least any segment length needs
    Q = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(16)]
    rc = L.kda_chunk_bwd(Q[0], Q[1], Q[2], Q[3], Q[4], None, Q[6], None, Q[8], Q[9], Q[10], Q[11],
                         Q[12], None, Q[14], mn - 1, B, T, H, dk, dv, 1, 0, None)
    assert rc == E.KDA_ERR_INVALID_ARGUMENT
    assert "workspace" in _lib.kda_last_error()


def test_gate_backward_validation(L):
    E = _lib
    # per-row-range shares of dA: about 1024 workgroups of 256 columns, at most
    # 256 ranges, at most one per row
    assert L.kda_gate_bwd_workspace_size(4, 4096, 32, 128) == 64 * 32 * 128 * 4
    assert L.kda_gate_bwd_workspace_size(1, 3, 1, 32) == 3 * 32 * 4
    assert L.kda_gate_bwd_workspace_size(2, 500, 1, 32) == 256 * 32 * 4
    assert L.kda_gate_bwd_workspace_size(1, 64, 1, 48) == 0
    Q = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(8)]
    gb = lambda z=Q[0], dz=Q[3], dA=Q[4], ws=Q[5], wsb=1 << 20, dk=32, dt=1: L.kda_gate_bwd(
        z, Q[1], Q[2], dz, dA, ws, wsb, 2, 8, 1, dk, dt, None)
    assert gb(z=NULL) == E.KDA_ERR_INVALID_ARGUMENT
    assert gb(ws=NULL) == E.KDA_ERR_INVALID_ARGUMENT
    assert gb(wsb=4) == E.KDA_ERR_INVALID_ARGUMENT
    assert "workspace" in _lib.kda_last_error()
    assert gb(dk=48) == E.KDA_ERR_UNSUPPORTED
    assert gb(dt=7) == E.KDA_ERR_UNSUPPORTED
    assert gb(dz=Q[2]) == E.KDA_ERR_INVALID_ARGUMENT         # dz aliases dg
    assert gb(dA=Q[3]) == E.KDA_ERR_INVALID_ARGUMENT         # dA aliases dz
    assert gb(z=BAD) == E.KDA_ERR_INVALID_ARGUMENT           # misaligned


def gated(L, q=P, k=P, v=P, z=P3, A=P2, beta=P, S0=NULL, ST=NULL, o=ctypes.c_void_p(0x400000),
          ws=NULL, wsb=0, B=1, T=64, H=1, dk=128, dv=128, dt=1, flags=0):
    return L.kda_chunk_fwd_gated(q, k, v, z, A, beta, S0, ST, o, ws, wsb, B, T, H, dk, dv, dt, flags,
                                 None)


def test_gated_validation(L):
    """kda_chunk_fwd_gated: host validation before any HIP call (every call
    here fails, so no fake pointer is dereferenced)."""
    E = _lib
    assert gated(L, z=NULL) == E.KDA_ERR_INVALID_ARGUMENT
    assert "z and A" in _lib.kda_last_error()
    assert gated(L, A=NULL) == E.KDA_ERR_INVALID_ARGUMENT
    assert gated(L, q=NULL) == E.KDA_ERR_INVALID_ARGUMENT
    assert gated(L, z=BAD) == E.KDA_ERR_INVALID_ARGUMENT              # misaligned z
    assert gated(L, o=P3) == E.KDA_ERR_INVALID_ARGUMENT               # o aliases z
    assert gated(L, o=P2) == E.KDA_ERR_INVALID_ARGUMENT               # o aliases A
    assert gated(L, dt=7) == E.KDA_ERR_UNSUPPORTED
    assert gated(L, dk=48) == E.KDA_ERR_UNSUPPORTED
    assert gated(L, dt=0) == E.KDA_ERR_INVALID_ARGUMENT               # fp32, dk = 128: no workspace
    # the range check takes a caller's g; here g is the gate's own output
    assert gated(L, flags=E.KDA_FLAG_CHECK_RANGE, ws=ctypes.c_void_p(0x500000),
                 wsb=1 << 20) == E.KDA_ERR_INVALID_ARGUMENT
    assert "CHECK_RANGE" in _lib.kda_last_error()
    # shapes without the fused kernel stage g in the workspace: none, or too
    # small, is rejected before the gate runs
    assert gated(L, dk=64, dv=64) == E.KDA_ERR_INVALID_ARGUMENT
    assert gated(L, dk=64, dv=64, ws=ctypes.c_void_p(0x500000), wsb=1024) == E.KDA_ERR_INVALID_ARGUMENT
    assert "workspace" in _lib.kda_last_error()
    # the workspace may not be a tensor
    assert gated(L, dk=64, dv=64, ws=P, wsb=1 << 20) == E.KDA_ERR_INVALID_ARGUMENT


def test_gated_workspace_query(L):
    q = L.kda_chunk_fwd_gated_workspace_size
    base = L.kda_chunk_fwd_workspace_size
    # fused shapes: exactly what kda_chunk_fwd takes (range counter, split buffers)
    assert q(8, 32768, 32, 128, 128, 1) == base(8, 32768, 32, 128, 128, 1) == 256
    assert q(4, 32768, 32, 128, 128, 1) == base(4, 32768, 32, 128, 128, 1) > 256
    assert q(1, 1 << 20, 32, 128, 128, 1) == base(1, 1 << 20, 32, 128, 128, 1) > 256
    # staged shapes: g (B T H dk fp32, rounded to 256 bytes) in front
    assert q(2, 100, 3, 64, 64, 1) == 256 + (2 * 100 * 3 * 64 * 4 + 255) // 256 * 256
    assert q(1, 7, 1, 32, 32, 0) == 256 + 1024          # 7*32*4 = 896 -> 1024
    assert q(0, 64, 1, 128, 128, 1) == 0 and q(1, 64, 1, 48, 128, 1) == 0


def test_varlen_pooled_gated_validation(L):
    E = _lib
    f = L.kda_chunk_fwd_varlen_pooled_gated
    cu, pool, slots, o = (ctypes.c_void_p(a) for a in (0x600000, 0x700000, 0x800000, 0x900000))
    args = lambda z=P3, A=P2, cu_=cu, dk=128, dv=128, flags=0: (
        P, P, P, z, A, P, pool, slots, cu_, o, 2, 100, 4, 1, dk, dv, 1, flags, None)
    assert f(*args(z=NULL)) == E.KDA_ERR_INVALID_ARGUMENT
    assert f(*args(cu_=NULL)) == E.KDA_ERR_INVALID_ARGUMENT
    assert f(*args(dk=64, dv=64)) == E.KDA_ERR_UNSUPPORTED             # fused shapes only
    assert f(*args(flags=E.KDA_FLAG_CHECK_RANGE)) == E.KDA_ERR_INVALID_ARGUMENT


def test_binding_constants_match_the_header():
    """The binding's error codes and flag bits are the values include/kda.h
    gives them."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    header = {n: int(v.rstrip("u"), 0)
              for n, v in re.findall(r"\b(KDA_(?:OK|ERR_\w+|FLAG_\w+))\s*=\s*(-?\w+)", text)}
    assert len(header) >= 11, header
    for n, v in header.items():
        assert getattr(_lib, n) == v, n


def test_chunk_plan(L):
    """The plan the chunked prefill follows: segments and workgroup layout
    for the library's choice and under each flag (host only)."""
    E = _lib
    plan = _lib.kda_chunk_fwd_plan
    CH, SL, seg = E.KDA_FLAG_WORKGROUP_PER_CHAIN, E.KDA_FLAG_WORKGROUP_PER_SLICE, E.kda_flag_segments
    # the library's choice agrees with kda_chunk_fwd_auto_segments
    for B, T, H in ((8, 32768, 32), (4, 32768, 32), (1, 1 << 20, 32), (1, 4096, 8), (1, 383, 1)):
        P, _ = plan(B, T, H, 128, 128, 1)
        assert P == L.kda_chunk_fwd_auto_segments(B, T, H, 128, 128, 1), (B, T, H)
    # 256 chains: one workgroup each, one pass; 128 chains: two segments of each
    assert plan(8, 32768, 32, 128, 128, 1) == (1, True)
    assert plan(4, 32768, 32, 128, 128, 1) == (2, True)
    # one pass forced: 256 slice workgroups beat 128 chain workgroups
    assert plan(4, 32768, 32, 128, 128, 1, seg(1)) == (1, False)
    # forced layouts, with the count chosen for that layout
    assert plan(4, 32768, 32, 128, 128, 1, SL) == (1, False)
    assert plan(4, 32768, 32, 128, 128, 1, CH | seg(1)) == (1, True)
    assert plan(4, 32768, 32, 128, 128, 1, CH | seg(3)) == (3, True)
    # a requested count reports the count its aligned segment length gives
    assert plan(1, 64, 2, 128, 64, 1, seg(3)) == (2, False)
    # per-slice only: dv = 64, the position-pair path, other shapes
    assert plan(4, 32768, 32, 128, 64, 1)[1] is False
    assert plan(4, 32768, 32, 128, 128, 1, E.KDA_FLAG_PAIRWISE_DIAGONAL)[1] is False
    assert plan(4, 32768, 32, 64, 64, 1) == (1, False)
    assert plan(4, 32768, 32, 128, 128, 0) == (1, False)       # fp32
    # rejected as the call rejects them
    with pytest.raises(_lib.KdaError):
        plan(4, 32768, 32, 128, 64, 1, CH)
    with pytest.raises(_lib.KdaError):
        plan(4, 32768, 32, 128, 128, 1, CH | SL)
    with pytest.raises(_lib.KdaError):
        plan(1, 64, 1, 32, 32, 1, seg(3))
    with pytest.raises(_lib.KdaError):
        plan(0, 64, 1, 128, 128, 1)


def test_plan_and_workspace_agree_over_sizes(L):
    """Over a grid of sizes, for the library's choice, each layout flag and
    each split scheme: the plan's count is the automatic count, the
    library's workspace holds the buffers of whatever count a flag set
    leaves to the library, only a two-segment stopping split is guarded, and
    the per-chain layout appears only where it is supported (host only)."""
    E = _lib
    CH, SL, RR = E.KDA_FLAG_WORKGROUP_PER_CHAIN, E.KDA_FLAG_WORKGROUP_PER_SLICE, E.KDA_FLAG_SPLIT_FULL_RERUN
    for B in (1, 2, 4, 8, 16):
        for H in (1, 8, 32):
            for T in (64, 1000, 4096, 32768, 1 << 20):
                for dv in (64, 128):
                    if B * H * T > (1 << 24) * 4:
                        continue
                    ws = L.kda_chunk_fwd_workspace_size(B, T, H, 128, dv, 1)
                    P0 = L.kda_chunk_fwd_auto_segments(B, T, H, 128, dv, 1)
                    for fl in (0, RR, SL, SL | RR) + ((CH, CH | RR) if dv == 128 else ()):
                        P, wide, guarded = E.kda_chunk_fwd_plan(B, T, H, 128, dv, 1, fl, with_guard=True)
                        if fl == 0:
                            assert P == P0, (B, T, H, dv)
                        assert 1 <= P <= 255
                        assert not wide or dv == 128
                        assert not guarded or (P == 2 and not fl & RR), (B, T, H, dv, fl)
                        need = L.kda_chunk_fwd_workspace_size_segments(B, T, H, 128, dv, 1, P)
                        assert need <= ws, (B, T, H, dv, fl, P, need, ws)
