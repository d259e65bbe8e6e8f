"""fp64 oracle: ctypes wrapper of kda_oracle.c plus a NumPy twin.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")

# Gate floor and tile length ("Kimi K3 internal structure analysis", section
# "Sequence mixing: 3 KDA layers per global MLA layer": gmin = -5; the
# cumulative log-decay of a 16-token tile stays inside (-80, 0)).
GMIN = -5.0
TILE = 16

_lib_handle = None


def build_oracle(force: bool = True) -> str:
    """Compile kda_oracle.c into libkda_oracle.so with gcc (fp64, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_LIB):
            build_oracle(force=True)
        L = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        L.kda_oracle_gate.argtypes = [dp, dp, dp, i64, i64, i64, i64]
        L.kda_oracle_gate.restype = None
        L.kda_oracle_forward.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp,
                                         i64, i64, i64, i64, i64, i64, ctypes.c_int]
        L.kda_oracle_forward.restype = None
        L.kda_oracle_decode_step.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp,
                                             i64, i64, i64, i64]
        L.kda_oracle_decode_step.restype = None
        L.kda_oracle_max_threads.argtypes = []
        L.kda_oracle_max_threads.restype = ctypes.c_int
        _lib_handle = L
    return _lib_handle


def _f64(x) -> np.ndarray:
    """Any tensor/array -> C-contiguous float64 numpy array (exact for bf16/fp32)."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return int(_lib().kda_oracle_max_threads())


def rho(x, ref) -> float:
    """Parity metric max|x - ref| / max|ref| over the whole tensor: the largest
    absolute deviation, relative to the largest magnitude of the reference.

    The two must have the same shape (no broadcasting: a reference for one
    chain must not be compared against a whole batch).  An all-zero reference
    gives the absolute deviation; a NaN anywhere gives NaN, which fails every
    `<=` tolerance check."""
    x = _f64(x)
    ref = _f64(ref)
    if x.shape != ref.shape:
        raise ValueError(f"rho: shapes differ: {x.shape} vs reference {ref.shape}")
    if ref.size == 0:
        return 0.0
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(x - ref)))
    if np.isnan(den) or np.isnan(num):
        return float("nan")
    if den == 0.0:
        return num
    return num / den


class RhoAccumulator:
    """rho of a tensor compared in pieces (token windows, chain by chain): the
    running max|x - ref| and max|ref| over every piece seen, so that value()
    equals rho(x, ref) of the whole tensor whatever the split."""

    def __init__(self):
        self.num = 0.0
        self.den = 0.0
        self.nan = False

    def add(self, x, ref) -> None:
        x = _f64(x)
        ref = _f64(ref)
        if x.shape != ref.shape:
            raise ValueError(f"RhoAccumulator: shapes differ: {x.shape} vs reference {ref.shape}")
        if ref.size == 0:
            return
        d = float(np.max(np.abs(x - ref)))
        r = float(np.max(np.abs(ref)))
        if np.isnan(d) or np.isnan(r):
            self.nan = True
            return
        self.num = max(self.num, d)
        self.den = max(self.den, r)

    def value(self) -> float:
        if self.nan:
            return float("nan")
        return self.num if self.den == 0.0 else self.num / self.den


# ----------------------------------------------------------------------------
# C oracle wrappers
# ----------------------------------------------------------------------------

def gate(z, A) -> np.ndarray:
    """g = -5 sigmoid(exp(A) z); z [B,T,H,dk] (or [N,H,dk]), A [H,dk]."""
    z = _f64(z)
    A = _f64(A)
    H, dk = A.shape
    assert z.shape[-1] == dk and z.shape[-2] == H
    rows = int(np.prod(z.shape[:-2])) if z.ndim > 2 else 1
    g = np.empty_like(z)
    _lib().kda_oracle_gate(_ptr(z), _ptr(A), _ptr(g), 1, rows, H, dk)
    return g


def forward(q, k, v, g, beta, S0=None, want_o: bool = True,
            col_block: Optional[int] = None, nthreads: int = 0
            ) -> Tuple[Optional[np.ndarray], np.ndarray]:
    """Token-by-token fp64 recurrence.  Returns (o [B,T,H,dv] or None, S_T [B,H,dk,dv])."""
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    assert q.shape == k.shape == g.shape and v.shape == (B, T, H, dv)
    assert beta.shape == (B, T, H)
    S0 = _f64(S0)
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    o = np.empty((B, T, H, dv)) if want_o else None
    ST = np.empty((B, H, dk, dv))
    if col_block is None:
        col_block = dv
    _lib().kda_oracle_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0),
                              _ptr(o), _ptr(ST), B, T, H, dk, dv, int(col_block),
                              int(nthreads))
    return o, ST


def decode_step(q, k, v, z, A, beta, state, inplace: bool = False
                ) -> Tuple[np.ndarray, np.ndarray]:
    """One decode step.  Returns (o [N,H,dv], new state [N,H,dk,dv]).  Inputs are
    untouched, except that with inplace=True a C-contiguous float64 `state` is
    overwritten with the new state and returned (no copy of a large state)."""
    q, k, v, z, A, beta = (_f64(x) for x in (q, k, v, z, A, beta))
    if inplace:
        if not (isinstance(state, np.ndarray) and state.dtype == np.float64
                and state.flags.c_contiguous):
            raise ValueError("inplace decode_step needs a C-contiguous float64 numpy state")
        S = state
    else:
        S = _f64(state).copy()
    N, H, dk = k.shape
    dv = v.shape[-1]
    o = np.empty((N, H, dv))
    _lib().kda_oracle_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A), _ptr(beta),
                                  _ptr(S), _ptr(o), N, H, dk, dv)
    return o, S


# ----------------------------------------------------------------------------
# NumPy twin (plain loops over tokens; for small cases and cross-checks)
# ----------------------------------------------------------------------------

def _sigmoid_np(x: np.ndarray) -> np.ndarray:
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def gate_np(z, A) -> np.ndarray:
    z = _f64(z)
    A = _f64(A)
    return GMIN * _sigmoid_np(np.exp(A) * z)


def forward_np(q, k, v, g, beta, S0=None) -> Tuple[np.ndarray, np.ndarray]:
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    S0 = _f64(S0)
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else S0[b, h].copy()
            for t in range(T):
                S = np.exp(g[b, t, h])[:, None] * S          # retention first
                u = beta[b, t, h] * (v[b, t, h] - S.T @ k[b, t, h])
                S = S + np.outer(k[b, t, h], u)              # delta-rule write
                o[b, t, h] = S.T @ q[b, t, h]                # post-update read
            ST[b, h] = S
    return o, ST


def decode_step_np(q, k, v, z, A, beta, state) -> Tuple[np.ndarray, np.ndarray]:
    q, k, v, z, beta = (_f64(x) for x in (q, k, v, z, beta))
    S = _f64(state).copy()
    g = gate_np(z, A)
    N, H, dk = k.shape
    dv = v.shape[-1]
    o = np.zeros((N, H, dv))
    for n in range(N):
        for h in range(H):
            Sh = np.exp(g[n, h])[:, None] * S[n, h]
            u = beta[n, h] * (v[n, h] - Sh.T @ k[n, h])
            Sh = Sh + np.outer(k[n, h], u)
            o[n, h] = Sh.T @ q[n, h]
            S[n, h] = Sh
    return o, S


def tile_log_decay_sums(g, tile: int = TILE) -> np.ndarray:
    """Sum of g over each aligned `tile`-token tile, per (b, h, channel).

    g [B,T,H,dk] -> [B, ceil(T/tile), H, dk].  Tiles are aligned to token 0;
    the last tile may be partial.
    """
    g = _f64(g)
    B, T, H, dk = g.shape
    nt = (T + tile - 1) // tile
    pad = nt * tile - T
    if pad:
        g = np.concatenate([g, np.zeros((B, pad, H, dk))], axis=1)
    return g.reshape(B, nt, tile, H, dk).sum(axis=2)


# ----------------------------------------------------------------------------
# Reverse mode of the recurrence (plain loops over tokens, fp64)
# ----------------------------------------------------------------------------

def gate_backward_np(z, A, dg) -> dict:
    """Gradients of L = <g, dg> through the gate g = -5 sigmoid(x), x = exp(A) z
    (the gate of `gate_np`; A [H, dk] is shared by every row of z):
        dz = -5 sigmoid'(x) exp(A) dg
        dA = sum over the rows of z of -5 sigmoid'(x) x dg      (dx/dA = x)
    with sigmoid'(x) = sigmoid(x) sigmoid(-x) = e^{-|x|} / (1 + e^{-|x|})^2,
    written in the form that stays accurate for large |x|.
    Returns dz (the shape of z) and dA [H, dk]."""
    z, A, dg = _f64(z), _f64(A), _f64(dg)
    H, dk = A.shape
    assert z.shape == dg.shape and z.shape[-2:] == (H, dk)
    eA = np.exp(A)
    x = eA * z
    e = np.exp(-np.abs(x))
    t = GMIN * dg * e / (1.0 + e) ** 2
    return dict(dz=t * eA, dA=(t * x).reshape(-1, H, dk).sum(axis=0))


def backward_np(q, k, v, g, beta, S0=None, do=None, dST=None) -> dict:
    """Gradients of L = <o, do> + <S_T, dST> through the token recurrence.

    Each token's step is differentiated as written (retention, delta-rule
    write, post-update read), walking the tokens in reverse:
        dS_t += q_t do_t^T;             dq_t = S_t do_t
        du = dS_t^T k_t;                dk_t = dS_t u_t (+ below)
        dbeta_t = du . (v_t - w);       dv_t = beta_t du;   dw = -beta_t du
        dS' = dS_t + k_t dw^T;          dk_t += S' dw       (w = S'^T k_t)
        da = rowsum(S_{t-1} * dS');     dg_t = a * da       (a = exp(g_t))
        dS_{t-1} = Diag(a) dS'
    Returns dq, dk, dv, dg, dbeta (input shapes) and dS0 [B,H,dk,dv].
    """
    q, k, v, g, beta = (_f64(x) for x in (q, k, v, g, beta))
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    S0 = _f64(S0)
    do = np.zeros((B, T, H, dv)) if do is None else _f64(do)
    dST = None if dST is None else _f64(dST)
    out = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dg", g),
                                            ("dbeta", beta))}
    out["dS0"] = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else S0[b, h].copy()
            states = [S]                                   # states[t] = S before token t
            for t in range(T):
                S = np.exp(g[b, t, h])[:, None] * S
                u = beta[b, t, h] * (v[b, t, h] - S.T @ k[b, t, h])
                S = S + np.outer(k[b, t, h], u)
                states.append(S)
            dS = np.zeros((dk, dv)) if dST is None else dST[b, h].copy()
            for t in range(T - 1, -1, -1):
                a = np.exp(g[b, t, h])
                kt, qt, vt, bt = k[b, t, h], q[b, t, h], v[b, t, h], beta[b, t, h]
                Sp = a[:, None] * states[t]                 # S'
                w = Sp.T @ kt
                u = bt * (vt - w)
                St = states[t + 1]
                dS = dS + np.outer(qt, do[b, t, h])
                out["dq"][b, t, h] = St @ do[b, t, h]
                du = dS.T @ kt
                dkt = dS @ u
                out["dbeta"][b, t, h] = du @ (vt - w)
                out["dv"][b, t, h] = bt * du
                dw = -bt * du
                dSp = dS + np.outer(kt, dw)
                dkt = dkt + Sp @ dw
                out["dk"][b, t, h] = dkt
                da = np.sum(states[t] * dSp, axis=1)
                out["dg"][b, t, h] = a * da
                dS = a[:, None] * dSp
            out["dS0"][b, h] = dS
    return out
