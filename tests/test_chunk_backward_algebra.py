"""The chunked reverse mode's equations, in fp64 NumPy, against the oracle's
token-level reverse mode (CPU only).

The GPU backward evaluates the recurrence's reverse mode chunk by chunk
(16-token chunks, pair factors referenced to the chunk's middle token, the
gradient of that reference dropped because it cancels, and snapshots of
every other chunk with the missing states formed from their neighbours).
This test writes those equations out on their own and checks that they
reach the same gradients as `oracle.backward_np`, so an error in the
derivation (a sign, a transposed operand, a missing decay term) fails here
on the CPU, independently of the kernels."""
import numpy as np
import pytest

import oracle

C = 16


def _chunks(x, T):
    nc = (T + C - 1) // C
    pad = nc * C - T
    return np.concatenate([x, np.zeros((pad,) + x.shape[1:])], 0), nc


def chunked_backward(q, k, v, g, beta, S0, dO, dST, mid=7):
    T, dk = q.shape
    (q, nc), (k, _), (v, _), (g, _), (beta, _), (dO, _) = (
        _chunks(a, T) for a in (q, k, v, g, beta, dO))
    pre = []
    for c in range(nc):
        sl = slice(c * C, c * C + C)
        b = np.cumsum(g[sl], 0)
        m, bC = b[mid], b[-1]
        d = dict(sl=sl, b=b, m=m, bC=bC, bt=beta[sl], q=q[sl], k=k[sl])
        d["Qt"], d["Kt"], d["Kh"] = q[sl] * np.exp(b), k[sl] * np.exp(b), k[sl] * np.exp(bC - b)
        d["Qp"], d["Kp"], d["Kpp"] = q[sl] * np.exp(b - m), k[sl] * np.exp(b - m), k[sl] * np.exp(m - b)
        d["At"] = d["Kp"] @ d["Kpp"].T
        A = np.tril(d["bt"][:, None] * d["At"], -1)
        d["X"] = np.linalg.inv(np.eye(C) + A)
        d["P"] = np.tril(d["Qp"] @ d["Kpp"].T)
        pre.append(d)
    # forward pass: snapshots of the state entering every even chunk, W of all
    S = S0.copy()
    snapS, W = {}, {}
    for c, d in enumerate(pre):
        if c % 2 == 0:
            snapS[c // 2] = S.copy()
        W[c] = v[d["sl"]] - d["Kt"] @ S
        U = d["X"] @ (d["bt"][:, None] * W[c])
        S = np.exp(d["bC"])[:, None] * S + d["Kh"].T @ U
    # reverse pass: snapshots of the gradient leaving every odd (or the last) chunk
    dN = dST.copy()
    snapN, dU = {}, {}
    for c in reversed(range(nc)):
        d = pre[c]
        if c % 2 == 1 or c == nc - 1:
            snapN[c // 2] = dN.copy()
        dU[c] = d["P"].T @ dO[d["sl"]] + d["Kh"] @ dN
        dW = d["bt"][:, None] * (d["X"].T @ dU[c])
        dN = np.exp(d["bC"])[:, None] * dN + d["Qt"].T @ dO[d["sl"]] - d["Kt"].T @ dW
    dS0 = dN
    # token gradients, chunk pairs: the missing state and gradient formed from the neighbour
    out = {n: np.zeros((nc * C, dk)) for n in ("dq", "dk", "dg")}
    out["dv"], out["dbeta"] = np.zeros((nc * C, v.shape[1])), np.zeros(nc * C)
    for p in range((nc + 1) // 2):
        c0, c1 = 2 * p, 2 * p + 1
        states = {c0: snapS[p]}
        grads = {}
        if c1 < nc:
            d0, d1 = pre[c0], pre[c1]
            U0 = d0["X"] @ (d0["bt"][:, None] * W[c0])
            states[c1] = np.exp(d0["bC"])[:, None] * snapS[p] + d0["Kh"].T @ U0
            grads[c1] = snapN[p]
            dW1 = d1["bt"][:, None] * (d1["X"].T @ dU[c1])
            grads[c0] = (np.exp(d1["bC"])[:, None] * snapN[p] + d1["Qt"].T @ dO[d1["sl"]]
                         - d1["Kt"].T @ dW1)
        else:
            grads[c0] = snapN[p]
        for c in states:
            d, Sc, dNc, sl = pre[c], states[c], grads[c], pre[c]["sl"]
            X, bt = d["X"], d["bt"]
            U = X @ (bt[:, None] * W[c])
            dWc = bt[:, None] * (X.T @ dU[c])
            out["dv"][sl] = dWc
            dT = dU[c] @ W[c].T
            dX = dT * bt[None, :]
            dbeta = (X * dT).sum(0)
            dA = np.tril(-X.T @ dX @ X.T, -1)
            dbeta += (dA * d["At"]).sum(1)
            dAt = bt[:, None] * dA
            dP = np.tril(dO[sl] @ U.T)
            dQp, dKp = dP @ d["Kpp"], dAt @ d["Kpp"]
            dKpp = dAt.T @ d["Kp"] + dP.T @ d["Qp"]
            dQt, dKt, dKh = dO[sl] @ Sc.T, -dWc @ Sc.T, U @ dNc.T
            b, m, bC = d["b"], d["m"], d["bC"]
            out["dq"][sl] = dQt * np.exp(b) + dQp * np.exp(b - m)
            out["dk"][sl] = (dKt * np.exp(b) + dKh * np.exp(bC - b) + dKp * np.exp(b - m)
                             + dKpp * np.exp(m - b))
            db = (dQt * d["Qt"] + dKt * d["Kt"] - dKh * d["Kh"] + dQp * d["Qp"] + dKp * d["Kp"]
                  - dKpp * d["Kpp"])
            db[-1] += (dKh * d["Kh"]).sum(0) + np.exp(bC) * (Sc * dNc).sum(1)
            out["dg"][sl] = np.cumsum(db[::-1], 0)[::-1]
            out["dbeta"][sl] = dbeta
    out = {n: a[:T] for n, a in out.items()}
    out["dS0"] = dS0
    return out


def _case(seed, T, dk, dv, decay="gate"):
    """decay: "gate" (g = -5 sigmoid(z)), "stress" (z shifted by +3, g near
    the floor) or "weak" (g in [-0.1, 0], so that e^{b_C} of a full chunk
    and every term through it carry weight)."""
    r = np.random.default_rng(seed)
    unit = lambda a: a / np.linalg.norm(a, axis=-1, keepdims=True)
    q, k = unit(r.normal(size=(T, dk))), unit(r.normal(size=(T, dk)))
    v = r.normal(size=(T, dv))
    beta = 1.0 / (1.0 + np.exp(-r.normal(size=T)))
    z = r.normal(size=(T, dk)) + (3.0 if decay == "stress" else 0.0)
    g = (-0.1 if decay == "weak" else -5.0) / (1.0 + np.exp(-z))
    S0 = 0.3 * r.normal(size=(dk, dv))
    return q, k, v, g, beta, S0, r.normal(size=(T, dv)), r.normal(size=(dk, dv))


@pytest.mark.parametrize("T,dk,dv,decay", [(1, 8, 4, "gate"), (16, 8, 8, "gate"), (37, 32, 16, "gate"),
                                           (48, 16, 24, "stress"), (70, 16, 8, "gate"),
                                           (64, 8, 8, "stress"), (32, 16, 8, "weak"),
                                           (45, 8, 16, "weak")])
def test_chunked_reverse_mode_equals_the_token_reverse_mode(T, dk, dv, decay):
    q, k, v, g, beta, S0, dO, dST = _case(T + dk, T, dk, dv, decay)
    got = chunked_backward(q, k, v, g, beta, S0, dO, dST)
    e = lambda a: a[None, :, None]
    ref = oracle.backward_np(e(q), e(k), e(v), e(g), beta[None, :, None], S0[None, None], e(dO),
                             dST[None, None])
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        r = ref[name][0, :, 0]
        err = np.max(np.abs(got[name] - r)) / max(np.max(np.abs(r)), 1e-300)
        assert err < 1e-11, (name, err)
    err = np.max(np.abs(got["dS0"] - ref["dS0"][0, 0])) / np.max(np.abs(ref["dS0"]))
    assert err < 1e-11, ("dS0", err)


def test_the_mid_reference_gradient_cancels():
    """m = b_7 appears in K', Q', K" only through e^{b_r - m} e^{m - b_s}: its
    gradient, -sum(dQ'Q' + dK'K') + sum(dK"K"), is zero, so the kernels drop it."""
    q, k, v, g, beta, S0, dO, dST = _case(5, 16, 8, 8)
    b = np.cumsum(g, 0)
    m = b[7]
    Qp, Kp, Kpp = q * np.exp(b - m), k * np.exp(b - m), k * np.exp(m - b)
    r = np.random.default_rng(6)
    dP = np.tril(r.normal(size=(16, 16)))
    dAt = np.tril(r.normal(size=(16, 16)), -1)
    dQp, dKp = dP @ Kpp, dAt @ Kpp
    dKpp = dAt.T @ Kp + dP.T @ Qp
    dm = -(dQp * Qp + dKp * Kp).sum(0) + (dKpp * Kpp).sum(0)
    assert np.max(np.abs(dm)) < 1e-12 * np.max(np.abs(dKpp * Kpp))
