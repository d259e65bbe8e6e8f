"""Pins of the oracle's reverse mode (`backward_np`) against central finite
differences of the fp64 forward recurrence on tiny inputs (brute force: every
input element), and against special cases with closed forms."""
import numpy as np
import pytest

import oracle


def _case(seed, B=1, T=6, H=2, dk=4, dv=3, s0=True):
    r = np.random.default_rng(seed)
    q = r.normal(size=(B, T, H, dk))
    k = r.normal(size=(B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.normal(size=(B, T, H, dv))
    g = -5.0 * r.uniform(size=(B, T, H, dk))
    beta = r.uniform(0.1, 0.9, size=(B, T, H))
    S0 = r.normal(scale=0.3, size=(B, H, dk, dv)) if s0 else None
    do = r.normal(size=(B, T, H, dv))
    dST = r.normal(size=(B, H, dk, dv))
    return dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0), do, dST


def _loss(x, do, dST):
    o, ST = oracle.forward_np(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"])
    return float(np.sum(o * do) + np.sum(ST * dST))


@pytest.mark.parametrize("seed", [0, 1])
def test_backward_matches_central_differences_everywhere(seed):
    x, do, dST = _case(seed)
    grads = oracle.backward_np(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], do, dST)
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "S0": "dS0"}
    h = 1e-6
    for name, gname in names.items():
        fd = np.zeros_like(x[name])
        it = np.nditer(x[name], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            orig = x[name][idx]
            x[name][idx] = orig + h
            lp = _loss(x, do, dST)
            x[name][idx] = orig - h
            lm = _loss(x, do, dST)
            x[name][idx] = orig
            fd[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(fd - grads[gname])) / max(1.0, np.max(np.abs(fd)))
        assert err < 1e-7, (name, err)


def test_backward_zero_initial_state_and_no_state_gradient():
    """S0 = None is a zero start (dS0 is still returned); dST = None means the
    loss reads only o; a change of the last token's v then moves only o_T."""
    x, do, _ = _case(2, s0=False)
    gr = oracle.backward_np(x["q"], x["k"], x["v"], x["g"], x["beta"], None, do, None)
    assert gr["dS0"].shape == (1, 2, 4, 3)
    # the last token's v reaches the loss only through o_T = S_T^T q_T:
    # dv_T = beta_T * (k_T . q_T) * do_T
    T = x["q"].shape[1]
    for hh in range(2):
        kq = x["k"][0, T - 1, hh] @ x["q"][0, T - 1, hh]
        expect = x["beta"][0, T - 1, hh] * kq * do[0, T - 1, hh]
        assert np.allclose(gr["dv"][0, T - 1, hh], expect, rtol=1e-12, atol=1e-14)


def test_backward_beta_zero_is_pure_decay():
    """beta = 0: S_t = Diag(prod alpha) S_0, so dS0 = sum_t Diag(prod_{j<=t} alpha_j) q_t do_t^T
    (+ the final-state term), and dv = 0."""
    x, do, dST = _case(3, T=4, s0=True)
    x["beta"][:] = 0.0
    gr = oracle.backward_np(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], do, dST)
    assert np.all(gr["dv"] == 0.0)
    for hh in range(2):
        a = np.exp(x["g"][0, :, hh])                         # [T, dk]
        cum = np.cumprod(a, axis=0)
        expect = cum[-1][:, None] * dST[0, hh]
        for t in range(4):
            expect = expect + cum[t][:, None] * np.outer(x["q"][0, t, hh], do[0, t, hh])
        assert np.allclose(gr["dS0"][0, hh], expect, rtol=1e-12, atol=1e-14)


# --- the gate's reverse mode ------------------------------------------------

def _gate_case(seed, rows=5, H=2, dk=3):
    r = np.random.default_rng(seed)
    z = r.normal(scale=2.0, size=(rows, H, dk))
    z[0, 0, 0] = 30.0                 # deep in the saturated tail
    z[1, 1, 2] = -25.0
    A = r.normal(scale=0.5, size=(H, dk))
    dg = r.normal(size=(rows, H, dk))
    return z, A, dg


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_gate_backward_matches_central_differences(seed):
    """dz and dA against central differences of <gate(z, A), dg>, with the
    gate from the C oracle (an independent evaluation of the forward)."""
    z, A, dg = _gate_case(seed)
    gr = oracle.gate_backward_np(z, A, dg)
    loss = lambda zz, AA: float(np.sum(oracle.gate(zz[None], AA)[0] * dg))
    h = 1e-6
    for name, x, gx in (("z", z, gr["dz"]), ("A", A, gr["dA"])):
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            orig = x[idx]
            x[idx] = orig + h
            lp = loss(z, A)
            x[idx] = orig - h
            lm = loss(z, A)
            x[idx] = orig
            fd[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(fd - gx)) / max(1.0, np.max(np.abs(fd)))
        assert err < 1e-7, (name, err)


def test_gate_backward_closed_forms():
    """z = 0: sigmoid'(0) = 1/4, so dz = -(5/4) e^A dg and dA = 0 (x = 0).
    A = 0: dz = -5 sigmoid(z) sigmoid(-z) dg.  Large |x|: the derivative
    decays like e^{-|x|} and stays finite."""
    r = np.random.default_rng(7)
    A = r.normal(scale=0.5, size=(2, 4))
    dg = r.normal(size=(3, 2, 4))
    gr = oracle.gate_backward_np(np.zeros((3, 2, 4)), A, dg)
    assert np.allclose(gr["dz"], -1.25 * np.exp(A) * dg, rtol=1e-15, atol=0)
    assert np.all(gr["dA"] == 0.0)
    z = r.normal(scale=3.0, size=(3, 2, 4))
    gr = oracle.gate_backward_np(z, np.zeros((2, 4)), dg)
    s = 1.0 / (1.0 + np.exp(-z))
    assert np.allclose(gr["dz"], -5.0 * s * (1.0 - s) * dg, rtol=1e-12, atol=1e-300)
    gr = oracle.gate_backward_np(np.full((1, 2, 4), 800.0), np.zeros((2, 4)), np.ones((1, 2, 4)))
    assert np.all(np.isfinite(gr["dz"])) and np.all(gr["dz"] <= 0.0)
