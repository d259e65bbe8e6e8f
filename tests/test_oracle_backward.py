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
