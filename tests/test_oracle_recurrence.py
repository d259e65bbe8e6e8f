"""Pins of the oracle's recurrence (CPU only).

Page: "Kimi K3 internal structure analysis", section "Sequence mixing: 3 KDA
layers per global MLA layer" -- a fixed-size state updated by the delta rule,
with a channel-wise retention applied before the current key/value pair is
written; "Infrastructure for a 3T-class MoE" -- a segment acts on its incoming
state through an affine transition, and transitions compose associatively.

Each test pins the oracle to something other than itself: a closed form, an
explicit product of the transition matrices, or an invariant.
"""
import numpy as np
import pytest

import oracle


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _problem(B, T, H, dk, dv, seed, s0=True, gscale=1.0):
    r = np.random.default_rng(seed)
    q = _unit(r.standard_normal((B, T, H, dk)))
    k = _unit(r.standard_normal((B, T, H, dk)))
    v = r.standard_normal((B, T, H, dv))
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((B, T, H))))
    z = r.standard_normal((B, T, H, dk)) * gscale
    A = r.standard_normal((H, dk)) * 0.5
    g = oracle.gate_np(z, A)
    S0 = r.standard_normal((B, H, dk, dv)) * 0.3 if s0 else None
    return q, k, v, g, beta, S0


IMPLS = {"c": oracle.forward, "np": oracle.forward_np}


@pytest.mark.parametrize("impl", ["c", "np"])
def test_beta_zero_is_pure_decay(impl):
    """beta = 0 writes nothing: S_t = Diag(exp(b_t)) S0, o_t = S0^T (exp(b_t) * q_t),
    with b_t the running sum of g up to and including t."""
    q, k, v, g, beta, S0 = _problem(1, 37, 2, 8, 5, 11)
    beta = np.zeros_like(beta)
    o, ST = IMPLS[impl](q, k, v, g, beta, S0)
    b = np.cumsum(g, axis=1)                                    # [B,T,H,dk]
    ref_o = np.einsum("bthc,bhcn->bthn", np.exp(b) * q, S0)
    ref_S = np.exp(b[:, -1])[..., None] * S0
    np.testing.assert_allclose(o, ref_o, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(ST, ref_S, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("impl", ["c", "np"])
def test_one_hot_keys_give_gated_cumulative_sum(impl):
    """Distinct one-hot keys and a zero initial state: every write lands in its own
    row, nothing is predicted, so row c_s of S_T = beta_s exp(b_{T,c_s} - b_{s,c_s}) v_s
    (the gated cumulative sum of k v^T)."""
    T, dk, dv = 12, 16, 7
    r = np.random.default_rng(12)
    perm = r.permutation(dk)[:T]
    k = np.zeros((1, T, 1, dk))
    k[0, np.arange(T), 0, perm] = 1.0
    q = _unit(r.standard_normal((1, T, 1, dk)))
    v = r.standard_normal((1, T, 1, dv))
    beta = r.uniform(0.1, 0.9, (1, T, 1))
    g = -r.uniform(0.0, 5.0, (1, T, 1, dk))
    o, ST = IMPLS[impl](q, k, v, g, beta, None)
    b = np.cumsum(g[0, :, 0], axis=0)                           # [T, dk]
    ref = np.zeros((dk, dv))
    for s, c in enumerate(perm):
        ref[c] = beta[0, s, 0] * np.exp(b[T - 1, c] - b[s, c]) * v[0, s, 0]
    np.testing.assert_allclose(ST[0, 0], ref, rtol=1e-13, atol=1e-16)
    # and each output reads the rows written so far
    for t in range(T):
        St = np.zeros((dk, dv))
        for s, c in enumerate(perm[: t + 1]):
            St[c] = beta[0, s, 0] * np.exp(b[t, c] - b[s, c]) * v[0, s, 0]
        np.testing.assert_allclose(o[0, t, 0], St.T @ q[0, t, 0], rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("impl", ["c", "np"])
def test_overwrite_with_orthonormal_keys(impl):
    """alpha = 1 (g = 0), beta = 1, orthonormal keys: writing (k_i, v) replaces the
    value stored under k_i exactly and leaves the other slots alone."""
    dk, dv = 8, 5
    r = np.random.default_rng(13)
    Qm, _ = np.linalg.qr(r.standard_normal((dk, dk)))
    keys = Qm.T                                                  # rows orthonormal
    order = [0, 1, 2, 3, 1, 4, 0, 2]                             # rewrites slots 0, 1, 2
    T = len(order)
    k = keys[order][None, :, None, :]
    v = r.standard_normal((1, T, 1, dv))
    q = np.broadcast_to(keys[0], (1, T, 1, dk)).copy()
    g = np.zeros((1, T, 1, dk))
    beta = np.ones((1, T, 1))
    S0 = r.standard_normal((1, 1, dk, dv))
    o, ST = IMPLS[impl](q, k, v, g, beta, S0)
    S = ST[0, 0]
    last = {}
    for t, i in enumerate(order):
        last[i] = v[0, t, 0]
    for i in range(dk):
        want = last[i] if i in last else S0[0, 0].T @ keys[i]
        np.testing.assert_allclose(S.T @ keys[i], want, rtol=0, atol=2e-14)
    # q = keys[0]: output t reads the value most recently written to slot 0
    cur = S0[0, 0].T @ keys[0]
    for t, i in enumerate(order):
        if i == 0:
            cur = v[0, t, 0]
        np.testing.assert_allclose(o[0, t, 0], cur, rtol=0, atol=2e-14)


@pytest.mark.parametrize("impl", ["c", "np"])
@pytest.mark.parametrize("T", [1, 2, 5, 8])
def test_brute_force_unrolled_products(impl, T):
    """S_T = Phi_{T,0} S0 + sum_s Phi_{T,s} beta_s k_s v_s^T with
    Phi_{T,s} = M_T ... M_{s+1},  M_r = (I - beta_r k_r k_r^T) Diag(alpha_r),
    all formed as explicit dk x dk matrices; o_t = S_t^T q_t.  dk != dv so a
    transposed operand cannot pass."""
    dk, dv = 6, 4
    q, k, v, g, beta, S0 = _problem(2, T, 2, dk, dv, 100 + T)
    o, ST = IMPLS[impl](q, k, v, g, beta, S0)
    I = np.eye(dk)
    for b in range(2):
        for h in range(2):
            M = [(I - beta[b, r, h] * np.outer(k[b, r, h], k[b, r, h])) @ np.diag(np.exp(g[b, r, h]))
                 for r in range(T)]
            for t in range(T):
                Phi = I.copy()
                terms = []
                for s in range(t, -1, -1):          # Phi_{t,s}: product of M_t..M_{s+1}
                    terms.append(Phi @ (beta[b, s, h] * np.outer(k[b, s, h], v[b, s, h])))
                    Phi = Phi @ M[s]
                St = Phi @ S0[b, h] + sum(terms)
                np.testing.assert_allclose(o[b, t, h], St.T @ q[b, t, h], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(ST[b, h], St, rtol=1e-12, atol=1e-14)


def test_norm_bound():
    """|I - beta k k^T| <= 1 for beta |k|^2 <= 2 and alpha <= 1, so
    ||S_t||_F <= ||S_{t-1}||_F + beta_t ||k_t|| ||v_t||."""
    q, k, v, g, beta, S0 = _problem(1, 64, 1, 16, 16, 21)
    prev = np.linalg.norm(S0[0, 0])
    S = S0
    for t in range(64):
        _, S = oracle.forward(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], g[:, t:t + 1],
                              beta[:, t:t + 1], S)
        cur = np.linalg.norm(S[0, 0])
        bound = prev + beta[0, t, 0] * np.linalg.norm(k[0, t, 0]) * np.linalg.norm(v[0, t, 0])
        assert cur <= bound * (1 + 1e-12)
        prev = cur


def test_split_invariance_is_bitwise():
    """Running T tokens equals running T1 tokens, handing over the state, and
    running the rest (the fixed-size state is the whole carry)."""
    q, k, v, g, beta, S0 = _problem(2, 50, 3, 8, 6, 22)
    o, ST = oracle.forward(q, k, v, g, beta, S0)
    for T1 in (1, 17, 49):
        o1, S1 = oracle.forward(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], S0)
        o2, S2 = oracle.forward(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:], S1)
        assert np.array_equal(np.concatenate([o1, o2], axis=1), o)
        assert np.array_equal(S2, ST)


def test_column_blocks_do_not_change_results():
    q, k, v, g, beta, S0 = _problem(1, 40, 2, 8, 12, 23)
    o, ST = oracle.forward(q, k, v, g, beta, S0)
    for cb in (1, 5, 8):
        o2, S2 = oracle.forward(q, k, v, g, beta, S0, col_block=cb)
        assert np.array_equal(o, o2) and np.array_equal(ST, S2)


def test_affine_segment_transitions_compose():
    """S_T(S0) = M S0 + L with M = run(S0 = I, v = 0) and L = run(S0 = 0); two
    segments compose as (M2 M1, M2 L1 + L2)."""
    dk, dv, T = 8, 5, 30
    q, k, v, g, beta, S0 = _problem(1, T, 1, dk, dv, 24)

    def ML(sl):
        _, M = oracle.forward(q[:, sl], k[:, sl], np.zeros((1, sl.stop - sl.start, 1, dk)),
                              g[:, sl], beta[:, sl], np.eye(dk)[None, None])
        _, L = oracle.forward(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl], None)
        return M[0, 0], L[0, 0]

    _, ST = oracle.forward(q, k, v, g, beta, S0)
    M, L = ML(slice(0, T))
    np.testing.assert_allclose(M @ S0[0, 0] + L, ST[0, 0], rtol=1e-12, atol=1e-14)
    M1, L1 = ML(slice(0, 13))
    M2, L2 = ML(slice(13, T))
    np.testing.assert_allclose(M2 @ M1, M, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(M2 @ L1 + L2, L, rtol=1e-12, atol=1e-14)


def test_c_and_numpy_agree():
    q, k, v, g, beta, S0 = _problem(2, 70, 3, 32, 16, 25)
    o1, S1 = oracle.forward(q, k, v, g, beta, S0)
    o2, S2 = oracle.forward_np(q, k, v, g, beta, S0)
    assert oracle.rho(o1, o2) <= 1e-13 and oracle.rho(S1, S2) <= 1e-13


def test_decode_steps_equal_prefill():
    """Applying decode_step token by token (gate fused) equals the forward run
    on the gate's output: the state is the only carry (fixed-size state)."""
    N, H, dk, dv, T = 3, 2, 16, 8, 9
    r = np.random.default_rng(26)
    q = _unit(r.standard_normal((N, T, H, dk)))
    k = _unit(r.standard_normal((N, T, H, dk)))
    v = r.standard_normal((N, T, H, dv))
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((N, T, H))))
    z = r.standard_normal((N, T, H, dk))
    A = r.standard_normal((H, dk)) * 0.5
    S0 = r.standard_normal((N, H, dk, dv)) * 0.02
    g = oracle.gate(z, A)
    o_ref, S_ref = oracle.forward(q, k, v, g, beta, S0)
    S = S0.copy()
    S_np = S0.copy()
    for t in range(T):
        o, S = oracle.decode_step(q[:, t], k[:, t], v[:, t], z[:, t], A, beta[:, t], S)
        o_np, S_np = oracle.decode_step_np(q[:, t], k[:, t], v[:, t], z[:, t], A, beta[:, t], S_np)
        np.testing.assert_allclose(o, o_ref[:, t], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(o_np, o, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(S, S_ref, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(S_np, S, rtol=1e-13, atol=1e-15)
