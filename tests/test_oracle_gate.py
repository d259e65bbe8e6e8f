"""Pins of the oracle's gate and of the 16-token tile bound (CPU only).

Page: "Kimi K3 internal structure analysis", section "Sequence mixing: 3 KDA
layers per global MLA layer": g = gmin * sigmoid(exp(A) * z), alpha = exp(g),
gmin = -5; the floor keeps a 16-token tile's cumulative log-decay in (-80, 0),
inside bf16's dynamic range.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
from linear_attention_sequence_gate_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


@pytest.mark.parametrize("impl", ["c", "np"])
def test_gate_at_zero_is_half_floor(impl):
    z = np.zeros((1, 3, 2, 8))
    A = _rand((2, 8), 1)
    f = oracle.gate if impl == "c" else oracle.gate_np
    g = f(z, A)
    # sigmoid(0) = 1/2 exactly, so g = -2.5 exactly whatever A is
    assert np.all(g == -2.5)


@pytest.mark.parametrize("impl", ["c", "np"])
def test_gate_reflection(impl):
    # sigmoid(x) + sigmoid(-x) = 1  =>  g(z) + g(-z) = gmin
    z = _rand((2, 5, 3, 16), 2, 3.0)
    A = _rand((3, 16), 3, 0.5)
    f = oracle.gate if impl == "c" else oracle.gate_np
    s = f(z, A) + f(-z, A)
    np.testing.assert_allclose(s, -5.0, rtol=0, atol=4e-15)


@pytest.mark.parametrize("impl", ["c", "np"])
def test_gate_against_library_sigmoid(impl):
    # A = 0 reduces the gate to -5 * expit(z); A = ln 2 doubles the argument.
    z = _rand((1, 7, 2, 32), 4, 4.0)
    f = oracle.gate if impl == "c" else oracle.gate_np
    np.testing.assert_allclose(f(z, np.zeros((2, 32))), -5.0 * expit(z), rtol=2e-15, atol=1e-300)
    A = np.full((2, 32), math.log(2.0))
    np.testing.assert_allclose(f(z, A), -5.0 * expit(2.0 * z), rtol=4e-15, atol=1e-300)
    # per-head, per-channel A: channel c of head h uses A[h, c]
    A = _rand((2, 32), 5, 0.5)
    ref = -5.0 * expit(np.exp(A)[None, None] * z)
    np.testing.assert_allclose(f(z, A), ref, rtol=4e-15, atol=1e-300)


def test_gate_range_and_monotone():
    z = np.linspace(-60, 60, 4001).reshape(1, -1, 1, 1)
    A = np.array([[0.3]])
    g = oracle.gate(z, A).ravel()
    assert np.all(g <= 0.0) and np.all(g >= -5.0)
    assert np.all(np.diff(g) <= 0.0)           # non-increasing in z
    assert g[0] > -1e-20 and g[-1] == -5.0       # the ends reach 0 and the floor


def test_gate_c_matches_numpy():
    z = _rand((2, 33, 3, 64), 6, 2.0)
    A = _rand((3, 64), 7, 0.5)
    np.testing.assert_allclose(oracle.gate(z, A), oracle.gate_np(z, A), rtol=4e-15, atol=0)


def test_pages_constants_fixture():
    with open(os.path.join(GOLDEN, "kda_pages_constants.json")) as f:
        c = json.load(f)
    assert oracle.GMIN == c["gmin"]["value"]
    assert oracle.TILE == c["tile_tokens"]["value"]
    lo, hi = c["tile_log_decay_interval"]["value"]
    assert lo == oracle.GMIN * oracle.TILE and hi == 0.0


def test_tile_bound_fits_bf16_range():
    fi = torch.finfo(torch.bfloat16)
    lo = oracle.GMIN * oracle.TILE
    assert math.exp(-lo) < fi.max                  # e^80 representable
    assert math.exp(lo) > fi.tiny                  # e^-80 is a normal number
    # a masked-out entry of a diagonal tile with unit q, k (|sum| <= d * e^80) stays finite
    assert 128 * math.exp(-lo) < fi.max
    f32 = torch.finfo(torch.float32)
    assert 128 * math.exp(-lo) < f32.max


@pytest.mark.parametrize("name", ["small_f32", "prefill_h8_t4k", "prefill_b4_h32_t32k",
                                  "prefill_h32_t1m", "decode_256x32"])
def test_tile_bound_on_workload_gates(name):
    """Every aligned 16-token tile sum of the gate lies in [-80, 0] (closed: in
    fp64 sigmoid rounds to 1 for large arguments, so the floor is reached)."""
    w = inputs.WORKLOADS[name]
    T = min(w.T, 512) if w.T > 1 else 64
    H = min(w.H, 32)
    x = inputs.make_prefill_inputs(1, T, H, w.dk, w.dv, w.dtype, w.seed,
                                   stress_heads_mean=w.stress_heads_mean)
    g = oracle.gate(x["z"], x["A"])
    sums = oracle.tile_log_decay_sums(g)
    assert np.all(sums <= 0.0) and np.all(sums >= -80.0)
    if w.stress_heads_mean is not None:
        # the stress heads push tiles close to the bound
        assert sums[:, :, H // 2:].min() < -79.0
