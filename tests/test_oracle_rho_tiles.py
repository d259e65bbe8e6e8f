"""Pins of the parity metric `oracle.rho` and of `oracle.tile_log_decay_sums`.

rho is the bar behind every GPU parity assertion: max|x - ref| / max|ref| over
the whole tensor.  Hand-built arrays with answers worked out by hand pin it, so
a changed denominator (a sum of magnitudes, a mean, |ref| at the deviation's
position), a missing absolute value or a silently broadcast shape fails here.

tile_log_decay_sums checks the pages' bound on each 16-token tile's cumulative
log-decay ("Kimi K3 internal structure analysis", section "Sequence mixing:
3 KDA layers per global MLA layer": the floor g >= -5 keeps every 16-token
tile's sum inside (-80, 0)).  Tiles are aligned to token 0 of the sequence and
the last one may be partial.  A g whose tile sums are known in closed form
(an arithmetic series in the token index, scaled per batch, head and channel)
pins it, so a strided regrouping, a dropped tail or a transposed axis fails.
"""
import numpy as np
import pytest

import oracle


# --------------------------------------------------------------------------- rho

def test_rho_hand_example():
    ref = np.array([[1.0, -4.0], [2.0, 0.0]])
    x = ref.copy()
    x[1, 0] += 0.5                       # |dev| 0.5 at an entry of magnitude 2
    assert oracle.rho(x, ref) == pytest.approx(0.125, abs=0)   # 0.5 / max|ref| = 0.5 / 4


def test_rho_negative_deviation_and_position():
    ref = np.array([[1.0, -4.0], [2.0, 0.0]])
    x = ref.copy()
    x[1, 1] -= 0.5                       # deviation where ref is 0, and negative
    assert oracle.rho(x, ref) == 0.125
    x = ref.copy()
    x[0, 0] -= 0.25
    x[0, 1] += 0.125                     # the largest deviation wins, not the last or the sum
    assert oracle.rho(x, ref) == 0.0625


def test_rho_is_relative_to_the_reference_only():
    ref = np.array([3.0, -1.0, 0.5])
    x = np.array([3.0, -1.0, 3.5])       # x's own magnitude (3.5) must not enter the denominator
    assert oracle.rho(x, ref) == 1.0
    assert oracle.rho(ref, x) == pytest.approx(3.0 / 3.5, abs=0)


def test_rho_exact_and_scale_invariant():
    rng = np.random.default_rng(5)
    ref = rng.standard_normal((3, 7, 2))
    assert oracle.rho(ref, ref) == 0.0
    x = ref + 1e-3 * rng.standard_normal(ref.shape)
    r = oracle.rho(x, ref)
    assert oracle.rho(1024.0 * x, 1024.0 * ref) == pytest.approx(r, rel=1e-15)


def test_rho_zero_reference_gives_absolute_error():
    ref = np.zeros((2, 3))
    x = np.zeros((2, 3))
    x[1, 2] = -0.75
    assert oracle.rho(x, ref) == 0.75
    assert oracle.rho(ref, ref) == 0.0


def test_rho_nan_fails_any_tolerance():
    ref = np.ones(4)
    x = ref.copy()
    x[2] = np.nan
    r = oracle.rho(x, ref)
    assert not (r <= 1e-2)
    r = oracle.rho(ref, x)
    assert not (r <= 1e-2)


def test_rho_rejects_shape_mismatch():
    ref = np.ones((1, 1, 4, 3))
    with pytest.raises(ValueError, match="shapes differ"):
        oracle.rho(np.ones((2, 5, 4, 3)), ref)          # would broadcast silently
    with pytest.raises(ValueError, match="shapes differ"):
        oracle.rho(np.ones((4, 3)), ref)


def test_rho_accepts_torch_bf16():
    torch = pytest.importorskip("torch")
    ref = np.array([0.5, -2.0])
    x = torch.tensor([0.5, -1.5], dtype=torch.bfloat16)   # exact in bf16
    assert oracle.rho(x, ref) == 0.25


# ---------------------------------------------------------------- tile sums

def _series_g(B, T, H, dk):
    """g[b,t,h,c] = -(t+1) * s[b,h,c] with a distinct scale per (b, h, c)."""
    t = np.arange(T, dtype=np.float64)
    s = np.empty((B, H, dk))
    for b in range(B):
        for h in range(H):
            for c in range(dk):
                s[b, h, c] = 1e-3 * (1 + c) * (1 + 7 * b + 13 * h)
    g = -(t[None, :, None, None] + 1.0) * s[:, None, :, :]
    return g, s


def _series_tile_sum(first, last, scale):
    """Sum over t = first..last of -(t+1) * scale (arithmetic series)."""
    n = last - first + 1
    return -scale * n * (first + 1 + last + 1) / 2.0


@pytest.mark.parametrize("T", [16, 45, 64, 100])
def test_tile_sums_closed_form(T):
    B, H, dk = 2, 3, 4
    g, s = _series_g(B, T, H, dk)
    got = oracle.tile_log_decay_sums(g)
    nt = (T + 15) // 16
    assert got.shape == (B, nt, H, dk)
    for b in range(B):
        for j in range(nt):
            first, last = 16 * j, min(16 * j + 15, T - 1)      # aligned to token 0; tail partial
            for h in range(H):
                for c in range(dk):
                    want = _series_tile_sum(first, last, s[b, h, c])
                    assert got[b, j, h, c] == pytest.approx(want, rel=1e-13), (b, j, h, c)


def test_tile_sums_tiles_start_mid_chunk():
    """Tile 1 covers tokens 16..31 and tile 5 tokens 80..95: neither starts a
    32- or 64-token chunk.  A one-hot g at token 17 only and token 95 only
    lands in exactly those tiles."""
    g = np.zeros((1, 100, 1, 2))
    g[0, 17, 0, 0] = -3.0
    g[0, 95, 0, 1] = -2.0
    g[0, 96, 0, 1] = -1.0          # first token of the partial tail tile (96..99)
    got = oracle.tile_log_decay_sums(g)
    want = np.zeros((1, 7, 1, 2))
    want[0, 1, 0, 0] = -3.0
    want[0, 5, 0, 1] = -2.0
    want[0, 6, 0, 1] = -1.0
    np.testing.assert_array_equal(got, want)


def test_tile_sums_floor_gives_minus_80():
    """g = -5 (the floor) everywhere: every full tile sums to exactly -80, the
    partial tail to -5 per token."""
    T = 16 * 3 + 5
    g = np.full((1, T, 2, 3), -5.0)
    got = oracle.tile_log_decay_sums(g)
    assert np.all(got[:, :3] == -80.0)
    assert np.all(got[:, 3] == -25.0)


def test_tile_sums_other_tile_length():
    g, s = _series_g(1, 10, 1, 1)
    got = oracle.tile_log_decay_sums(g, tile=4)
    want = [_series_tile_sum(0, 3, s[0, 0, 0]), _series_tile_sum(4, 7, s[0, 0, 0]),
            _series_tile_sum(8, 9, s[0, 0, 0])]
    np.testing.assert_allclose(got[0, :, 0, 0], want, rtol=1e-14)


# ------------------------------------------------------- rho in pieces

def test_rho_accumulator_equals_whole_tensor_rho():
    rng = np.random.default_rng(9)
    ref = rng.standard_normal((2, 50, 3, 4))
    ref[1, 33, 2, 1] = 7.0                      # max|ref| in one piece ...
    x = ref + 1e-5 * rng.standard_normal(ref.shape)
    x[0, 2, 0, 0] += 0.05                       # ... the largest deviation in another
    for cuts in ([0, 50], [0, 7, 8, 33, 34, 50], [0, 25, 50]):
        acc = oracle.RhoAccumulator()
        for a, b in zip(cuts[:-1], cuts[1:]):
            acc.add(x[:, a:b], ref[:, a:b])
        assert acc.value() == oracle.rho(x, ref)
    assert oracle.rho(x, ref) == pytest.approx(0.05 / 7.0, rel=1e-2)


def test_rho_accumulator_nan_zero_and_shapes():
    acc = oracle.RhoAccumulator()
    acc.add(np.zeros(3), np.zeros(3))
    acc.add(np.array([0.0, 0.5]), np.zeros(2))
    assert acc.value() == 0.5                  # all-zero reference: absolute deviation
    acc.add(np.array([np.nan]), np.ones(1))
    assert not (acc.value() <= 1e-2)
    with pytest.raises(ValueError, match="shapes differ"):
        oracle.RhoAccumulator().add(np.ones((2, 3)), np.ones((1, 3)))


def test_decode_step_inplace_equals_copy():
    rng = np.random.default_rng(11)
    N, H, dk, dv = 3, 2, 8, 5
    args = [rng.standard_normal((N, H, dk)), rng.standard_normal((N, H, dk)),
            rng.standard_normal((N, H, dv)), rng.standard_normal((N, H, dk)),
            rng.standard_normal((H, dk)), rng.random((N, H))]
    S = rng.standard_normal((N, H, dk, dv))
    o1, S1 = oracle.decode_step(*args, S)
    S2 = S.copy()
    o2, S2r = oracle.decode_step(*args, S2, inplace=True)
    assert S2r is S2
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)
    assert not np.array_equal(S, S1)            # the copying form left its input alone
