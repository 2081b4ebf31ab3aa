"""Pins of the float64 RoPE oracle (interleaved pairs, host inv-freq table)."""
import math

import numpy as np
import pytest

from oracle import rope as R

RNG = np.random.default_rng(99)


def test_inv_freq_values():
    """theta^(-2i/d): first entry 1; d = 64, theta = 1e4 -> entry 16 is
    1e4^(-1/2) = 0.01; strictly decreasing; float32 storage."""
    t = R.inv_freq(64, 1e4)
    assert t.dtype == np.float32 and t.shape == (32,)
    assert t[0] == 1.0
    assert t[16] == np.float32(0.01)
    assert np.all(np.diff(t.astype(np.float64)) < 0)
    t2 = R.inv_freq(4, 16.0)
    np.testing.assert_array_equal(t2, np.array([1.0, 0.25], np.float32))
    with pytest.raises(ValueError):
        R.inv_freq(5, 1e4)


def test_hand_computed_pair():
    """d = 2, table [1]: position 1 rotates (1, 0) to (cos 1, sin 1) and
    (0, 1) to (-sin 1, cos 1); position 0 is the identity."""
    table = np.array([1.0], np.float32)
    x = np.array([[[1.0, 0.0], [1.0, 0.0]], [[0.0, 1.0], [0.0, 1.0]]])  # [2, T=2, 2]
    y = R.rope(x, table)
    np.testing.assert_allclose(y[0, 0], [1.0, 0.0], atol=1e-15)
    np.testing.assert_allclose(y[0, 1], [math.cos(1), math.sin(1)], atol=1e-15)
    np.testing.assert_allclose(y[1, 1], [-math.sin(1), math.cos(1)], atol=1e-15)


def test_matches_complex_rotation():
    """(x[2i] + 1j x[2i+1]) * exp(1j * angle) -- numpy complex arithmetic."""
    B, H, T, d = 2, 3, 17, 8
    x = RNG.standard_normal((B, H, T, d))
    table = R.inv_freq(d, 1e4)
    y = R.rope(x, table)
    ang = (np.arange(T, dtype=np.float32)[:, None] * table[None, :]).astype(np.float64)
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * ang)
    np.testing.assert_allclose(y[..., 0::2], z.real, atol=1e-13)
    np.testing.assert_allclose(y[..., 1::2], z.imag, atol=1e-13)


def test_float32_angle_reading():
    """The angle is the float32 product of position and table entry."""
    table = R.inv_freq(8, 1e6)
    a = R.angles(8192, table)
    assert a.dtype == np.float32
    assert a[8191, 1] == np.float32(np.float32(8191.0) * table[1])


def test_identity_at_position_zero_and_norms():
    x = RNG.standard_normal((2, 2, 9, 16))
    y = R.rope(x, R.inv_freq(16, 1e4))
    np.testing.assert_allclose(y[:, :, 0], x[:, :, 0], atol=0)
    n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n1 = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(n0, n1, rtol=1e-13)


def test_backward_inverts_and_is_adjoint():
    x = RNG.standard_normal((2, 3, 33, 16))
    yv = RNG.standard_normal((2, 3, 33, 16))
    table = R.inv_freq(16, 1e6)
    np.testing.assert_allclose(R.rope_bwd(R.rope(x, table), table), x, atol=1e-13)
    lhs = (R.rope(x, table) * yv).sum()
    rhs = (x * R.rope_bwd(yv, table)).sum()
    assert abs(lhs - rhs) < 1e-10


def test_relative_position_property():
    """<R_m q, R_n k> = <q, R_(n-m) k>; a power-of-two table keeps the
    float32 angles exact so the identity holds to rounding."""
    d, T = 8, 40
    table = np.array([1.0, 0.5, 0.25, 0.125], np.float32)
    q = RNG.standard_normal(d)
    k = RNG.standard_normal(d)
    Q = R.rope(np.broadcast_to(q, (T, d)).copy(), table)
    K = R.rope(np.broadcast_to(k, (T, d)).copy(), table)
    for m, n in [(3, 10), (0, 39), (17, 20), (25, 25)]:
        assert abs(Q[m] @ K[n] - q @ K[n - m]) < 1e-12


def test_llama3_identity_cases():
    """factor 1 blends a frequency with itself; factor 0 is "off"."""
    plain = R.inv_freq(128, 5e5)
    np.testing.assert_array_equal(R.inv_freq_llama3(128, 5e5, 1.0), plain)
    np.testing.assert_array_equal(R.inv_freq_llama3(128, 5e5, 0.0), plain)


def test_llama3_bands():
    """High-frequency band unchanged, low-frequency band divided by factor,
    blend in between strictly between the two."""
    d, theta, factor, low, high, old = 128, 5e5, 32.0, 1.0, 4.0, 8192.0
    base = theta ** (-2.0 * np.arange(d // 2) / d)
    got = R.inv_freq_llama3(d, theta, factor, low, high, old).astype(np.float64)
    wavelen = 2 * np.pi / base
    hi = wavelen < old / high
    lo = wavelen > old / low
    mid = ~hi & ~lo
    assert hi.any() and lo.any() and mid.any()
    np.testing.assert_allclose(got[hi], base[hi], rtol=1e-7)
    np.testing.assert_allclose(got[lo], base[lo] / factor, rtol=1e-7)
    assert np.all(got[mid] < base[mid]) and np.all(got[mid] > base[mid] / factor)
    assert np.all(np.diff(got) < 0)


def test_llama3_blend_is_continuous_at_thresholds():
    """At wavelen = old/high the blend equals the unchanged frequency; at
    wavelen = old/low it equals inv/factor."""
    old, low, high, factor = 8192.0, 1.0, 4.0, 8.0
    for wl, want_div in ((old / high * (1 + 1e-12), 1.0), (old / low * (1 - 1e-12), factor)):
        inv = np.array([2 * np.pi / wl])
        got = R._llama3_scale(inv, factor, low, high, old)[0]
        assert abs(got - inv[0] / want_div) / inv[0] < 1e-9


def test_layer_rope_theta_gemma3():
    thetas = [R.layer_rope_theta(l, 1e4, 1e6, 6) for l in range(12)]
    assert thetas == [1e4] * 5 + [1e6] + [1e4] * 5 + [1e6]
    assert [R.layer_rope_theta(l, 1e4, 0.0, 6) for l in range(6)] == [1e4] * 6
