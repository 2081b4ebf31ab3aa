"""Pins of the float64 decode oracle: it is the last row of the (separately
pinned) causal attention oracle over the first lens[b] positions, meets
closed forms (zero query, window 1, empty cache), and the split-along-the-
cache merge identity reproduces it exactly."""
import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import decode as D

RNG = np.random.default_rng(4321)


@pytest.fixture(autouse=True)
def _fresh_rng(request):
    """Every test draws from its own seeded stream, so its inputs do not
    depend on which tests ran before it in the same process."""
    global RNG
    name = request.node.name
    RNG = np.random.default_rng(sum((i + 1) * ord(c) for i, c in enumerate(name)))


def _cache(B, H, Hkv, S, d, dv=None, sigma=1.0):
    q = RNG.standard_normal((B, H, d)) * sigma
    k = RNG.standard_normal((B, Hkv, S, d)) * sigma
    v = RNG.standard_normal((B, Hkv, S, dv or d))
    return q, k, v


@pytest.mark.parametrize("W,cap,H,Hkv,sinks", [
    (0, 0.0, 4, 2, None), (3, 0.0, 4, 1, None), (0, 5.0, 2, 2, (0.5, -1.0)),
    (5, 2.0, 6, 3, (1.0, 0.0, -2.0, 3.0, 0.2, -0.4)), (1, 0.0, 2, 1, None),
    (100, 0.0, 2, 2, None)])
def test_equals_last_row_of_prefill(W, cap, H, Hkv, sinks):
    """For each sequence, placing its query at row lens[b]-1 of a prefill
    over the first lens[b] cache positions gives the same o and lse."""
    B, S, d = 3, 11, 8
    q, k, v = _cache(B, H, Hkv, S, d)
    lens = [11, 7, 1]
    sk = None if sinks is None else np.array(sinks)
    o, lse = D.decode(q, k, v, lens, 0.4, W, cap, sk)
    for b, n in enumerate(lens):
        qf = RNG.standard_normal((1, H, n, d))
        qf[0, :, n - 1] = q[b]
        of, lf = A.attn_fwd(qf, k[b:b + 1, :, :n], v[b:b + 1, :, :n], 0.4, W, cap, sinks=sk)
        np.testing.assert_allclose(o[b], of[0, :, n - 1], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[b], lf[0, :, n - 1], rtol=1e-12, atol=1e-12)


def test_positions_past_length_are_not_read():
    q, k, v = _cache(2, 2, 1, 9, 4)
    lens = [5, 9]
    o1, l1 = D.decode(q, k, v, lens, 0.5)
    k2, v2 = k.copy(), v.copy()
    k2[0, :, 5:] = np.nan
    v2[0, :, 5:] = np.inf
    o2, l2 = D.decode(q, k2, v2, lens, 0.5)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


@pytest.mark.parametrize("W", [0, 3, 50])
def test_zero_query_closed_form(W):
    """q = 0: all visible scores are 0, so o is the mean of the visible
    values and lse = ln(number visible)."""
    B, H, Hkv, S, d = 2, 2, 2, 10, 4
    _, k, v = _cache(B, H, Hkv, S, d)
    q = np.zeros((B, H, d))
    lens = [10, 6]
    o, lse = D.decode(q, k, v, lens, 0.3, W, 7.0)
    for b, n in enumerate(lens):
        lo = max(0, n - W) if W else 0
        for h in range(H):
            # o is (1/n)(1 + O(eps)) times a sum of n O(1) values: an absolute
            # rounding term covers elements whose mean cancels to near zero
            np.testing.assert_allclose(o[b, h], v[b, h, lo:n].mean(axis=0), rtol=1e-13,
                                       atol=1e-14 * n * np.abs(v[b, h, lo:n]).max())
            assert abs(lse[b, h] - math.log(n - lo)) < 1e-13


def test_window_one_is_newest_value():
    q, k, v = _cache(2, 4, 2, 6, 8)
    lens = [6, 3]
    o, lse = D.decode(q, k, v, lens, 0.25, 1, 0.0)
    for b, n in enumerate(lens):
        for h in range(4):
            np.testing.assert_allclose(o[b, h], v[b, h // 2, n - 1], rtol=1e-13)
            assert abs(lse[b, h] - 0.25 * k[b, h // 2, n - 1] @ q[b, h]) < 1e-12


def test_empty_cache():
    q, k, v = _cache(1, 2, 1, 4, 4)
    o, lse = D.decode(q, k, v, [0], 0.5)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    o, lse = D.decode(q, k, v, [0], 0.5, sinks=np.array([0.7, -0.3]))
    assert np.all(o == 0)
    np.testing.assert_allclose(lse[0], [0.7, -0.3])


@pytest.mark.parametrize("splits", [[0, 4, 9, 13], [0, 1, 13], [0, 13]])
def test_split_merge_identity(splits):
    """Decoding over disjoint chunks of the cache and merging by lse equals
    decoding over the whole cache (empty chunks drop out)."""
    B, H, Hkv, S, d = 2, 3, 1, 13, 6
    q, k, v = _cache(B, H, Hkv, S, d, dv=5)
    lens = [13, 13]
    o, lse = D.decode(q, k, v, lens, 0.6, 0, 3.0)
    parts_o, parts_l = [], []
    for a, b in zip(splits[:-1], splits[1:]):
        # chunk [a, b): shift the query to see exactly these keys
        po, pl = D.decode(q, k[:, :, a:b], v[:, :, a:b], [b - a] * B, 0.6, 0, 3.0)
        parts_o.append(po)
        parts_l.append(pl)
    parts_o.append(np.zeros_like(o))           # an empty chunk
    parts_l.append(np.full(lse.shape, -np.inf))
    mo, ml = D.merge_partials(parts_o, parts_l)
    np.testing.assert_allclose(mo, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ml, lse, rtol=1e-12)
