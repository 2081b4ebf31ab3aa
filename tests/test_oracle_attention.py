"""Pins of the float64 attention oracle to things other than itself.

Each test ties a part of oracle.attention to a closed form, an invariant of
the definition, a library routine (torch's scaled_dot_product_attention in
float64 on the CPU) or brute force, chosen so that a plausible slip -- an
off-by-one in the window, the cap applied before the scale, a wrong GQA
head map, a dropped tanh' factor, a transposed operand -- fails one of them.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A

RNG = np.random.default_rng(1234)


def _rand(*shape, sigma=1.0):
    return RNG.standard_normal(shape) * sigma


def _n_visible(i, W):
    return i + 1 if W <= 0 else min(i + 1, W)


# ---------------------------------------------------------------- forward

@pytest.mark.parametrize("T,W,cap,H,Hkv", [
    (7, 0, 0.0, 2, 2), (9, 3, 0.0, 4, 2), (9, 1, 2.0, 2, 1), (12, 5, 50.0, 3, 3),
    (6, 6, 0.0, 2, 1), (6, 20, 2.0, 2, 2)])
def test_closed_form_zero_query(T, W, cap, H, Hkv):
    """q = 0: every visible score is 0 (tanh 0 = 0 too), so o_i is the mean
    of the visible v_j and lse_i = ln n_i with n_i = min(i+1, W)."""
    d = 4
    q = np.zeros((1, H, T, d))
    k = _rand(1, Hkv, T, d)
    v = _rand(1, Hkv, T, d)
    o, lse = A.attn_fwd(q, k, v, 0.5, W, cap)
    grp = H // Hkv
    for h in range(H):
        g = h // grp
        for i in range(T):
            n = _n_visible(i, W if W < T else 0)
            lo = i - n + 1
            np.testing.assert_allclose(o[0, h, i], v[0, g, lo:i + 1].mean(0),
                                       rtol=0, atol=1e-13)
            assert abs(lse[0, h, i] - math.log(n)) < 1e-13


@pytest.mark.parametrize("cap", [0.0, 0.7, 50.0])
def test_closed_form_single_position(cap):
    """T = 1: the only key is the query's own, so o = v and
    lse = S'_00 = cap*tanh(scale*<q,k>/cap) (scale applied before the cap)."""
    d, scale = 8, 0.3
    q = _rand(2, 3, 1, d, sigma=3.0)
    k = _rand(2, 3, 1, d, sigma=3.0)
    v = _rand(2, 3, 1, d)
    o, lse = A.attn_fwd(q, k, v, scale, 0, cap)
    np.testing.assert_allclose(o, v, atol=1e-14)
    for b in range(2):
        for h in range(3):
            s = scale * sum(q[b, h, 0, c] * k[b, h, 0, c] for c in range(d))
            want = cap * math.tanh(s / cap) if cap > 0 else s
            assert abs(lse[b, h, 0] - want) < 1e-12


@pytest.mark.parametrize("cap", [0.0, 2.0])
def test_closed_form_window_one(cap):
    """window = 1: each query sees only itself: o_i = v_i, lse_i = S'_ii."""
    T, d, scale = 10, 6, 0.4
    q = _rand(1, 4, T, d)
    k = _rand(1, 2, T, d)
    v = _rand(1, 2, T, d)
    o, lse = A.attn_fwd(q, k, v, scale, 1, cap)
    for h in range(4):
        g = h // 2
        np.testing.assert_allclose(o[0, h], v[0, g], atol=1e-14)
        s = scale * np.einsum("td,td->t", q[0, h], k[0, g])
        want = cap * np.tanh(s / cap) if cap > 0 else s
        np.testing.assert_allclose(lse[0, h], want, atol=1e-12)


@pytest.mark.parametrize("W,cap", [(0, 0.0), (4, 0.0), (3, 5.0)])
def test_probability_rows(W, cap):
    """Rows of P sum to 1, masked entries are exactly 0 and visible ones are
    positive; o = P v."""
    T, d = 11, 5
    q, k, v = _rand(T, d, sigma=2), _rand(T, d, sigma=2), _rand(T, d)
    o, lse, p = A.head_forward(q, k, v, 0.7, W, cap)
    np.testing.assert_allclose(p.sum(1), 1.0, atol=1e-14)
    for i in range(T):
        for j in range(T):
            vis = j <= i and (W == 0 or j > i - W)
            assert (p[i, j] > 0) == vis
    np.testing.assert_allclose(o, p @ v, atol=1e-14)


def test_window_at_least_T_is_causal():
    T, d = 9, 4
    q, k, v = _rand(1, 2, T, d), _rand(1, 2, T, d), _rand(1, 2, T, d)
    o0, l0 = A.attn_fwd(q, k, v, 0.5, 0, 0.0)
    for W in (T, T + 1, 10 * T):
        o1, l1 = A.attn_fwd(q, k, v, 0.5, W, 0.0)
        np.testing.assert_array_equal(o0, o1)
        np.testing.assert_array_equal(l0, l1)


def test_huge_softcap_is_no_softcap():
    T, d = 9, 4
    q, k, v = _rand(1, 2, T, d, sigma=3), _rand(1, 2, T, d, sigma=3), _rand(1, 2, T, d)
    o0, l0 = A.attn_fwd(q, k, v, 0.5, 3, 0.0)
    o1, l1 = A.attn_fwd(q, k, v, 0.5, 3, 1e8)
    np.testing.assert_allclose(o0, o1, atol=1e-12)
    np.testing.assert_allclose(l0, l1, atol=1e-12)


def test_gqa_equals_mha_with_repeated_heads():
    """GQA = MHA on K/V heads repeat-interleaved (head h reads h // grp)."""
    T, d, H, Hkv = 8, 4, 6, 2
    q, k, v = _rand(2, H, T, d), _rand(2, Hkv, T, d), _rand(2, Hkv, T, d)
    do = _rand(2, H, T, d)
    kr, vr = np.repeat(k, H // Hkv, axis=1), np.repeat(v, H // Hkv, axis=1)
    o0, l0 = A.attn_fwd(q, k, v, 0.5, 3, 2.0)
    o1, l1 = A.attn_fwd(q, kr, vr, 0.5, 3, 2.0)
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)
    dq0, dk0, dv0 = A.attn_bwd(q, k, v, do, 0.5, 3, 2.0)
    dq1, dk1, dv1 = A.attn_bwd(q, kr, vr, do, 0.5, 3, 2.0)
    np.testing.assert_allclose(dq0, dq1, atol=1e-13)
    grp = H // Hkv
    np.testing.assert_allclose(dk0, dk1.reshape(2, Hkv, grp, T, d).sum(2), atol=1e-13)
    np.testing.assert_allclose(dv0, dv1.reshape(2, Hkv, grp, T, d).sum(2), atol=1e-13)


def test_batch_and_head_independence():
    T, d = 6, 4
    q, k, v = _rand(2, 2, T, d), _rand(2, 2, T, d), _rand(2, 2, T, d)
    o, l = A.attn_fwd(q, k, v, 0.5, 0, 0.0)
    q2 = q.copy()
    q2[1, 0] += 1.0
    o2, l2 = A.attn_fwd(q2, k, v, 0.5, 0, 0.0)
    np.testing.assert_array_equal(o[0], o2[0])
    np.testing.assert_array_equal(o[1, 1], o2[1, 1])
    assert not np.allclose(o[1, 0], o2[1, 0])


def _sdpa_mask(T, W):
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    m = j <= i
    if W > 0:
        m &= j > i - W
    return m


@pytest.mark.parametrize("W", [0, 4])
def test_matches_torch_sdpa_float64(W):
    """Library routine: torch's scaled_dot_product_attention in float64 on
    the CPU with an explicit boolean mask (W = 0 also via is_causal)."""
    B, H, T, d, scale = 2, 3, 13, 8, 0.37
    q, k, v = _rand(B, H, T, d), _rand(B, H, T, d), _rand(B, H, T, d)
    o, lse = A.attn_fwd(q, k, v, scale, W, 0.0)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=_sdpa_mask(T, W), scale=scale).numpy()
    np.testing.assert_allclose(o, ref, atol=1e-12)
    if W == 0:
        ref2 = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, is_causal=True, scale=scale).numpy()
        np.testing.assert_allclose(o, ref2, atol=1e-12)
    # lse against torch.logsumexp of the masked library-scaled scores
    s = torch.matmul(tq, tk.transpose(-1, -2)) * scale
    s = s.masked_fill(~_sdpa_mask(T, W), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), atol=1e-12)


def test_bruteforce_python_loops():
    """Pure-Python scalar loops (math module only) on a tiny GQA case with a
    window and a softcap."""
    B, H, Hkv, T, d, scale, W, cap = 1, 4, 2, 5, 3, 0.9, 3, 1.5
    q, k, v = _rand(B, H, T, d, sigma=2), _rand(B, Hkv, T, d, sigma=2), _rand(B, Hkv, T, d)
    o, lse = A.attn_fwd(q, k, v, scale, W, cap)
    for h in range(H):
        g = h * Hkv // H
        for i in range(T):
            js = [j for j in range(T) if j <= i and j > i - W]
            sc = []
            for j in js:
                s = scale * sum(q[0, h, i, c] * k[0, g, j, c] for c in range(d))
                sc.append(cap * math.tanh(s / cap))
            mx = max(sc)
            den = sum(math.exp(x - mx) for x in sc)
            assert abs(lse[0, h, i] - (mx + math.log(den))) < 1e-12
            for c in range(d):
                want = sum(math.exp(x - mx) / den * v[0, g, j, c] for x, j in zip(sc, js))
                assert abs(o[0, h, i, c] - want) < 1e-12


def test_layer_window_patterns():
    """Mistral: every layer windowed; Gemma 3 5:1 -> every 6th layer global;
    Gemma 2 1:1 -> every 2nd layer global (local first)."""
    assert [A.layer_window(l, 4096, 0) for l in range(4)] == [4096] * 4
    g3 = [A.layer_window(l, 1024, 6) for l in range(12)]
    assert g3 == [1024] * 5 + [0] + [1024] * 5 + [0]
    g2 = [A.layer_window(l, 4096, 2) for l in range(4)]
    assert g2 == [4096, 0, 4096, 0]
    with pytest.raises(ValueError):
        A.layer_window(0, -1, 0)


# ---------------------------------------------------------------- backward

def _loss(q, k, v, r, scale, W, cap):
    o, _ = A.attn_fwd(q, k, v, scale, W, cap)
    return float((o * r).sum())


@pytest.mark.parametrize("Hkv,T,d,W,cap", [
    (1, 1, 4, 0, 0.0), (2, 5, 4, 0, 0.0), (1, 9, 8, 3, 0.0), (2, 9, 4, 1, 2.0),
    (1, 5, 8, 0, 2.0), (2, 9, 8, 3, 2.0)])
def test_gradcheck_central_differences(Hkv, T, d, W, cap):
    """Central finite differences (h = 1e-6) of L = sum(o * R)."""
    H, scale, h = 2, 0.6, 1e-6
    q, k, v = _rand(1, H, T, d, sigma=1.5), _rand(1, Hkv, T, d, sigma=1.5), _rand(1, Hkv, T, d)
    r = _rand(1, H, T, d)
    dq, dk, dv = A.attn_bwd(q, k, v, r, scale, W, cap)
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.empty_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, r, scale, W, cap)
            x[idx] = old - h
            lm = _loss(q, k, v, r, scale, W, cap)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        err = np.abs(num - g).max() / max(1e-3, np.abs(num).max())
        assert err < 1e-6, err


def test_backward_window_one_closed_form():
    """window = 1: o_i = v_i whatever q, k are, so dq = dk = 0 and
    dv_j = sum over the group's heads of dO_j."""
    T, d = 7, 4
    q, k, v, do = _rand(1, 4, T, d), _rand(1, 2, T, d), _rand(1, 2, T, d), _rand(1, 4, T, d)
    dq, dk, dv = A.attn_bwd(q, k, v, do, 0.5, 1, 2.0)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
    np.testing.assert_allclose(dv[0, 0], do[0, 0] + do[0, 1], atol=1e-14)
    np.testing.assert_allclose(dv[0, 1], do[0, 2] + do[0, 3], atol=1e-14)


@pytest.mark.parametrize("W", [0, 3])
def test_backward_zero_query_closed_form(W):
    """q = 0: P_ij = 1/n_i on visible pairs, so dv_j = sum_{i sees j} dO_i/n_i."""
    T, d = 8, 3
    q = np.zeros((1, 1, T, d))
    k, v, do = _rand(1, 1, T, d), _rand(1, 1, T, d), _rand(1, 1, T, d)
    _, _, dv = A.attn_bwd(q, k, v, do, 0.5, W, 0.0)
    for j in range(T):
        want = np.zeros(d)
        for i in range(j, T):
            if W == 0 or j > i - W:
                want += do[0, 0, i] / _n_visible(i, W)
        np.testing.assert_allclose(dv[0, 0, j], want, atol=1e-14)


@pytest.mark.parametrize("cap", [0.0, 2.0])
def test_backward_equal_keys_give_zero_dq(cap):
    """All keys equal: S' is constant along each row, P does not depend on q,
    so dq = 0 (with or without the cap)."""
    T, d = 9, 4
    q, v, do = _rand(1, 2, T, d), _rand(1, 2, T, d), _rand(1, 2, T, d)
    k = np.broadcast_to(_rand(1, 2, 1, d), (1, 2, T, d)).copy()
    dq, _, _ = A.attn_bwd(q, k, v, do, 0.5, 4, cap)
    assert np.abs(dq).max() < 1e-13


@pytest.mark.parametrize("W", [0, 5])
def test_backward_matches_torch_autograd_sdpa(W):
    """Library routine: torch.autograd through float64 CPU SDPA."""
    B, H, T, d, scale = 1, 2, 12, 8, 0.35
    q, k, v, do = (_rand(B, H, T, d) for _ in range(4))
    dq, dk, dv = A.attn_bwd(q, k, v, do, scale, W, 0.0)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=_sdpa_mask(T, W), scale=scale)
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


def test_rowsum_identity():
    """D_i = <dO_i, o_i> equals sum_j P_ij dP_ij (the identity the backward
    prologue relies on)."""
    T, d = 10, 5
    q, k, v, do = _rand(T, d), _rand(T, d), _rand(T, d), _rand(T, d)
    o, _, p = A.head_forward(q, k, v, 0.5, 4, 3.0)
    D = (do * o).sum(1)
    np.testing.assert_allclose(D, (p * (do @ v.T)).sum(1), atol=1e-13)


@pytest.mark.parametrize("W,cap", [(0, 0.0), (5, 2.0)])
def test_sampled_grads_match_full(W, cap):
    """The row/column-restricted evaluator used for large-T sampled checks
    agrees with the full-matrix definition."""
    T, d = 37, 6
    q, k, v, do = _rand(T, d), _rand(T, d), _rand(T, d), _rand(T, d)
    dq, dk, dv = A.head_backward(q, k, v, do, 0.5, W, cap)
    o, lse, _ = A.head_forward(q, k, v, 0.5, W, cap)
    qr, kr = np.array([0, 5, 36]), np.array([0, 17, 36])
    sq, sk, sv, so, sl = A.head_grads_sampled(q, k, v, do, 0.5, W, cap, qr, kr,
                                              row_block=8)
    np.testing.assert_allclose(sq, dq[qr], atol=1e-13)
    np.testing.assert_allclose(sk, dk[kr], atol=1e-13)
    np.testing.assert_allclose(sv, dv[kr], atol=1e-13)
    np.testing.assert_allclose(so, o, atol=1e-13)
    np.testing.assert_allclose(sl, lse, atol=1e-13)


# ------------------------------------------------ sinks, max logit, d_v != d_k

@pytest.mark.parametrize("W,sink", [(0, 0.7), (3, -1.2), (0, 4.0)])
def test_sink_closed_form_zero_query(W, sink):
    """q = 0: every visible logit is 0, so P_ij = 1/(n_i + e^s) and
    lse_i = ln(n_i + e^s); o_i = n_i/(n_i + e^s) * mean of the visible v."""
    T, d = 9, 4
    q = np.zeros((1, 2, T, d))
    k, v = _rand(1, 1, T, d), _rand(1, 1, T, d)
    o, lse = A.attn_fwd(q, k, v, 0.5, W, 0.0, sinks=np.array([sink, sink]))
    for i in range(T):
        n = _n_visible(i, W)
        z = n + math.exp(sink)
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, i - n + 1:i + 1].sum(0) / z, atol=1e-13)
        assert abs(lse[0, 1, i] - math.log(z)) < 1e-13


def test_very_negative_sink_is_no_sink():
    T, d = 8, 4
    q, k, v, do = _rand(1, 2, T, d), _rand(1, 1, T, d), _rand(1, 1, T, d), _rand(1, 2, T, d)
    o0, l0 = A.attn_fwd(q, k, v, 0.5, 3, 2.0)
    o1, l1 = A.attn_fwd(q, k, v, 0.5, 3, 2.0, sinks=np.array([-1e4, -1e4]))
    np.testing.assert_allclose(o0, o1, atol=1e-14)
    np.testing.assert_allclose(l0, l1, atol=1e-14)
    g0 = A.attn_bwd(q, k, v, do, 0.5, 3, 2.0)
    g1 = A.attn_bwd(q, k, v, do, 0.5, 3, 2.0, sinks=np.array([-1e4, -1e4]))
    for a, b in zip(g0, g1[:3]):
        np.testing.assert_allclose(a, b, atol=1e-13)
    assert np.abs(g1[3]).max() < 1e-12


@pytest.mark.parametrize("W,cap,dv", [(0, 0.0, 4), (3, 2.0, 4), (0, 0.0, 3)])
def test_sink_and_dv_gradcheck(W, cap, dv):
    """Central differences w.r.t. q, k, v and the sinks, including a value
    head size different from the query/key head size (d_v = 3, d = 4)."""
    H, T, d, scale, h = 2, 6, 4, 0.6, 1e-6
    q, k = _rand(1, H, T, d, sigma=1.5), _rand(1, 1, T, d, sigma=1.5)
    v = _rand(1, 1, T, dv)
    r = _rand(1, H, T, dv)
    sinks = np.array([0.3, -0.8])

    def loss():
        o, _ = A.attn_fwd(q, k, v, scale, W, cap, sinks=sinks)
        return float((o * r).sum())

    dq, dk, dvv, ds = A.attn_bwd(q, k, v, r, scale, W, cap, sinks=sinks)
    for x, g in ((q, dq), (k, dk), (v, dvv), (sinks, ds)):
        num = np.empty_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            lp = loss()
            x[idx] = old - h
            lm = loss()
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        err = np.abs(num - g).max() / max(1e-3, np.abs(num).max())
        assert err < 1e-6, err


def test_dv_differs_from_dk_closed_form():
    """q = 0 with d_v != d: o_i is the mean of the visible v rows."""
    T = 7
    q = np.zeros((1, 1, T, 5))
    k, v = _rand(1, 1, T, 5), _rand(1, 1, T, 3)
    o, lse = A.attn_fwd(q, k, v, 0.3, 0, 0.0)
    assert o.shape == (1, 1, T, 3)
    for i in range(T):
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, :i + 1].mean(0), atol=1e-14)


def test_max_logit_bruteforce_and_window_one():
    B, H, Hkv, T, d, scale = 1, 4, 2, 6, 3, 0.7
    q, k = _rand(B, H, T, d, sigma=2), _rand(B, Hkv, T, d, sigma=2)
    for W, cap in ((0, 0.0), (2, 0.0), (0, 1.5)):
        got = A.max_logit(q, k, scale, W, cap)
        for h in range(H):
            best = -math.inf
            for i in range(T):
                for j in range(T):
                    if j <= i and (W == 0 or j > i - W):
                        s = scale * sum(q[0, h, i, c] * k[0, h // 2, j, c] for c in range(d))
                        best = max(best, cap * math.tanh(s / cap) if cap else s)
            assert abs(got[0, h] - best) < 1e-12
    got = A.max_logit(q, k, scale, 1, 0.0)
    for h in range(H):
        diag = scale * np.einsum("td,td->t", q[0, h], k[0, h // 2])
        assert abs(got[0, h] - diag.max()) < 1e-12
