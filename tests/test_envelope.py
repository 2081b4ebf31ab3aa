"""Pins of the bf16 error envelope (tests/envelope.py), on the CPU.

1. An emulation of the roundings the envelope allows -- float32 scores and
   sums, P rounded to bf16 before P V and P^T dO, D from the bf16 o, P
   recomputed from the float32 lse, dS rounded to bf16 before dS K, the
   factor of (dP - D) and then dS rounded before dS^T Q, every output
   rounded to bf16 -- stays inside the envelope with no RMS allowance at
   all (R_BAR = 0): the envelope is not tighter than the roundings it
   names.
2. Emulations with a planted mistake (a window one key too wide, the tanh'
   factor dropped, the wrong GQA head, D dropped, a shifted lse on a few
   rows, one corrupted output element) fall outside it at the stated bar
   R_BAR = 2e-2: it is tight enough to catch localized errors.

The emulation is numpy float32 with round-to-nearest-even to bf16; it is
test code, independent of the HIP kernels.
"""
import math

import numpy as np
import pytest

from tests import envelope as EV

LOG2E = 1.4426950408889634
LN2 = 0.6931471805599453


def bf16(x):
    """Round float32 values to bfloat16 (nearest, ties to even); float32 out."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    r = ((b >> 16) & 1) + 0x7FFF
    return ((b + r) & 0xFFFF0000).astype(np.uint32).view(np.float32)


def emulate_head(q, k, v, do, scale, W, cap, sink=None, plant=None):
    """One (b, h) of the bf16 path with the allowed roundings, float32."""
    f = np.float32
    q, k, v, do = (np.asarray(x, dtype=np.float32) for x in (q, k, v, do))
    T = k.shape[0]
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    Wv = W + 1 if plant == "window" and W > 0 else W
    vis = j <= i
    if Wv > 0:
        vis &= j > i - Wv
    s = q @ k.T
    if cap > 0:
        e = np.exp2(s * f(2 * scale * LOG2E / cap))
        th = f(1) - f(2) / (e + f(1))
        x2 = th * f(cap * LOG2E)
        t = f(1) - th * th
        if plant == "tanh":
            t = np.ones_like(t)
    else:
        x2 = s * f(scale * LOG2E)
        t = f(1)
    x2 = np.where(vis, x2, -np.inf).astype(np.float32)
    m = x2.max(1)
    if sink is not None:
        m = np.maximum(m, f(sink * LOG2E))
    p = np.exp2(x2 - m[:, None])
    l = p.sum(1, dtype=np.float32)
    if sink is not None:
        l = l + np.exp2(f(sink * LOG2E) - m)
    o = (bf16(p) @ v) / l[:, None]
    ob = bf16(o)
    lse = ((m + np.log2(l)) * f(LN2)).astype(np.float32)
    if plant == "lse":
        lse = lse.copy()
        lse[T // 3] += f(0.01)
    D = (do * ob).sum(1, dtype=np.float32)
    if plant == "D":
        D = np.zeros_like(D)
    p2 = np.exp2(x2 - (lse * f(LOG2E))[:, None])
    dP = do @ v.T
    dS = p2 * (dP - D[:, None]) * t
    dq = f(scale) * (bf16(dS) @ k)
    dSk = bf16(bf16(p2 * t) * (dP - D[:, None]))
    dk = f(scale) * (dSk.T @ q)
    dv = bf16(p2).T @ do
    if plant == "elem":
        ob = ob.copy()
        rms = float(np.sqrt(np.mean(o.astype(np.float64) ** 2)))
        ob[T // 2, 3] += f(0.05 * rms)
    return dict(o=ob, lse=lse, dq=bf16(dq), dk=bf16(dk), dv=bf16(dv))


def emulate(q, k, v, do, scale, W, cap, sinks=None, plant=None):
    B, H, T, _ = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    out = {n: [] for n in ("o", "lse", "dq")}
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(B):
        for h in range(H):
            g = h % Hkv if plant == "gqa" else h // G
            sk = None if sinks is None else float(sinks[h])
            r = emulate_head(q[b, h], k[b, g], v[b, g], do[b, h], scale, W, cap, sk, plant)
            for n in out:
                out[n].append(r[n])
            dk[b, g] += r["dk"]
            dv[b, g] += r["dv"]
    res = {n: np.stack(x).reshape((B, H) + x[0].shape) for n, x in out.items()}
    # the GPU rounds dk, dv once, after summing the group in float32
    res["dk"] = bf16(dk.astype(np.float32))
    res["dv"] = bf16(dv.astype(np.float32))
    return res


def draw(B, H, Hkv, T, d, dv, sig, seed):
    rng = np.random.default_rng(seed)
    r = lambda *s: bf16(rng.standard_normal(s).astype(np.float32)).astype(np.float64)
    return r(B, H, T, d) * sig, r(B, Hkv, T, d) * sig, r(B, Hkv, T, dv), r(B, H, T, dv)


# (B, H, Hkv, T, d, d_v, window, cap, sigma_qk, sinks)
CASES = [
    (1, 2, 2, 200, 64, 64, 0, 0.0, 1.0, False),
    (1, 4, 2, 300, 128, 128, 65, 0.0, 1.0, False),
    (1, 2, 1, 257, 256, 256, 100, 50.0, 2.0, False),
    (1, 2, 2, 129, 64, 64, 0, 2.0, 2.0, False),
    (1, 4, 4, 160, 128, 128, 0, 0.0, 1.0, True),
    (1, 2, 2, 150, 192, 128, 40, 20.0, 2.0, False),
]


def _envelopes(case, seed):
    B, H, Hkv, T, d, dvv, W, cap, sig, sk = case
    q, k, v, do = draw(B, H, Hkv, T, d, dvv, sig, seed)
    # powers of two keep the input exactly representable in bf16
    q, k = bf16(q.astype(np.float32)).astype(np.float64), bf16(k.astype(np.float32)).astype(np.float64)
    sinks = np.linspace(-1.0, 2.0, H) if sk else None
    scale = 1.0 / math.sqrt(d)
    env = EV.full_envelopes(q, k, v, do, scale, W, cap, sinks=sinks)
    return (q, k, v, do, scale, W, cap, sinks), env


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[3]}d{c[4]}/{c[5]}W{c[6]}cap{c[7]:g}"
                                             f"{'sink' if c[9] else ''}" for c in CASES])
def test_allowed_roundings_stay_inside_without_rms_allowance(case):
    args, env = _envelopes(case, seed=CASES.index(case))
    emu = emulate(*args)
    ref = {n: env[n] for n in ("o", "lse", "dq", "dk", "dv")}
    for n in ref:
        ex = EV.excess(emu[n], ref[n], env["E_" + n], r_bar=0.0)
        assert ex <= 1.0, f"{n}: emulated rounding exceeds the envelope x{ex:.2f}"
        # and the stated bar's RMS part
        assert EV.rms_rel(emu[n], ref[n]) <= EV.R_BAR, n


@pytest.mark.parametrize("plant,case,outputs", [
    ("window", CASES[1], ("o", "dq", "dk", "dv")),
    ("tanh", CASES[3], ("dq", "dk")),
    ("gqa", CASES[1], ("o", "dq", "dk", "dv")),
    ("D", CASES[0], ("dq", "dk")),
    ("lse", CASES[0], ("lse",)),
    ("elem", CASES[4], ("o",)),
])
def test_planted_mistakes_fall_outside(plant, case, outputs):
    args, env = _envelopes(case, seed=CASES.index(case))
    emu = emulate(*args, plant=plant)
    for n in outputs:
        ex = EV.excess(emu[n], env[n], env["E_" + n], r_bar=EV.r_bar_for(n))
        assert ex > 1.0, f"{plant}: {n} stays inside the envelope (x{ex:.2f})"


def test_envelope_reference_values_are_the_oracle():
    """The reference values the envelope module hands out are the oracle's
    own (attn_fwd / attn_bwd on the same inputs)."""
    from oracle import attention as OA
    (q, k, v, do, scale, W, cap, _), env = _envelopes(CASES[1], seed=11)
    o, lse = OA.attn_fwd(q, k, v, scale, W, cap)
    dq, dk, dv = OA.attn_bwd(q, k, v, do, scale, W, cap)
    for n, r in dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv).items():
        np.testing.assert_allclose(env[n], r, rtol=1e-12, atol=1e-12)
