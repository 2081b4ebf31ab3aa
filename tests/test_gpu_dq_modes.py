"""The two dQ strategies of the bf16 backward through the C ABI: dQ from the
dS tiles the dK/dV pass stores (fa_set_dq_mode(2); the default at d = 256)
and the recomputing dQ pass (fa_set_dq_mode(1); the default at d = 128).

On the same inputs both hand the dK/dV pass the same D, so dk and dv must be
the same bits; dq from either strategy must meet the oracle's bar (every
element within the derived bf16 envelope).  The shapes put query and key
tiles on the workspace band's edges: T one below, at and one above the tile
multiples, windows one below, at and one above multiples of 32 (the band
width ceil((W - 1) / 32) + 1 changes there), GQA, softcap, fused RoPE, at
d = 128 (the single-wave dK/dV pass) and d = 256 (the paired one).  At
full-size shapes the two dq agree within the bar of each other (no oracle).
"""
import math

import numpy as np
import pytest
import torch

from causal_attention_fa_amd import synth
from tests.gpu_util import check, dev, oracle_full, poison, say

pytestmark = pytest.mark.gpu

CASES = [  # B, H, Hkv, T, d, window, cap, seed
    (1, 2, 2, 1, 128, 0, 0.0, 1),
    (1, 2, 1, 33, 128, 0, 0.0, 2),
    (2, 4, 2, 127, 128, 32, 0.0, 3),
    (1, 4, 1, 129, 128, 33, 0.0, 4),
    (1, 2, 2, 200, 128, 31, 20.0, 5),
    (2, 8, 2, 300, 128, 1, 0.0, 6),
    (1, 7, 1, 385, 128, 97, 50.0, 7),
    (1, 4, 4, 513, 128, 0, 5.0, 8),
    (1, 4, 2, 640, 128, 257, 0.0, 9),
    (1, 2, 1, 1000, 128, 999, 0.0, 10),
    (1, 2, 2, 1, 256, 0, 0.0, 21),
    (1, 4, 2, 95, 256, 0, 50.0, 22),
    (2, 4, 1, 161, 256, 33, 0.0, 23),
    (1, 2, 1, 257, 256, 64, 30.0, 24),
    (1, 6, 3, 400, 256, 129, 50.0, 25),
    (1, 4, 2, 513, 256, 0, 0.0, 26),
]


def _run(fa, tensors, w, W, cap, mode, rope_tab=None):
    qd, kd, vd, o, lse, dod = tensors
    gq, gk, gv = poison(qd.shape, qd.dtype), poison(kd.shape, kd.dtype), poison(vd.shape, vd.dtype)
    prev = fa.fa_set_dq_mode(mode)
    try:
        if rope_tab is None:
            fa.fa_bwd(qd, kd, vd, o, lse, dod, gq, gk, gv, w.B, w.H, w.Hkv, w.T, w.d, w.scale, W,
                      0, cap)
        else:
            fa.fa_bwd_rope(qd, kd, vd, o, lse, dod, rope_tab, gq, gk, gv, w.B, w.H, w.Hkv, w.T,
                           w.d, w.scale, W, 0, cap)
        torch.cuda.synchronize()
    finally:
        fa.fa_set_dq_mode(prev)
    return {n: t.float().cpu().numpy() for n, t in dict(dq=gq, dk=gk, dv=gv).items()}


def _forward(fa, q, k, v, w, W, cap):
    qd, kd, vd = (t.to(dev()) for t in (q, k, v))
    o = poison(q.shape, q.dtype)
    lse = poison((w.B, w.H, w.T), torch.float32)
    fa.fa_fwd(qd, kd, vd, o, lse, w.B, w.H, w.Hkv, w.T, w.d, w.scale, W, 0, cap)
    return qd, kd, vd, o, lse


@pytest.mark.parametrize("case", CASES, ids=[
    f"B{c[0]}H{c[1]}/{c[2]}T{c[3]}d{c[4]}W{c[5]}cap{c[6]:g}" for c in CASES])
def test_dq_modes_against_oracle(case):
    from causal_attention_fa_amd import fa
    B, H, Hkv, T, d, W, cap, seed = case
    prev = fa.fa_set_dq_mode(2)
    try:
        assert fa.fa_bwd_kernels(d) == ["rowdot", "dkdv", "dq_ds"]
    finally:
        fa.fa_set_dq_mode(prev)
    w = synth.Workload("dqm", "bf16", B, H, Hkv, T, d, sigma_qk=2.0 if cap else 1.0, seed=seed)
    q, k, v, do = synth.draw(w)
    say(f"[dq modes] B{B} H{H}/{Hkv} T{T} d{d} W{W} cap{cap} seed{seed}")
    qd, kd, vd, o, lse = _forward(fa, q, k, v, w, W, cap)
    t = (qd, kd, vd, o, lse, do.to(dev()))
    stored = _run(fa, t, w, W, cap, 2)
    recomp = _run(fa, t, w, W, cap, 1)
    for n in ("dk", "dv"):
        assert np.array_equal(stored[n], recomp[n]), f"{n}: differs between the dQ strategies"
    ref = oracle_full(q, k, v, do, w.scale, W, cap)
    e0 = check("dq (stored dS)", stored["dq"], ref["dq"], env=ref["E_dq"], qty="dq")
    e1 = check("dq (recomputed)", recomp["dq"], ref["dq"], env=ref["E_dq"], qty="dq")
    for n in ("dk", "dv"):
        check(n, stored[n], ref[n], env=ref["E_" + n])
    say(f"  dq rms-relative: stored {e0:.2e}, recomputed {e1:.2e}")


def test_dq_modes_fused_rope():
    """fa_bwd_rope rotates dq back at its store in both dQ passes."""
    from causal_attention_fa_amd import fa
    w = synth.Workload("dqr", "bf16", 1, 4, 2, 300, 128, window=100, rope_theta=1e4, seed=11)
    q, k, v, do = synth.draw(w)
    tab = torch.from_numpy(fa.fa_rope_inv_freq(w.d, w.rope_theta)).to(dev())
    say("[dq modes, fused rope] B1 H4/2 T300 d128 W100")
    qr = poison(q.shape, q.dtype)
    kd = k.to(dev())
    kr = torch.empty_like(kd)
    fa.rope_apply(kd, kr, tab, w.B, w.Hkv, w.T, w.d)
    vd = v.to(dev())
    o = poison(q.shape, q.dtype)
    lse = poison((w.B, w.H, w.T), torch.float32)
    fa.fa_fwd_rope(q.to(dev()), kr, vd, o, lse, tab, qr, w.B, w.H, w.Hkv, w.T, w.d, w.scale,
                   w.window, 0, 0.0)
    t = (qr, kr, vd, o, lse, do.to(dev()))
    stored = _run(fa, t, w, w.window, 0.0, 2, rope_tab=tab)
    recomp = _run(fa, t, w, w.window, 0.0, 1, rope_tab=tab)
    for n in ("dk", "dv"):
        assert np.array_equal(stored[n], recomp[n]), n
    diff = stored["dq"] - recomp["dq"]
    rel = math.sqrt(float(np.mean(diff ** 2)) / float(np.mean(recomp["dq"] ** 2)))
    say(f"  dq stored vs recomputed rms-relative {rel:.2e}")
    assert np.isfinite(stored["dq"]).all() and rel <= 1e-2


@pytest.mark.parametrize("name", ["mistral", "gemma-global"])
def test_dq_modes_full_size(name):
    """Full-size workloads (mistral: B4 H32/8 T8192 d128, window 4096;
    gemma-global: B2 H8/4 T8192 d256, softcap 50): the two dq agree within
    the bf16 bar of each other, dk and dv are the same bits."""
    from causal_attention_fa_amd import fa
    w = synth.WORKLOADS[name]
    q, k, v, do = synth.draw(w)
    say(f"[dq modes, full size] {name}")
    qd, kd, vd, o, lse = _forward(fa, q, k, v, w, w.window, w.softcap)
    t = (qd, kd, vd, o, lse, do.to(dev()))
    stored = _run(fa, t, w, w.window, w.softcap, 2)
    recomp = _run(fa, t, w, w.window, w.softcap, 1)
    for n in ("dk", "dv"):
        assert np.array_equal(stored[n], recomp[n]), n
    diff = stored["dq"] - recomp["dq"]
    rel = math.sqrt(float(np.mean(diff ** 2)) / float(np.mean(recomp["dq"] ** 2)))
    say(f"  dq stored vs recomputed rms-relative {rel:.2e}")
    assert np.isfinite(stored["dq"]).all() and rel <= 1e-2


@pytest.mark.parametrize("d,T,W,cap", [(256, 3001, 777, 30.0), (128, 2999, 1001, 0.0)])
def test_dq_modes_ragged_mid_size(d, T, W, cap):
    """Ragged T and window (no multiple of 32 or 128) at a size between the
    oracle shapes and the full workloads, GQA 3: the two dq agree within
    the bf16 bar of each other, dk and dv are the same bits."""
    from causal_attention_fa_amd import fa
    w = synth.Workload("dqrag", "bf16", 2, 6, 2, T, d, sigma_qk=2.0 if cap else 1.0, seed=77)
    q, k, v, do = synth.draw(w)
    say(f"[dq modes, ragged] B2 H6/2 T{T} d{d} W{W} cap{cap}")
    qd, kd, vd, o, lse = _forward(fa, q, k, v, w, W, cap)
    t = (qd, kd, vd, o, lse, do.to(dev()))
    stored = _run(fa, t, w, W, cap, 2)
    recomp = _run(fa, t, w, W, cap, 1)
    for n in ("dk", "dv"):
        assert np.array_equal(stored[n], recomp[n]), n
    diff = stored["dq"] - recomp["dq"]
    rel = math.sqrt(float(np.mean(diff ** 2)) / float(np.mean(recomp["dq"] ** 2)))
    say(f"  dq stored vs recomputed rms-relative {rel:.2e}")
    assert np.isfinite(stored["dq"]).all() and rel <= 1e-2
