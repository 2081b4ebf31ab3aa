"""GPU checks of RoPE fused into the attention (fa_fwd_rope / fa_bwd_rope).

The fused forward must produce, bit for bit, what rope_apply followed by
fa_fwd produces (the rotated q it writes equals rope_apply(q)); the fused
backward's dk and dv equal fa_bwd's bit for bit, and its dq (gradient with
respect to the un-rotated q: the inverse rotation is applied before the one
bf16 rounding) is checked against the oracle: the oracle's dq for the GPU's
rotated inputs, rotated back by oracle.rope.rope_bwd (stage-isolated, bf16
bar), and end to end from the un-rotated inputs (RMS bar)."""
import math

import numpy as np
import pytest
import torch

from causal_attention_fa_amd import synth
from oracle import attention as OA
from oracle import rope as OR
from tests import envelope as EV
from tests.gpu_util import check, dev, poison, say

pytestmark = pytest.mark.gpu

# (B, H, Hkv, T, d, window, softcap, theta)
CASES = [
    (1, 2, 2, 1, 64, 0, 0.0, 1e4),
    (2, 6, 6, 200, 64, 0, 0.0, 1e4),
    (1, 7, 1, 333, 128, 0, 0.0, 1e6),
    (1, 4, 2, 515, 128, 100, 30.0, 1e4),
    (1, 8, 4, 1024, 128, 1, 0.0, 5e5),
    (1, 4, 2, 700, 256, 300, 50.0, 1e4),
]


def _run(q, k, v, do, table, scale, W, cap):
    from causal_attention_fa_amd import fa
    B, H, T, d = q.shape
    Hkv = k.shape[1]
    tab = torch.from_numpy(table).to(dev())
    q_, k_, v_, do_ = (t.to(dev()) for t in (q, k, v, do))
    kr = poison(k.shape, k.dtype)
    fa.rope(k_, tab, out=kr)
    # separate path
    qr_sep = poison(q.shape, q.dtype)
    fa.rope(q_, tab, out=qr_sep)
    o_s, l_s = poison(q.shape, q.dtype), poison((B, H, T), torch.float32)
    fa.fa_fwd(qr_sep, kr, v_, o_s, l_s, B, H, Hkv, T, d, scale, W, 0, cap)
    dq_s, dk_s, dv_s = poison(q.shape, q.dtype), poison(k.shape, k.dtype), poison(v.shape, v.dtype)
    fa.fa_bwd(qr_sep, kr, v_, o_s, l_s, do_, dq_s, dk_s, dv_s, B, H, Hkv, T, d, scale, W, 0, cap)
    # fused path
    qr_f = poison(q.shape, q.dtype)
    o_f, l_f = poison(q.shape, q.dtype), poison((B, H, T), torch.float32)
    fa.fa_fwd_rope(q_, kr, v_, o_f, l_f, tab, qr_f, B, H, Hkv, T, d, scale, W, 0, cap)
    dq_f, dk_f, dv_f = poison(q.shape, q.dtype), poison(k.shape, k.dtype), poison(v.shape, v.dtype)
    fa.fa_bwd_rope(qr_f, kr, v_, o_f, l_f, do_, tab, dq_f, dk_f, dv_f, B, H, Hkv, T, d, scale, W,
                   0, cap)
    # forward without the rotated-q output
    o_n = poison(q.shape, q.dtype)
    fa.fa_fwd_rope(q_, kr, v_, o_n, l_f.clone(), tab, None, B, H, Hkv, T, d, scale, W, 0, cap)
    torch.cuda.synchronize()
    c = lambda t: t.float().cpu().numpy()
    return dict(kr=kr.cpu(), qr_sep=c(qr_sep), qr_f=c(qr_f), qr_f_t=qr_f.cpu(), o_s=c(o_s),
                l_s=c(l_s), o_f=c(o_f), l_f=c(l_f), o_n=c(o_n), dq_s=c(dq_s), dk_s=c(dk_s),
                dv_s=c(dv_s), dq_f=c(dq_f), dk_f=c(dk_f), dv_f=c(dv_f))


@pytest.mark.parametrize("case", CASES, ids=[
    f"B{c[0]}H{c[1]}/{c[2]}T{c[3]}d{c[4]}W{c[5]}cap{c[6]:g}" for c in CASES])
def test_fused_rope(case):
    from causal_attention_fa_amd import fa
    B, H, Hkv, T, d, W, cap, theta = case
    w = synth.Workload("rf", "bf16", B, H, Hkv, T, d, sigma_qk=2.0 if cap else 1.0,
                       seed=400 + CASES.index(case))
    q, k, v, do = synth.draw(w)
    table = fa.fa_rope_inv_freq(d, theta)
    scale = 1.0 / math.sqrt(d)
    say(f"[rope fused] B{B} H{H}/{Hkv} T{T} d{d} W{W} cap{cap} theta{theta:g}")
    r = _run(q, k, v, do, table, scale, W, cap)
    for a, b in [("qr_sep", "qr_f"), ("o_s", "o_f"), ("l_s", "l_f"), ("o_s", "o_n"),
                 ("dk_s", "dk_f"), ("dv_s", "dv_f")]:
        assert np.array_equal(r[a], r[b]), (a, b)
    # stage-isolated dq: oracle backward on the GPU's rotated q and k, rotated back
    qr64, kr64 = synth.to_f64(r["qr_f_t"]), synth.to_f64(r["kr"])
    vf, dof = synth.to_f64(v), synth.to_f64(do)
    st = EV.full_envelopes(qr64, kr64, vf, dof, scale, W, cap)
    e1 = check("dq (stage)", r["dq_f"], OR.rope_bwd(st["dq"], table), env=EV.rotate_env(st["E_dq"]),
               qty="dq")
    # end to end from the un-rotated inputs: the envelope on the oracle's own
    # rotation rounded to bf16, plus what that rounding moves the result
    q64, k64 = synth.to_f64(q), synth.to_f64(k)
    qe, ke = OR.rope(q64, table), OR.rope(k64, table)
    rnd = lambda x: torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    ex = EV.full_envelopes(qe, ke, vf, dof, scale, W, cap)
    rb = EV.full_envelopes(rnd(qe), rnd(ke), vf, dof, scale, W, cap)
    dq_ref, dq_rb = OR.rope_bwd(ex["dq"], table), OR.rope_bwd(rb["dq"], table)
    e2 = check("dq (e2e)", r["dq_f"], dq_ref,
               env=EV.rotate_env(rb["E_dq"]) + np.abs(dq_ref - dq_rb), qty="dq")
    e3 = check("o (e2e)", r["o_f"], ex["o"], env=rb["E_o"] + np.abs(ex["o"] - rb["o"]), qty="o")
    say(f"  dq stage {e1:.2e} dq e2e {e2:.2e} o e2e {e3:.2e}")
