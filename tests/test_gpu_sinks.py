"""GPU parity of fa_fwd_sink / fa_bwd_sink (attention sinks and the per-head
max logit) against the float64 oracle.

Sinks: o, lse, dq, dk, dv to the bf16 bar of the other parity tests; the
sink gradient (a sum over every row of the batch and head, accumulated with
float atomics) within 2^-6 of sum_i |p_sink,i * D_i| -- the sum of the
magnitudes of its terms, so that cancellation between rows of opposite sign
does not inflate a relative bar; each term's own error is that of D_i from
the bf16 output (2^-8 relative) plus the exponent's.
Max logit: the largest post-cap logit of each (batch, head), to 1e-4 *
(1 + |ref|) (fp32 dot products of bf16 inputs)."""
import math

import numpy as np
import pytest
import torch

from causal_attention_fa_amd import synth
from oracle import attention as OA
from tests import envelope as EV
from tests.gpu_util import check, dev, poison, run_gpu, say

pytestmark = pytest.mark.gpu

# (B, H, Hkv, T, d, window, softcap, sigma_qk, sink values cycled over heads)
CASES = [
    (1, 2, 2, 1, 64, 0, 0.0, 1.0, (0.5, -0.5)),
    (2, 4, 2, 97, 64, 0, 0.0, 1.0, (0.0, 2.0, -3.0, 6.0)),
    (1, 4, 1, 300, 128, 0, 0.0, 1.0, (1.0, -1.0)),
    (1, 8, 2, 257, 128, 65, 30.0, 2.0, (0.3, 4.0, -2.0)),
    (1, 2, 2, 200, 128, 1, 0.0, 1.0, (2.0, -30.0)),
    (1, 4, 2, 515, 256, 100, 50.0, 2.0, (-0.7, 1.5)),
    (2, 2, 1, 640, 128, 0, 0.0, 1.0, (8.0, -8.0)),
]


def _sinks(H, vals):
    return np.array([vals[h % len(vals)] for h in range(H)], np.float32)


def run_gpu_sink(q, k, v, do, sinks, scale, window, softcap):
    from causal_attention_fa_amd import fa
    B, H, T, d = q.shape
    Hkv = k.shape[1]
    q_, k_, v_, do_ = (t.to(dev()) for t in (q, k, v, do))
    s_ = torch.from_numpy(sinks).to(dev())
    o = poison(q.shape, q.dtype)
    lse = poison((B, H, T), torch.float32)
    ml = poison((B, H), torch.float32)
    fa.fa_fwd_sink(q_, k_, v_, o, lse, s_, ml, B, H, Hkv, T, d, scale, window, 0, softcap)
    gq, gk, gv = poison(q.shape, q.dtype), poison(k.shape, k.dtype), poison(v.shape, v.dtype)
    ds = poison((H,), torch.float32)
    fa.fa_bwd_sink(q_, k_, v_, o, lse, do_, s_, gq, gk, gv, ds, B, H, Hkv, T, d, scale, window, 0,
                   softcap)
    torch.cuda.synchronize()
    return {n: t.float().cpu().numpy() for n, t in
            dict(o=o, lse=lse, dq=gq, dk=gk, dv=gv, dsinks=ds, max_logit=ml).items()}


def _draw(B, H, Hkv, T, d, sig, seed):
    w = synth.Workload("sink", "bf16", B, H, Hkv, T, d, sigma_qk=sig, seed=seed)
    return synth.draw(w)


@pytest.mark.parametrize("case", CASES, ids=[
    f"B{c[0]}H{c[1]}/{c[2]}T{c[3]}d{c[4]}W{c[5]}cap{c[6]:g}" for c in CASES])
def test_sink_parity_vs_oracle(case):
    B, H, Hkv, T, d, W, cap, sig, vals = case
    q, k, v, do = _draw(B, H, Hkv, T, d, sig, seed=100 + CASES.index(case))
    sinks = _sinks(H, vals)
    scale = 1.0 / math.sqrt(d)
    say(f"[sink] B{B} H{H}/{Hkv} T{T} d{d} W{W} cap{cap} sinks {sinks.tolist()}")
    got = run_gpu_sink(q, k, v, do, sinks, scale, W, cap)
    qf, kf, vf, dof = (synth.to_f64(t) for t in (q, k, v, do))
    s64 = sinks.astype(np.float64)
    ref = EV.full_envelopes(qf, kf, vf, dof, scale, W, cap, sinks=s64)
    o, lse = ref["o"], ref["lse"]
    _, _, _, dsk = OA.attn_bwd(qf, kf, vf, dof, scale, W, cap, sinks=s64)
    errs = {n: check(n, got[n], ref[n], env=ref["E_" + n]) for n in ("o", "lse", "dq", "dk", "dv")}
    # sink gradient: bound by the magnitude sum of its terms
    G = H // Hkv
    Dm = np.sum(dof * o, axis=-1)                              # [B, H, T]
    terms = np.exp(s64[None, :, None] - lse) * Dm
    mag = np.abs(terms).sum(axis=(0, 2))
    derr = np.abs(got["dsinks"] - dsk)
    assert np.all(np.isfinite(got["dsinks"])), got["dsinks"]
    assert np.all(derr <= 2.0 ** -6 * mag + 1e-6), (got["dsinks"], dsk, mag)
    ml = OA.max_logit(qf, kf, scale, W, cap)
    merr = np.abs(got["max_logit"] - ml)
    assert np.all(merr <= 1e-4 * (1.0 + np.abs(ml))), (got["max_logit"], ml)
    say(f"  errors {errs} dsink {float(np.max(derr / (mag + 1e-30))):.2e} "
        f"max_logit {float(merr.max()):.2e} (G={G})")


def test_null_sinks_equal_plain_path():
    """fa_fwd_sink / fa_bwd_sink without sinks or max logit are fa_fwd /
    fa_bwd, bit for bit."""
    from causal_attention_fa_amd import fa
    B, H, Hkv, T, d = 1, 4, 2, 333, 128
    q, k, v, do = _draw(B, H, Hkv, T, d, 1.0, seed=7)
    ref = run_gpu(q, k, v, do, 0.09, 100, 20.0)
    q_, k_, v_, do_ = (t.to(dev()) for t in (q, k, v, do))
    o = poison(q.shape, q.dtype)
    lse = poison((B, H, T), torch.float32)
    fa.fa_fwd_sink(q_, k_, v_, o, lse, None, None, B, H, Hkv, T, d, 0.09, 100, 0, 20.0)
    gq, gk, gv = poison(q.shape, q.dtype), poison(k.shape, k.dtype), poison(v.shape, v.dtype)
    fa.fa_bwd_sink(q_, k_, v_, o, lse, do_, None, gq, gk, gv, None, B, H, Hkv, T, d, 0.09, 100,
                   0, 20.0)
    torch.cuda.synchronize()
    for n, t in dict(o=o, lse=lse, dq=gq, dk=gk, dv=gv).items():
        assert np.array_equal(t.float().cpu().numpy(), ref[n]), n


def test_max_logit_alone_and_very_negative_sink():
    """max_logit without sinks; a sink of -1e4 changes nothing visible
    (exp underflows) and its gradient is 0."""
    from causal_attention_fa_amd import fa
    B, H, Hkv, T, d = 2, 2, 2, 190, 64
    q, k, v, do = _draw(B, H, Hkv, T, d, 2.0, seed=11)
    scale = 0.125
    ref = run_gpu(q, k, v, do, scale, 0, 0.0)
    q_, k_, v_, do_ = (t.to(dev()) for t in (q, k, v, do))
    o = poison(q.shape, q.dtype)
    lse = poison((B, H, T), torch.float32)
    ml = poison((B, H), torch.float32)
    fa.fa_fwd_sink(q_, k_, v_, o, lse, None, ml, B, H, Hkv, T, d, scale, 0, 0, 0.0)
    torch.cuda.synchronize()
    assert np.array_equal(o.float().cpu().numpy(), ref["o"])
    want = OA.max_logit(synth.to_f64(q), synth.to_f64(k), scale, 0, 0.0)
    assert np.allclose(ml.cpu().numpy(), want, rtol=1e-4, atol=1e-4)
    sinks = torch.full((H,), -1e4, dtype=torch.float32, device=dev())
    fa.fa_fwd_sink(q_, k_, v_, o, lse, sinks, ml, B, H, Hkv, T, d, scale, 0, 0, 0.0)
    gq, gk, gv = poison(q.shape, q.dtype), poison(k.shape, k.dtype), poison(v.shape, v.dtype)
    ds = poison((H,), torch.float32)
    fa.fa_bwd_sink(q_, k_, v_, o, lse, do_, sinks, gq, gk, gv, ds, B, H, Hkv, T, d, scale, 0, 0,
                   0.0)
    torch.cuda.synchronize()
    assert np.array_equal(o.float().cpu().numpy(), ref["o"])
    assert np.array_equal(gq.float().cpu().numpy(), ref["dq"])
    assert np.all(ds.cpu().numpy() == 0.0)
