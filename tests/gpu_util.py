"""Helpers shared by the GPU parity tests (device setup, NaN poisoning,
error metrics, oracle calls on the exact inputs)."""
import math
import sys

import numpy as np
import torch

from causal_attention_fa_amd import synth
from oracle import attention as OA
from oracle import rope as OR
from tests import envelope as EV

# bf16 bar, per output tensor (o, lse, dq, dk, dv): the oracle's value on
# the exact inputs, rms(gpu - oracle) / rms(oracle) <= 2e-2, and every
# element within 2e-2 * rms(oracle) + E, where E is the envelope that
# tests/envelope.py derives from the roundings the method allows (lse: E
# alone).  fp32 twins: max-abs 1e-4.
BF16_TOL = EV.R_BAR
F32_TOL = 1e-4    # max|gpu - oracle|, per output tensor


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def poison(shape, dtype):
    """Output buffer pre-filled with NaN so an unwritten element fails."""
    return torch.full(shape, float("nan"), dtype=dtype, device=dev())


def max_abs_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not np.all(np.isfinite(got)):
        return float("inf")
    return float(np.max(np.abs(got - ref))) if got.size else 0.0


def check(name, got, ref, f32=False, env=None, qty=None):
    """Assert the parity bar; returns the RMS-relative error (bf16) or the
    max-abs error (fp32).  bf16 needs the element envelope ``env`` (same
    shape as ref); ``qty`` names the output (o, lse, dq, dk, dv; default:
    the name) -- lse has no RMS allowance per element."""
    if f32:
        err = max_abs_err(got, ref)
        assert err <= F32_TOL, f"{name}: max-abs error {err:.3e} > {F32_TOL:.0e}"
        return err
    assert env is not None, f"{name}: a bf16 check needs its envelope"
    err = EV.rms_rel(got, ref)
    assert err <= BF16_TOL, f"{name}: rms-relative error {err:.3e} > {BF16_TOL:.0e}"
    ex = EV.excess(got, ref, env, r_bar=EV.r_bar_for(qty or name))
    assert ex <= 1.0, (f"{name}: an element exceeds 2e-2*rms + its rounding envelope by "
                       f"x{ex:.2f} (max-abs {max_abs_err(got, ref):.3e})")
    return err


def run_gpu(q, k, v, do, scale, window, softcap, global_every=0):
    """fa_fwd + fa_bwd through the C ABI on NaN-poisoned outputs."""
    from causal_attention_fa_amd import fa
    B, H, T, d = q.shape
    Hkv = k.shape[1]
    f32 = q.dtype == torch.float32
    dq_, dk_, dv_ = (t.to(dev()) for t in (q, k, v))
    o = poison(q.shape, q.dtype)
    lse = poison((B, H, T), torch.float32)
    (fa.fa_fwd_f32 if f32 else fa.fa_fwd)(dq_, dk_, dv_, o, lse, B, H, Hkv, T, d, scale,
                                          window, global_every, softcap)
    ddo = do.to(dev())
    gq = poison(q.shape, q.dtype)
    gk = poison(k.shape, k.dtype)
    gv = poison(v.shape, v.dtype)
    (fa.fa_bwd_f32 if f32 else fa.fa_bwd)(dq_, dk_, dv_, o, lse, ddo, gq, gk, gv, B, H, Hkv, T,
                                          d, scale, window, global_every, softcap)
    torch.cuda.synchronize()
    return {n: t.float().cpu().numpy() for n, t in
            dict(o=o, lse=lse, dq=gq, dk=gk, dv=gv).items()}


def oracle_full(q, k, v, do, scale, window, softcap, sinks=None, envelopes=True):
    """Oracle o, lse, dq, dk, dv on the exact inputs; with ``envelopes``
    also their bf16 envelopes E_o .. E_dv (tests/envelope.py)."""
    qf, kf, vf, dof = (synth.to_f64(t) for t in (q, k, v, do))
    if envelopes:
        return EV.full_envelopes(qf, kf, vf, dof, scale, window, softcap, sinks=sinks)
    o, lse = OA.attn_fwd(qf, kf, vf, scale, window, softcap)
    dq, dk, dv = OA.attn_bwd(qf, kf, vf, dof, scale, window, softcap)
    return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)
