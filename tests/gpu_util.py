"""Helpers shared by the GPU parity tests (device setup, NaN poisoning,
error metrics, oracle calls on the exact inputs)."""
import math
import sys

import numpy as np
import torch

from causal_attention_fa_amd import synth
from oracle import attention as OA
from oracle import rope as OR

# bf16 bar, per output tensor (o, lse, dq, dk, dv):
#   rms(gpu - oracle) / rms(oracle) <= 2e-2  (the bar), and, as a guard
#   against localized errors that an RMS can average away, every element
#   within 0.1 * rms(oracle) + 2^-6 * |oracle|.
# The max-abs / rms reading of "2e-2 relative to the output's RMS" is not
# attainable by any bf16-output implementation: rounding the exact float64
# result to bf16 alone gives max|err| / rms up to ~0.09 at T = 1000 (large
# early-row outputs, small RMS).  The guard's 0.1 * rms covers the
# standard bf16 backward's element errors (dS rounded to bf16, D from the
# bf16 o), measured at up to ~0.08 * rms in rows with few visible keys.
BF16_TOL = 2e-2
BF16_ELEM_RMS = 0.1
BF16_ELEM_REL = 2.0 ** -6
F32_TOL = 1e-4    # max|gpu - oracle|, per output tensor


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def poison(shape, dtype):
    """Output buffer pre-filled with NaN so an unwritten element fails."""
    return torch.full(shape, float("nan"), dtype=dtype, device=dev())


def rel_rms_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if not np.all(np.isfinite(got)):
        return float("inf")
    rms = math.sqrt(float(np.mean(ref * ref))) or 1.0
    return float(np.max(np.abs(got - ref))) / rms


def max_abs_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not np.all(np.isfinite(got)):
        return float("inf")
    return float(np.max(np.abs(got - ref))) if got.size else 0.0


def rms_rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not np.all(np.isfinite(got)):
        return float("inf")
    rms = math.sqrt(float(np.mean(ref * ref))) or 1.0
    return math.sqrt(float(np.mean((got - ref) ** 2))) / rms


def elem_excess(got, ref):
    """max over elements of |err| / (0.1 rms(ref) + 2^-6 |ref|)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not np.all(np.isfinite(got)):
        return float("inf")
    rms = math.sqrt(float(np.mean(ref * ref))) or 1.0
    bound = BF16_ELEM_RMS * rms + BF16_ELEM_REL * np.abs(ref)
    return float(np.max(np.abs(got - ref) / bound)) if got.size else 0.0


def check(name, got, ref, f32, elem_guard=True):
    """Assert the parity bar; returns the headline error figure.  elem_guard
    False keeps only the RMS bar (end-to-end chains whose inputs differ by
    the bf16 rounding of an intermediate, which is not a kernel error)."""
    if f32:
        err = max_abs_err(got, ref)
        assert err <= F32_TOL, f"{name}: max-abs error {err:.3e} > {F32_TOL:.0e}"
        return err
    err = rms_rel_err(got, ref)
    assert err <= BF16_TOL, f"{name}: rms-relative error {err:.3e} > {BF16_TOL:.0e}"
    ex = elem_excess(got, ref) if elem_guard else 0.0
    assert ex <= 1.0, (f"{name}: an element exceeds 0.1*rms + 2^-6*|ref| by x{ex:.2f} "
                       f"(max-abs/rms {rel_rms_err(got, ref):.3e})")
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


def oracle_full(q, k, v, do, scale, window, softcap):
    qf, kf, vf, dof = (synth.to_f64(t) for t in (q, k, v, do))
    o, lse = OA.attn_fwd(qf, kf, vf, scale, window, softcap)
    dq, dk, dv = OA.attn_bwd(qf, kf, vf, dof, scale, window, softcap)
    return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)
