"""GPU parity of rope_apply / rope_apply_bwd (bf16 and fp32) against the
float64 oracle: per-element error within 2^-8 of the pair's norm (bf16
output rounding plus fp32 sincos) -- 1e-5 for fp32 -- at T up to 8192 where
angles reach ~8e3 rad; in-place operation; backward inverts forward."""
import numpy as np
import pytest
import torch

from causal_attention_fa_amd import synth
from oracle import rope as OR
from tests.gpu_util import dev, poison, say

pytestmark = pytest.mark.gpu


def _pair_norm(x):
    n = np.sqrt(x[..., 0::2] ** 2 + x[..., 1::2] ** 2)
    return np.repeat(n, 2, axis=-1)


@pytest.mark.parametrize("dtype,B,H,T,d,theta", [
    ("bf16", 2, 3, 513, 64, 1e4), ("bf16", 1, 4, 2048, 128, 1e6),
    ("bf16", 1, 2, 8192, 256, 1e4), ("f32", 2, 2, 300, 128, 1e4),
    ("f32", 1, 2, 8192, 64, 1e6), ("bf16", 1, 2, 33, 6, 1e4), ("f32", 1, 1, 17, 2, 10.0)])
def test_rope_parity(dtype, B, H, T, d, theta):
    from causal_attention_fa_amd import fa
    say(f"[rope] {dtype} B{B} H{H} T{T} d{d} theta{theta:g}")
    w = synth.Workload("rope", dtype, B, H, H, T, d)
    x, _, _, _ = synth.draw(w, need_do=False)
    table = fa.fa_rope_inv_freq(d, theta)
    tab = torch.from_numpy(table).to(dev())
    xd = x.to(dev())
    y = poison(x.shape, x.dtype)
    fa.rope(xd, tab, out=y)
    dx = poison(x.shape, x.dtype)
    fa.rope(y, tab, out=dx, backward=True)
    torch.cuda.synchronize()
    xf = synth.to_f64(x)
    ref = OR.rope(xf, table)
    tol = 1e-5 if dtype == "f32" else 2.0 ** -8
    got = y.double().cpu().numpy()
    err = np.abs(got - ref) / np.maximum(_pair_norm(xf), 1e-30)
    assert np.isfinite(got).all() and err.max() <= tol, err.max()
    # backward of the GPU output against the oracle backward of that output
    yref = synth.to_f64(y.cpu())
    gb = dx.double().cpu().numpy()
    rb = OR.rope_bwd(yref, table)
    errb = np.abs(gb - rb) / np.maximum(_pair_norm(yref), 1e-30)
    assert errb.max() <= tol, errb.max()
    # in place gives the same bits
    xin = x.to(dev())
    fa.rope(xin, tab, out=xin)
    torch.cuda.synchronize()
    assert torch.equal(xin.cpu(), y.cpu())


@pytest.mark.parametrize("theta,factor", [(5e5, 32.0), (1e4, 8.0)])
def test_rope_llama3_table(theta, factor):
    """RoPE with the llama3-rescaled table (host helper) against the oracle's
    own rescaled table and rotation, T = 8192 (angles ~ 8e3 rad)."""
    from causal_attention_fa_amd import fa
    B, H, T, d = 1, 2, 8192, 128
    say(f"[rope llama3] theta{theta:g} factor{factor:g}")
    w = synth.Workload("rope3", "bf16", B, H, H, T, d)
    x, _, _, _ = synth.draw(w, need_do=False)
    tab = torch.from_numpy(fa.fa_rope_inv_freq_llama3(d, theta, factor)).to(dev())
    y = poison(x.shape, x.dtype)
    fa.rope(x.to(dev()), tab, out=y)
    torch.cuda.synchronize()
    xf = synth.to_f64(x)
    ref = OR.rope(xf, OR.inv_freq_llama3(d, theta, factor))
    err = np.abs(y.double().cpu().numpy() - ref) / np.maximum(_pair_norm(xf), 1e-30)
    assert err.max() <= 2.0 ** -8, err.max()
