"""Float64 definition of rotary position embedding on interleaved pairs.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Forge README (commit "Add HF streaming data pipeline and three research
reports"): RoPE rotates interleaved pairs, i.e. (x[2i], x[2i+1]).  Forge
attention.h commit log, "Wave 1": the RoPE kernels read a frequency table
computed on the host instead of computing frequencies inline; the table is
also what carries a per-layer theta (rope_theta / rope_theta_global).

Readings where the pages are silent:
  * inv_freq[i] = theta^(-2i/d), i < d/2 (the standard form; the pages never
    print it), evaluated in float64 and stored as float32;
  * position t = 0 .. T-1 along the sequence axis, no offset;
  * the angle is the float32 product fl32(t * inv_freq_f32[i]) (what a kernel
    reading a float32 table computes); cos/sin of that angle are taken in
    float64 here;
  * forward rotates by +angle:
        y[2i]   = x[2i] cos - x[2i+1] sin
        y[2i+1] = x[2i] sin + x[2i+1] cos
    backward (the transpose) rotates the gradient by -angle.
"""
from __future__ import annotations

import numpy as np

__all__ = ["inv_freq", "inv_freq_llama3", "layer_rope_theta", "angles", "rope", "rope_bwd"]


def inv_freq(d: int, theta: float) -> np.ndarray:
    """Host table theta^(-2i/d) for i < d/2, returned as float32.

    Pinned: inv_freq[0] == 1; d = 64, theta = 1e4 gives inv_freq[16] ==
    fl32(0.01); strictly decreasing for theta > 1.
    """
    if d <= 0 or d % 2:
        raise ValueError("d must be even and positive")
    i = np.arange(d // 2, dtype=np.float64)
    return (float(theta) ** (-2.0 * i / d)).astype(np.float32)


def inv_freq_llama3(d: int, theta: float, factor: float, low: float = 1.0,
                    high: float = 4.0, orig_ctx: float = 8192.0) -> np.ndarray:
    """Inverse frequencies with the "llama3" context-extension rescaling.

    Forge ARCHITECTURES.md, "Formules clés" (llama3 RoPE scaling, applied
    per component): with wavelen = 2*pi/inv_freq, components whose
    wavelength is shorter than orig_ctx/high keep their frequency, those
    longer than orig_ctx/low are divided by `factor`, and in between the
    two are blended with s = (orig_ctx/wavelen - low)/(high - low):
    (1-s)*inv_freq/factor + s*inv_freq.  Config defaults (forge-studio
    RESEARCH.md section 2): low 1, high 4, orig_ctx 8192; factor 0 = off.
    Evaluated in float64, stored as float32.

    Pinned: factor 1 and factor 0 give the plain table; components in the
    high-frequency band are unchanged and those in the low band are exactly
    inv_freq/factor; the blend meets both bands continuously at the two
    thresholds; the scaled table stays strictly decreasing.
    """
    if d <= 0 or d % 2:
        raise ValueError("d must be even and positive")
    base = (float(theta) ** (-2.0 * np.arange(d // 2, dtype=np.float64) / d))
    if factor <= 0:
        return base.astype(np.float32)
    if not (high > low > 0) or orig_ctx <= 0:
        raise ValueError("need high > low > 0 and orig_ctx > 0")
    return _llama3_scale(base, factor, low, high, orig_ctx).astype(np.float32)


def _llama3_scale(inv, factor, low, high, orig_ctx):
    inv = np.asarray(inv, dtype=np.float64)
    wavelen = 2.0 * np.pi / inv
    s = (orig_ctx / wavelen - low) / (high - low)
    blended = (1.0 - s) * inv / factor + s * inv
    out = np.where(wavelen > orig_ctx / low, inv / factor, blended)
    return np.where(wavelen < orig_ctx / high, inv, out)


def layer_rope_theta(layer: int, theta: float, theta_global: float,
                     global_every: int) -> float:
    """RoPE base of one layer of a local:global stack: global layers (every
    global_every-th layer, as for the attention window) use theta_global
    when it is set (> 0), every other layer uses theta.  Forge attention.h
    commit log, "Wave 2": rope_theta_global gives Gemma 3 its dual base
    (ARCHITECTURES.md family table: 10k local / 1M global).

    Pinned: the Gemma 3 pattern with global_every 6; theta_global 0 leaves
    every layer at theta.
    """
    if layer < 0 or global_every < 0:
        raise ValueError("layer and global_every must be >= 0")
    if theta_global > 0 and global_every > 0 and (layer + 1) % global_every == 0:
        return float(theta_global)
    return float(theta)


def angles(T: int, table_f32: np.ndarray) -> np.ndarray:
    """[T, d/2] float32 angles fl32(t * inv_freq[i])."""
    t = np.arange(T, dtype=np.float32)[:, None]
    return t * np.asarray(table_f32, dtype=np.float32)[None, :]


def _rotate(x, table_f32, sign):
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[-2]
    ang = angles(T, table_f32).astype(np.float64)
    c = np.cos(ang)
    s = sign * np.sin(ang)
    xe = x[..., 0::2]
    xo = x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = xe * c - xo * s
    y[..., 1::2] = xe * s + xo * c
    return y


def rope(x, table_f32):
    """Rotate x [..., T, d] (pairs (2i, 2i+1)) by +t*inv_freq[i].

    Pinned: t = 0 identity; pair norms preserved; equals multiplication of
    the complex numbers x[2i] + 1j*x[2i+1] by exp(1j*angle); relative
    position property <R_m q, R_n k> = <q, R_(n-m) k> for exact angles.
    """
    return _rotate(x, table_f32, 1.0)


def rope_bwd(dy, table_f32):
    """Gradient of rope: rotate dy by -t*inv_freq[i].

    Pinned: rope_bwd(rope(x)) == x; adjoint <rope(x), y> == <x, rope_bwd(y)>.
    """
    return _rotate(dy, table_f32, -1.0)
