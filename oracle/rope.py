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

__all__ = ["inv_freq", "angles", "rope", "rope_bwd"]


def inv_freq(d: int, theta: float) -> np.ndarray:
    """Host table theta^(-2i/d) for i < d/2, returned as float32.

    Pinned: inv_freq[0] == 1; d = 64, theta = 1e4 gives inv_freq[16] ==
    fl32(0.01); strictly decreasing for theta > 1.
    """
    if d <= 0 or d % 2:
        raise ValueError("d must be even and positive")
    i = np.arange(d // 2, dtype=np.float64)
    return (float(theta) ** (-2.0 * i / d)).astype(np.float32)


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
