"""GPU parity of fa_fwd / fa_bwd (and the fp32 twins) against the float64
oracle, element by element, at sizes that span several tiles and ragged
tails, with the edge cases of the method: T = 1, windows 1, 2, T-1, T, 2T,
window edges inside a tile, GQA ratios 1..16, H = 7, softcap on and off,
d = 64, 128, 256.  Outputs are NaN-poisoned first so an unwritten element
fails; each case also runs twice and must be bitwise identical (no atomics
on this path)."""
import math

import numpy as np
import pytest
import torch

from causal_attention_fa_amd import synth
from tests.gpu_util import check, oracle_full, run_gpu, say

pytestmark = pytest.mark.gpu

# (B, H, Hkv, T, d, window, softcap, sigma_qk)
BF16_CASES = [
    (1, 2, 2, 1, 64, 0, 0.0, 1.0),
    (1, 2, 1, 2, 128, 0, 0.0, 1.0),
    (2, 4, 2, 63, 64, 0, 0.0, 1.0),
    (1, 4, 4, 65, 128, 0, 2.0, 1.0),
    (1, 2, 1, 127, 256, 0, 0.0, 1.0),
    (1, 7, 7, 129, 64, 64, 0.0, 1.0),
    (1, 8, 2, 300, 128, 65, 0.0, 1.0),
    (1, 4, 1, 300, 256, 100, 50.0, 2.0),
    (2, 2, 2, 257, 128, 1, 0.0, 1.0),
    (1, 2, 2, 200, 64, 2, 5.0, 2.0),
    (1, 2, 2, 200, 128, 199, 0.0, 1.0),
    (1, 2, 2, 200, 128, 200, 0.0, 1.0),
    (1, 2, 2, 200, 128, 400, 0.0, 1.0),
    (1, 4, 2, 1000, 128, 0, 0.0, 1.0),
    (1, 2, 1, 515, 256, 0, 30.0, 2.0),
    (1, 8, 8, 1000, 64, 300, 0.0, 1.0),
    (1, 8, 1, 384, 128, 128, 50.0, 2.0),
    (1, 4, 2, 640, 256, 257, 0.0, 1.0),
    (1, 16, 1, 700, 64, 0, 0.0, 1.0),
    (1, 32, 2, 333, 128, 100, 20.0, 2.0),
    # d = 256 workgroups with an odd number of key units (ragged last block,
    # short windows): the last step's parity branch joins after the O MFMAs
    (1, 7, 1, 600, 256, 1, 0.0, 1.0),
    (2, 4, 1, 191, 256, 10, 30.0, 2.0),
]

F32_CASES = [
    (1, 2, 2, 128, 64, 0, 0.0, 1.0),
    (1, 4, 2, 100, 128, 30, 2.0, 2.0),
    (1, 2, 1, 67, 256, 0, 50.0, 2.0),
    (2, 2, 2, 1, 64, 0, 0.0, 1.0),
    (1, 3, 3, 129, 64, 1, 0.0, 1.0),
]


def _inputs(B, H, Hkv, T, d, sigma, dtype, seed):
    w = synth.Workload("case", dtype, B, H, Hkv, T, d, sigma_qk=sigma, seed=seed)
    return synth.draw(w)


CASES = [("bf16",) + c for c in BF16_CASES] + [("f32",) + c for c in F32_CASES]


@pytest.mark.parametrize("case", CASES, ids=[
    f"{c[0]}-B{c[1]}H{c[2]}/{c[3]}T{c[4]}d{c[5]}W{c[6]}cap{c[7]:g}" for c in CASES])
def test_parity_vs_oracle(case):
    dtype, B, H, Hkv, T, d, W, cap, sig = case
    f32 = dtype == "f32"
    q, k, v, do = _inputs(B, H, Hkv, T, d, sig, dtype, seed=CASES.index(case))
    scale = 1.0 / math.sqrt(d)
    say(f"[parity] {dtype} B{B} H{H}/{Hkv} T{T} d{d} W{W} cap{cap}")
    got = run_gpu(q, k, v, do, scale, W, cap)
    ref = oracle_full(q, k, v, do, scale, W, cap, envelopes=not f32)
    errs = {n: check(n, got[n], ref[n], f32, env=ref.get("E_" + n))
            for n in ("o", "lse", "dq", "dk", "dv")}
    say(f"  errors {errs}")
    again = run_gpu(q, k, v, do, scale, W, cap)
    for n in got:
        assert np.array_equal(got[n], again[n]), f"{n} not deterministic"


def test_window_at_least_T_matches_causal_on_gpu():
    q, k, v, do = _inputs(1, 4, 2, 333, 128, 1.0, "bf16", seed=5)
    a = run_gpu(q, k, v, do, 0.1, 0, 0.0)
    b = run_gpu(q, k, v, do, 0.1, 333, 0.0)
    c = run_gpu(q, k, v, do, 0.1, 5000, 0.0)
    for n in a:
        assert np.array_equal(a[n], b[n]) and np.array_equal(a[n], c[n]), n


def test_single_unit_after_nan_lds():
    """Workgroups whose key (or query) range is one unit still compute their
    first step's next tiles; those must come from zero-filling loads, never
    from stale LDS (a masked P of 0 times a NaN left there is NaN).  Each
    one-unit shape runs before and after a pass over NaN K and V on every CU
    (which leaves NaN tiles in LDS): the outputs must be finite and bitwise
    identical (the kernels are deterministic; their accuracy on these shapes
    is the parity cases' business)."""
    for d in (128, 256):
        shapes = [(T, _inputs(1, 2, 1, T, d, 1.0, "bf16", seed=12 + T)) for T in (2, 31)]
        before = [run_gpu(*x, d ** -0.5, 0, 0.0) for _, x in shapes]
        q, k, v, do = _inputs(1, 32, 8, 1024, d, 1.0, "bf16", seed=11)
        k[:] = float("nan")
        v[:] = float("nan")
        say(f"[stale-lds] NaN pass d{d}")
        run_gpu(q, k, v, do, d ** -0.5, 0, 0.0)
        for (T, x), a in zip(shapes, before):
            say(f"[stale-lds] T{T} d{d}")
            b = run_gpu(*x, d ** -0.5, 0, 0.0)
            for n in ("o", "lse", "dq", "dk", "dv"):
                assert np.isfinite(b[n]).all(), f"{n} not finite (T={T}, d={d})"
                assert np.array_equal(a[n], b[n]), f"{n} depends on LDS contents (T={T}, d={d})"


def test_nan_input_propagates_not_hangs():
    q, k, v, do = _inputs(1, 2, 2, 130, 64, 1.0, "bf16", seed=6)
    q[0, 0, 100, 3] = float("nan")
    got = run_gpu(q, k, v, do, 0.125, 0, 0.0)
    assert np.isnan(got["o"][0, 0, 100]).all()
    assert np.isfinite(got["o"][0, 0, :100]).all()
    assert np.isfinite(got["o"][0, 1]).all()
