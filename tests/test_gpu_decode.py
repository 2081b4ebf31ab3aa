"""GPU parity of fa_decode (single-query decode over a preallocated KV cache,
split along the cache) against the float64 decode oracle.

Small cases compare every output; the cache positions at or past each
sequence's length are filled with NaN, so any read of them fails.  Lengths
cover 0, 1, a tile edge +-1 and S; windows 1, inside a tile and past S;
GQA ratios 1..32; d 64, 128, 256; cap on/off; sinks; several chunks; both
split-kernel shapes at d = 128 (two waves per workgroup, and one wave when
there are many (b, KV head, chunk) units).  The full-size qwen25-decode
workload is checked on sampled sequences."""
import math

import numpy as np
import pytest
import torch

from causal_attention_fa_amd import synth
from oracle import decode as OD
from tests import envelope as EV
from tests.gpu_util import check, dev, poison, say

pytestmark = pytest.mark.gpu

# (B, H, Hkv, S, d, window, cap, sinks?, lens)
CASES = [
    (1, 2, 2, 1, 64, 0, 0.0, False, [1]),
    (4, 4, 2, 70, 64, 0, 0.0, False, [1, 31, 33, 70]),
    (3, 8, 1, 300, 128, 0, 0.0, True, [300, 32, 0]),
    (2, 28, 4, 1000, 128, 0, 0.0, False, [1000, 517]),
    (2, 8, 2, 777, 128, 100, 0.0, False, [777, 64]),
    (2, 4, 4, 260, 128, 1, 30.0, True, [260, 5]),
    (2, 8, 4, 900, 256, 0, 50.0, False, [900, 257]),
    (1, 4, 2, 5000, 256, 4096, 50.0, True, [4999]),
    (1, 32, 8, 4100, 128, 0, 0.0, False, [4100]),
    (2, 2, 1, 3000, 64, 5000, 0.0, False, [3000, 2999]),
    (1, 32, 1, 600, 128, 0, 0.0, False, [600]),
    (2, 64, 2, 300, 64, 100, 20.0, True, [300, 150]),
    (1, 32, 1, 2000, 256, 0, 50.0, False, [1999]),
    # chunks wholly past a short sequence's length (empty chunks) beside a sink
    (2, 8, 2, 3000, 128, 0, 0.0, True, [3000, 100]),
    # enough (b, KV head, chunk) units (12 x 64 x 3) for the one-wave split at d = 128
    (12, 64, 64, 3000, 128, 0, 0.0, False,
     [3000, 1, 1500, 2999, 1025, 1023, 0, 2048, 3000, 17, 2500, 1999]),
]


def _draw(B, H, Hkv, S, d, seed, sigma=1.0):
    w = synth.DecodeWorkload("case", B, H, Hkv, S, d, sigma_qk=sigma, seed=seed)
    q, k, v, _ = synth.draw_decode(w, device="cpu")
    return q, k, v


def run_decode(q, k, v, lens, sinks, scale, window, cap):
    from causal_attention_fa_amd import fa
    B, H, d = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    q_, k_, v_ = (t.to(dev()) for t in (q, k, v))
    l_ = torch.tensor(lens, dtype=torch.int32, device=dev())
    s_ = None if sinks is None else torch.from_numpy(sinks).to(dev())
    o = poison((B, H, d), torch.bfloat16)
    lse = poison((B, H), torch.float32)
    fa.fa_decode(q_, k_, v_, l_, o, lse, s_, B, H, Hkv, S, d, scale, window, cap)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("case", CASES, ids=[
    f"B{c[0]}H{c[1]}/{c[2]}S{c[3]}d{c[4]}W{c[5]}cap{c[6]:g}{'sink' if c[7] else ''}"
    for c in CASES])
def test_decode_parity_vs_oracle(case):
    from causal_attention_fa_amd import fa
    B, H, Hkv, S, d, W, cap, use_sink, lens = case
    q, k, v = _draw(B, H, Hkv, S, d, seed=200 + CASES.index(case), sigma=2.0 if cap else 1.0)
    for b, n in enumerate(lens):     # positions past the length must never be read
        k[b, :, n:] = float("nan")
        v[b, :, n:] = float("nan")
    sinks = (np.linspace(-1.0, 2.0, H).astype(np.float32) if use_sink else None)
    scale = 1.0 / math.sqrt(d)
    ns, ch = fa.fa_decode_splits(B, Hkv, S, W)
    say(f"[decode] B{B} H{H}/{Hkv} S{S} d{d} W{W} cap{cap} sink{use_sink} lens {lens} "
        f"chunks {ns}x{ch}")
    o, lse = run_decode(q, k, v, lens, sinks, scale, W, cap)
    kf, vf = synth.to_f64(k), synth.to_f64(v)
    ro, rl = OD.decode(synth.to_f64(q), np.nan_to_num(kf), np.nan_to_num(vf), lens, scale, W, cap,
                       None if sinks is None else sinks.astype(np.float64))
    live = np.array(lens) > 0
    if (~live).any():
        assert np.all(o[~live] == 0.0)
        want = -np.inf if sinks is None else None
        for b in np.nonzero(~live)[0]:
            if want is None:
                np.testing.assert_allclose(lse[b], sinks, rtol=1e-6)
            else:
                assert np.all(np.isneginf(lse[b]))
    Eo, El = EV.decode_envelopes(synth.to_f64(q), np.nan_to_num(kf), np.nan_to_num(vf), lens,
                                 scale, W, cap, None if sinks is None else sinks.astype(np.float64))
    errs = dict(o=check("o", o[live], ro[live], env=Eo[live]),
                lse=check("lse", lse[live], rl[live], env=El[live]))
    say(f"  errors {errs}")
    o2, l2 = run_decode(q, k, v, lens, sinks, scale, W, cap)
    assert np.array_equal(o, o2) and np.array_equal(lse, l2, equal_nan=True), "not deterministic"


def test_decode_full_size_sampled():
    """qwen25-decode (B32 H28/4, 32k cache, ragged lengths) at full size;
    the oracle evaluates three sequences."""
    from causal_attention_fa_amd import fa
    w = synth.DECODE_WORKLOADS["qwen25-decode"]
    q, k, v, lens = synth.draw_decode(w, device=dev())
    o = poison((w.B, w.H, w.d), torch.bfloat16)
    lse = poison((w.B, w.H), torch.float32)
    say(f"[decode full] {w}")
    fa.fa_decode(q, k, v, lens, o, lse, None, w.B, w.H, w.Hkv, w.S, w.d, w.scale, w.window,
                 w.softcap)
    torch.cuda.synchronize()
    lens_h = lens.cpu().numpy()
    o_h, l_h = o.float().cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.isfinite(o_h)) and np.all(np.isfinite(l_h))
    for b in (0, int(np.argmax(lens_h)), w.B - 1):
        n = int(lens_h[b])
        kb = synth.to_f64(k[b:b + 1, :, :n].cpu())
        vb = synth.to_f64(v[b:b + 1, :, :n].cpu())
        qb = synth.to_f64(q[b:b + 1].cpu())
        ro, rl = OD.decode(qb, kb, vb, [n], w.scale, w.window, w.softcap)
        Eo, El = EV.decode_envelopes(qb, kb, vb, [n], w.scale, w.window, w.softcap)
        e1 = check("o", o_h[b:b + 1], ro, env=Eo)
        e2 = check("lse", l_h[b:b + 1], rl, env=El)
        say(f"  b={b} len={n} errors o {e1:.2e} lse {e2:.2e}")
