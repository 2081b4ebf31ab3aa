"""fa_bwd_noalloc (the backward with its row statistics in a fixed device
array, for callers that cannot allocate) against fa_bwd through the C ABI:
two calls in a row, the second on a smaller input, each bit for bit equal to
fa_bwd under dQ mode 1 on the same inputs (the same kernels run; only where
D lives differs); against fa_bwd in the default mode (dQ from stored dS at
d = 128) dk and dv bit for bit, and all three within the oracle's bf16
envelope."""
import math

import numpy as np
import pytest
import torch

from causal_attention_fa_amd import synth
from tests.gpu_util import check, dev, oracle_full, poison, say

pytestmark = pytest.mark.gpu


def _bwd(fn, q, k, v, o, lse, do, w):
    gq, gk, gv = poison(q.shape, q.dtype), poison(k.shape, k.dtype), poison(v.shape, v.dtype)
    fn(q, k, v, o, lse, do, gq, gk, gv, w.B, w.H, w.Hkv, w.T, w.d, w.scale, w.window, 0,
       w.softcap)
    torch.cuda.synchronize()
    return {n: t.float().cpu().numpy() for n, t in dict(dq=gq, dk=gk, dv=gv).items()}


def test_noalloc_matches_fa_bwd_twice():
    from causal_attention_fa_amd import fa
    cases = [synth.Workload("na1", "bf16", 2, 8, 2, 1100, 128, window=300, softcap=20.0,
                            sigma_qk=2.0, seed=31),
             synth.Workload("na2", "bf16", 1, 4, 4, 333, 256, seed=32)]   # smaller second call
    for w in cases:
        say(f"[noalloc] B{w.B} H{w.H}/{w.Hkv} T{w.T} d{w.d} W{w.window} cap{w.softcap}")
        q, k, v, do = synth.draw(w)
        qd, kd, vd, dod = (t.to(dev()) for t in (q, k, v, do))
        o = poison(q.shape, q.dtype)
        lse = poison((w.B, w.H, w.T), torch.float32)
        fa.fa_fwd(qd, kd, vd, o, lse, w.B, w.H, w.Hkv, w.T, w.d, w.scale, w.window, 0, w.softcap)
        dflt = _bwd(fa.fa_bwd, qd, kd, vd, o, lse, dod, w)
        prev = fa.fa_set_dq_mode(1)
        try:
            ref = _bwd(fa.fa_bwd, qd, kd, vd, o, lse, dod, w)
        finally:
            fa.fa_set_dq_mode(prev)
        got = _bwd(fa.fa_bwd_noalloc, qd, kd, vd, o, lse, dod, w)
        for n in got:
            assert np.array_equal(got[n], ref[n]), f"{n}: fa_bwd_noalloc differs from fa_bwd"
        for n in ("dk", "dv"):
            assert np.array_equal(got[n], dflt[n]), f"{n}: differs from the default-mode fa_bwd"
        orc = oracle_full(q, k, v, do, w.scale, w.window, w.softcap)
        check("dq(default mode)", dflt["dq"], orc["dq"], env=orc["E_dq"])
        errs = {n: check(n, got[n], orc[n], env=orc["E_" + n]) for n in got}
        say(f"  equal to fa_bwd; oracle rms-relative {errs}")
