"""GPU parity of fa_fwd / fa_bwd on seeded random shapes at tile edges.

The hand-picked cases of test_gpu_attention.py cover the method's edge cases;
these add shapes drawn from sizes one below, at and one above the kernels'
tile multiples (32, 64, 128 rows and keys), with windows drawn from the same
sizes and from T - 1, T, T + 1, softcap on and off, GQA ratios 1 to 7, and
d = 64, 128, 256.  Workgroups then end on ragged key and query ranges with
odd and even numbers of units, the case that once exposed a missing wait in
the d = 256 forward.  Same bar as the other parity tests: every element
against the float64 oracle within the derived bf16 envelope."""
import math
import random

import pytest

from causal_attention_fa_amd import synth
from tests.gpu_util import check, oracle_full, run_gpu, say

pytestmark = pytest.mark.gpu

EDGE = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 191, 192, 193, 255, 256, 257, 383, 384, 385,
        511, 512, 513, 639, 640, 641]


def _cases(n, seed=20261203):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        d = rng.choice([64, 128, 256, 256])
        T = rng.choice(EDGE)
        W = rng.choice([0, 0] + [w for w in EDGE if w <= T + 1] + [max(T - 1, 0), T, T + 1])
        cap = rng.choice([0.0, 0.0, 5.0, 50.0])
        Hkv = rng.choice([1, 2])
        G = rng.choice([1, 2, 4, 7])
        B = rng.choice([1, 2]) if T <= 256 else 1
        out.append((B, Hkv * G, Hkv, T, d, W, cap, rng.randint(0, 10**6)))
    return out


CASES = _cases(28)


@pytest.mark.parametrize("case", CASES, ids=[
    f"B{c[0]}H{c[1]}/{c[2]}T{c[3]}d{c[4]}W{c[5]}cap{c[6]:g}s{c[7]}" for c in CASES])
def test_random_shape_parity(case):
    B, H, Hkv, T, d, W, cap, seed = case
    w = synth.Workload("rand", "bf16", B, H, Hkv, T, d, sigma_qk=2.0 if cap else 1.0, seed=seed)
    q, k, v, do = synth.draw(w)
    scale = 1.0 / math.sqrt(d)
    say(f"[random] B{B} H{H}/{Hkv} T{T} d{d} W{W} cap{cap} seed{seed}")
    got = run_gpu(q, k, v, do, scale, W, cap)
    ref = oracle_full(q, k, v, do, scale, W, cap)
    errs = {n: check(n, got[n], ref[n], env=ref["E_" + n]) for n in ("o", "lse", "dq", "dk", "dv")}
    say(f"  errors {errs}")
