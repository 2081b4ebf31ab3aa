"""GPU parity of fa_fwd_vdim / fa_bwd_vdim (value head size d_v different
from the query/key head size d: the decompressed MLA head, d = 192,
d_v = 128, scale 1/sqrt(192)) against the float64 oracle, over tile
tails, GQA, windows and the softcap; with d == d_v the entry points must be
fa_fwd / fa_bwd bit for bit; the full-size mla workload is checked on
sampled rows."""
import math

import numpy as np
import pytest
import torch

from causal_attention_fa_amd import synth
from oracle import attention as OA
from tests import envelope as EV
from tests.gpu_util import check, dev, oracle_full, poison, run_gpu, say

pytestmark = pytest.mark.gpu

# (B, H, Hkv, T, window, softcap, sigma_qk)
CASES = [
    (1, 2, 2, 1, 0, 0.0, 1.0),
    (1, 2, 1, 33, 0, 0.0, 1.0),
    (2, 4, 4, 130, 0, 0.0, 1.0),
    (1, 4, 2, 300, 70, 0.0, 1.0),
    (1, 2, 2, 257, 1, 20.0, 2.0),
    (1, 8, 2, 640, 0, 50.0, 2.0),
    (1, 2, 2, 1000, 300, 0.0, 1.0),
]
DK, DV = 192, 128


def run_vdim(q, k, v, do, scale, window, cap):
    from causal_attention_fa_amd import fa
    B, H, T, d = q.shape
    Hkv, dv = k.shape[1], v.shape[-1]
    q_, k_, v_, do_ = (t.to(dev()) for t in (q, k, v, do))
    o = poison((B, H, T, dv), torch.bfloat16)
    lse = poison((B, H, T), torch.float32)
    fa.fa_fwd_vdim(q_, k_, v_, o, lse, B, H, Hkv, T, d, dv, scale, window, 0, cap)
    gq, gk, gv = poison(q.shape, q.dtype), poison(k.shape, k.dtype), poison(v.shape, v.dtype)
    fa.fa_bwd_vdim(q_, k_, v_, o, lse, do_, gq, gk, gv, B, H, Hkv, T, d, dv, scale, window, 0,
                   cap)
    torch.cuda.synchronize()
    return {n: t.float().cpu().numpy() for n, t in
            dict(o=o, lse=lse, dq=gq, dk=gk, dv=gv).items()}


def _draw(B, H, Hkv, T, sig, seed):
    w = synth.Workload("vdim", "bf16", B, H, Hkv, T, DK, sigma_qk=sig, seed=seed, d_v=DV)
    return synth.draw(w)


@pytest.mark.parametrize("case", CASES, ids=[
    f"B{c[0]}H{c[1]}/{c[2]}T{c[3]}W{c[4]}cap{c[5]:g}" for c in CASES])
def test_vdim_parity_vs_oracle(case):
    B, H, Hkv, T, W, cap, sig = case
    q, k, v, do = _draw(B, H, Hkv, T, sig, seed=300 + CASES.index(case))
    scale = 1.0 / math.sqrt(DK)
    say(f"[vdim] B{B} H{H}/{Hkv} T{T} d{DK}/{DV} W{W} cap{cap}")
    got = run_vdim(q, k, v, do, scale, W, cap)
    ref = oracle_full(q, k, v, do, scale, W, cap)
    errs = {n: check(n, got[n], ref[n], env=ref["E_" + n]) for n in ("o", "lse", "dq", "dk", "dv")}
    say(f"  errors {errs}")
    again = run_vdim(q, k, v, do, scale, W, cap)
    for n in got:
        assert np.array_equal(got[n], again[n]), f"{n} not deterministic"


@pytest.mark.parametrize("d", [64, 128, 256])
def test_equal_sizes_match_plain_entry_points(d):
    w = synth.Workload("eq", "bf16", 1, 4, 2, 200, d, window=50, softcap=10.0, seed=9)
    q, k, v, do = synth.draw(w)
    a = run_gpu(q, k, v, do, w.scale, w.window, w.softcap)
    b = run_vdim(q, k, v, do, w.scale, w.window, w.softcap)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


def test_unsupported_pair_is_rejected():
    from causal_attention_fa_amd import fa
    t = torch.zeros(1 << 16, dtype=torch.bfloat16, device=dev())
    lse = torch.zeros(1 << 10, dtype=torch.float32, device=dev())
    with pytest.raises(fa.FAError) as e:
        fa.fa_fwd_vdim(t[:4096], t[8192:12288], t[16384:20480], t[24576:28672], lse,
                       1, 1, 1, 8, 128, 64, 0.1)
    assert e.value.code == fa.FA_ERR_UNSUPPORTED


def test_mla_full_size():
    """mla workload (B2 H16 T8192 d192/128) at full size: o and lse on every
    row of every (b, h); dq, dk, dv on sampled rows of four heads."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    w = synth.WORKLOADS["mla"]
    q, k, v, do = synth.draw(w)
    say(f"[mla full] {w}")
    got = run_vdim(q, k, v, do, w.scale, w.window, w.softcap)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    grad_heads = {(0, 0), (1, 15), (0, 7), (1, 3)}
    q_rows = np.array([0, 5, 31, 32, 2047, 4096, 6000, 8191])
    kv_rows = np.array([0, 1, 100, 4095, 4096, 8191])

    def one(bh):
        b, h = bh
        qf, kf, vf, dof = (synth.to_f64(t) for t in (q[b, h], k[b, h], v[b, h], do[b, h]))
        if bh in grad_heads:
            return bh, EV.head_envelopes(qf, kf, vf, dof, w.scale, 0, 0.0, q_rows=q_rows,
                                         kv_rows=kv_rows)
        return bh, EV.head_envelopes(qf, kf, vf, None, w.scale, 0, 0.0)

    with threadpool_limits(1), ThreadPoolExecutor(16) as ex:
        res = dict(ex.map(one, heads))
    for (b, h), r in res.items():
        check(f"o[{b},{h}]", got["o"][b, h], r["o"], env=r["E_o"], qty="o")
        check(f"lse[{b},{h}]", got["lse"][b, h], r["lse"], env=r["E_lse"], qty="lse")
        if (b, h) in grad_heads:
            kvc = EV.combine_kv([r])     # H = Hkv: one query head per KV head
            check(f"dq[{b},{h}]", got["dq"][b, h][q_rows], r["dq"], env=r["E_dq"], qty="dq")
            check(f"dk[{b},{h}]", got["dk"][b, h][kv_rows], kvc["dk"], env=kvc["E_dk"], qty="dk")
            check(f"dv[{b},{h}]", got["dv"][b, h][kv_rows], kvc["dv"], env=kvc["E_dv"], qty="dv")
    say(f"  {len(heads)} heads: o, lse every row; grads on {sorted(grad_heads)}")
