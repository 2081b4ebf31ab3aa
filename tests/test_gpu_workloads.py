"""Full-size parity of every workload, in the launch configuration the
benchmark times, against the float64 oracle on sampled outputs.

For each workload the whole GPU path runs at full size (RoPE on Q and K
first where the workload has it, fa_fwd, fa_bwd, RoPE backward on dQ and
dK).  The oracle then evaluates, for two sampled (batch, KV-head) groups,
every query head of the group: o and lse on all rows, dq on sampled rows,
and the group's dk, dv on sampled key rows (their exact definition needs
the lse and D of every query row, which the oracle computes).  RoPE
workloads are checked twice: stage-isolated (the oracle attends over the
GPU's bf16 RoPE output) and end to end (the oracle applies its own RoPE
to the original inputs and rotates the gradients back).  forge-f32 is small
and is compared on every element at 1e-4.
"""
import math

import numpy as np
import pytest
import torch

from causal_attention_fa_amd import synth
from oracle import attention as OA
from oracle import rope as OR
from tests.gpu_util import check, dev, poison, say

pytestmark = pytest.mark.gpu


def _gpu_path(w, q, k, v, do, softcap):
    """The benchmarked step on device tensors; returns device tensors."""
    from causal_attention_fa_amd import fa
    B, H, Hkv, T, d = w.B, w.H, w.Hkv, w.T, w.d
    f32 = w.dtype == "f32"
    qd, kd, vd, dod = (t.to(dev()) for t in (q, k, v, do))
    tab = None
    if w.rope_theta:
        tab = torch.from_numpy(fa.fa_rope_inv_freq(d, w.rope_theta)).to(dev())
        qr, kr = poison(q.shape, q.dtype), poison(k.shape, k.dtype)
        fa.rope(qd, tab, out=qr)
        fa.rope(kd, tab, out=kr)
    else:
        qr, kr = qd, kd
    o = poison(q.shape, q.dtype)
    lse = poison((B, H, T), torch.float32)
    (fa.fa_fwd_f32 if f32 else fa.fa_fwd)(qr, kr, vd, o, lse, B, H, Hkv, T, d, w.scale,
                                          w.window, w.global_every, softcap)
    gq, gk, gv = poison(q.shape, q.dtype), poison(k.shape, k.dtype), poison(v.shape, v.dtype)
    (fa.fa_bwd_f32 if f32 else fa.fa_bwd)(qr, kr, vd, o, lse, dod, gq, gk, gv, B, H, Hkv, T, d,
                                          w.scale, w.window, w.global_every, softcap)
    out = dict(qr=qr, kr=kr, o=o, lse=lse, dq=gq, dk=gk, dv=gv)
    if tab is not None:
        dqi, dki = poison(q.shape, q.dtype), poison(k.shape, k.dtype)
        fa.rope(gq, tab, out=dqi, backward=True)
        fa.rope(gk, tab, out=dki, backward=True)
        out.update(dq_in=dqi, dk_in=dki, table=tab)
    torch.cuda.synchronize()
    return out


def _rows(T, W, rng, n=48):
    fixed = [0, 1, T - 1, T // 2]
    if 0 < W < T:
        fixed += [W - 1, W, min(T - 1, W + 1)]
    extra = rng.choice(T, size=min(n, T), replace=False).tolist()
    return np.array(sorted(set(x for x in fixed + extra if 0 <= x < T)))


def _oracle_group(w, qh, kg, vg, doh, softcap, qrows, kvrows):
    """qh, doh: [G, T, d] float64 of the group's query heads; kg, vg: [T, d]."""
    res = dict(o=[], lse=[], dq=[])
    dk = np.zeros((len(kvrows), w.d))
    dv = np.zeros((len(kvrows), w.d))
    for r in range(qh.shape[0]):
        gq_, gk_, gv_, o, lse = OA.head_grads_sampled(
            qh[r], kg, vg, doh[r], w.scale, w.window if w.window < w.T else 0, softcap,
            qrows, kvrows)
        res["o"].append(o)
        res["lse"].append(lse)
        res["dq"].append(gq_)
        dk += gk_
        dv += gv_
    return {n: np.stack(x) for n, x in res.items()} | dict(dk=dk, dv=dv)


def _compare_groups(w, got, q_in, k_in, v_in, do_in, softcap, e2e_table=None, tag=""):
    """q_in/k_in: CPU tensors the oracle attends over (GPU RoPE output for the
    stage-isolated check, original inputs when e2e_table is given)."""
    rng = np.random.default_rng(0)
    G = w.H // w.Hkv
    f32 = w.dtype == "f32"
    groups = [(0, 0), (w.B - 1, w.Hkv - 1)] if (w.B, w.Hkv) != (1, 1) else [(0, 0)]
    for b, g in sorted(set(groups)):
        hs = list(range(g * G, (g + 1) * G))
        if e2e_table is not None:   # small-T workloads: every row, so the
            qrows = kvrows = np.arange(w.T)  # oracle's rope_bwd applies as is
        else:
            qrows = _rows(w.T, w.window, rng)
            kvrows = _rows(w.T, w.window, rng)
        qh = synth.to_f64(q_in[b, hs])
        kg = synth.to_f64(k_in[b, g])
        if e2e_table is not None:
            qh = OR.rope(qh, e2e_table)
            kg = OR.rope(kg, e2e_table)
        ref = _oracle_group(w, qh, kg, synth.to_f64(v_in[b, g]), synth.to_f64(do_in[b, hs]),
                            softcap, qrows, kvrows)
        dq_ref, dk_ref = ref["dq"], ref["dk"]
        gdq = got["dq_in"] if e2e_table is not None else got["dq"]
        gdk = got["dk_in"] if e2e_table is not None else got["dk"]
        if e2e_table is not None:
            # gradient w.r.t. the un-rotated inputs: the oracle's RoPE backward
            dq_ref = OR.rope_bwd(dq_ref, e2e_table)
            dk_ref = OR.rope_bwd(dk_ref, e2e_table)
        gotg = dict(
            o=got["o"][b, hs].double().cpu().numpy(),
            lse=got["lse"][b, hs].double().cpu().numpy(),
            dq=gdq[b, hs][:, qrows].double().cpu().numpy(),
            dk=gdk[b, g][kvrows].double().cpu().numpy(),
            dv=got["dv"][b, g][kvrows].double().cpu().numpy())
        refg = dict(o=ref["o"], lse=ref["lse"], dq=dq_ref, dk=dk_ref, dv=ref["dv"])
        # end to end, the oracle attends over exactly rotated Q, K while the
        # GPU attends over their bf16 rounding: only the RMS bar applies
        errs = {n: check(f"{tag}{n}[b{b},g{g}]", gotg[n], refg[n], f32,
                         elem_guard=e2e_table is None) for n in refg}
        say(f"  {tag}b{b} g{g}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))


WL = ["forge-default", "qwen25", "mistral", "gemma-local", "gemma-global", "gemma3-local"]


@pytest.mark.parametrize("name,softcap", [(n, synth.WORKLOADS[n].softcap) for n in WL]
                         + [("gemma3-local", 0.0)])
def test_workload_sampled_parity(name, softcap):
    w = synth.WORKLOADS[name]
    say(f"[workload] {name} B{w.B} H{w.H}/{w.Hkv} T{w.T} d{w.d} W{w.window} cap{softcap}")
    q, k, v, do = synth.draw(w)
    got = _gpu_path(w, q, k, v, do, softcap)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert torch.isfinite(got[n]).all(), f"{n} has unwritten/non-finite entries"
    if w.rope_theta:
        _compare_groups(w, got, got["qr"].cpu(), got["kr"].cpu(), v, do, softcap,
                        tag="stage:")
        table = got["table"].cpu().numpy()
        _compare_groups(w, got, q, k, v, do, softcap, e2e_table=table, tag="e2e:")
    else:
        _compare_groups(w, got, q, k, v, do, softcap)


def test_long_sequence_sampled_parity():
    """T = 16384 (twice the longest workload), GQA 8:1, a window that is not
    a multiple of any tile: the 64-bit offsets, the tile bounds of long
    loops and the dK/dV head loop, against the oracle on sampled rows."""
    w = synth.Workload("long", "bf16", 1, 8, 1, 16384, 128, window=5000, seed=77)
    say(f"[long] B{w.B} H{w.H}/{w.Hkv} T{w.T} d{w.d} W{w.window}")
    q, k, v, do = synth.draw(w)
    got = _gpu_path(w, q, k, v, do, 0.0)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert torch.isfinite(got[n]).all(), f"{n} has unwritten/non-finite entries"
    _compare_groups(w, got, q, k, v, do, 0.0)


def test_forge_f32_every_element():
    w = synth.WORKLOADS["forge-f32"]
    say(f"[workload] forge-f32 B{w.B} H{w.H} T{w.T} d{w.d}")
    q, k, v, do = synth.draw(w)
    got = _gpu_path(w, q, k, v, do, 0.0)
    qf, kf, vf, dof = (synth.to_f64(t) for t in (q, k, v, do))
    o, lse = OA.attn_fwd(qf, kf, vf, w.scale, 0, 0.0)
    dq, dk, dv = OA.attn_bwd(qf, kf, vf, dof, w.scale, 0, 0.0)
    for n, ref in dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv).items():
        e = check(n, got[n].double().cpu().numpy(), ref, True)
        say(f"  {n} max-abs {e:.2e}")
