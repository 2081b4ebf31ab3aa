"""Full-size parity of every workload, in the launch configuration the
benchmark times, against the float64 oracle.

For each workload the whole GPU path runs once at full size (RoPE on Q and
K first where the workload has it, fa_fwd, fa_bwd, RoPE backward on dQ and
dK).  The oracle then evaluates every (batch, query head): o and lse on
every row, and for every (batch, KV head) group dq on sampled rows of each
of its query heads and the group's dk, dv on sampled key rows (their exact
definition needs the lse and D of every query row, which the oracle
computes); each output element against the bf16 envelope of
tests/envelope.py.  RoPE workloads are checked stage-isolated on every head
(the oracle attends over the GPU's bf16 RoPE output) and end to end on two
groups (the oracle applies its own RoPE to the original inputs; the
envelope then adds the effect of rounding the rotated Q, K to bf16, which
the oracle computes as the difference of its own results on the exact and
on the rounded rotation).  forge-f32 is small and is compared on every
element at 1e-4.  Heads are evaluated on a thread pool (numpy releases the
interpreter lock in its kernels), one BLAS thread each.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

from causal_attention_fa_amd import synth
from oracle import attention as OA
from oracle import rope as OR
from tests import envelope as EV
from tests.gpu_util import check, dev, poison, say

pytestmark = pytest.mark.gpu

WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


def _gpu_path(w, q, k, v, do, softcap):
    """The benchmarked step on device tensors; returns CPU tensors."""
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
    return {n: t.cpu() for n, t in out.items()}


def _rows(T, W, rng, n):
    fixed = [0, 1, T - 1, T // 2]
    if 0 < W < T:
        fixed += [W - 1, W, min(T - 1, W + 1)]
    extra = rng.choice(T, size=min(n, T), replace=False).tolist()
    return np.array(sorted(set(x for x in fixed + extra if 0 <= x < T)))


def _np(t):
    return t.double().numpy()


def _check_group(w, got, parts, b, g, qrows, kvrows, tag):
    G = w.H // w.Hkv
    hs = list(range(g * G, (g + 1) * G))
    kvc = EV.combine_kv(parts)
    ref = dict(o=np.stack([p["o"] for p in parts]), lse=np.stack([p["lse"] for p in parts]),
               dq=np.stack([p["dq"] for p in parts]), dk=kvc["dk"], dv=kvc["dv"])
    env = dict(o=np.stack([p["E_o"] for p in parts]), lse=np.stack([p["E_lse"] for p in parts]),
               dq=np.stack([p["E_dq"] for p in parts]), dk=kvc["E_dk"], dv=kvc["E_dv"])
    gotg = dict(o=_np(got["o"][b, hs]), lse=_np(got["lse"][b, hs]),
                dq=_np(got["dq"][b, hs][:, qrows]), dk=_np(got["dk"][b, g][kvrows]),
                dv=_np(got["dv"][b, g][kvrows]))
    return {n: check(f"{tag}{n}[b{b},g{g}]", gotg[n], ref[n], env=env[n], qty=n) for n in ref}


_CACHE = {}


def _run(name, softcap):
    key = (name, softcap)
    if key not in _CACHE:
        _CACHE.clear()
        w = synth.WORKLOADS[name]
        q, k, v, do = synth.draw(w)
        _CACHE[key] = (w, (q, k, v, do), _gpu_path(w, q, k, v, do, softcap))
    return _CACHE[key]


WL = ["forge-default", "qwen25", "mistral", "gemma-local", "gemma-global", "gemma3-local"]


@pytest.mark.parametrize("name,softcap", [(n, synth.WORKLOADS[n].softcap) for n in WL]
                         + [("gemma3-local", 0.0)])
def test_workload_every_head(name, softcap):
    """Every (b, h): o and lse on all rows; every (b, KV head) group: dq, dk,
    dv on sampled rows (stage-isolated for RoPE workloads)."""
    w, (q, k, v, do), got = _run(name, softcap)
    say(f"[workload] {name} B{w.B} H{w.H}/{w.Hkv} T{w.T} d{w.d} W{w.window} cap{softcap}")
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert torch.isfinite(got[n]).all(), f"{n} has unwritten/non-finite entries"
    G = w.H // w.Hkv
    q_in = got["qr"] if w.rope_theta else q
    k_in = got["kr"] if w.rope_theta else k
    rng = np.random.default_rng(0)
    groups = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    # fewer sampled rows per group where there are many groups
    nrows = 6 if len(groups) >= 32 else 12
    samples = {bg: (_rows(w.T, w.window, rng, nrows), _rows(w.T, w.window, rng, nrows))
               for bg in groups}

    def job(bgr):
        b, g, r = bgr
        h = g * G + r
        qrows, kvrows = samples[(b, g)]
        W = w.window if w.window < w.T else 0
        return bgr, EV.head_envelopes(synth.to_f64(q_in[b, h]), synth.to_f64(k_in[b, g]),
                                      synth.to_f64(v[b, g]), synth.to_f64(do[b, h]), w.scale, W,
                                      softcap, q_rows=qrows, kv_rows=kvrows)

    worst = {}
    parts = {}
    with threadpool_limits(1), ThreadPoolExecutor(WORKERS) as ex:
        for (b, g, r), p in ex.map(job, [(b, g, r) for b, g in groups for r in range(G)]):
            parts.setdefault((b, g), {})[r] = p
            if len(parts[(b, g)]) < G:
                continue
            qrows, kvrows = samples[(b, g)]
            errs = _check_group(w, got, [parts[(b, g)][i] for i in range(G)], b, g, qrows,
                                kvrows, "stage:" if w.rope_theta else "")
            del parts[(b, g)]
            for n, e in errs.items():
                worst[n] = max(worst.get(n, 0.0), e)
    say(f"  {len(groups)} groups x {G} heads; worst rms-relative: "
        + " ".join(f"{n}={e:.2e}" for n, e in worst.items()))


@pytest.mark.parametrize("name", ["forge-default", "qwen25"])
def test_workload_rope_end_to_end(name):
    """RoPE workloads end to end on two groups: the oracle rotates the
    original Q, K itself; gradients w.r.t. the un-rotated inputs."""
    w, (q, k, v, do), got = _run(name, synth.WORKLOADS[name].softcap)
    table = got["table"].numpy()
    G = w.H // w.Hkv
    W = w.window if w.window < w.T else 0
    say(f"[e2e] {name}")
    for b, g in [(0, 0), (w.B - 1, w.Hkv - 1)]:
        hs = list(range(g * G, (g + 1) * G))
        allr = np.arange(w.T)
        qe = OR.rope(synth.to_f64(q[b, hs]), table)           # exact rotation
        ke = OR.rope(synth.to_f64(k[b, g]), table)
        rnd = lambda x: torch.from_numpy(x).to(torch.bfloat16).double().numpy()
        qb, kb = rnd(qe), rnd(ke)                               # rounded to bf16
        vf, dof = synth.to_f64(v[b, g]), synth.to_f64(do[b, hs])

        def run(qx, kx):
            return [EV.head_envelopes(qx[r], kx, vf, dof[r], w.scale, W, w.softcap, q_rows=allr,
                                      kv_rows=allr) for r in range(G)]

        with threadpool_limits(1), ThreadPoolExecutor(2) as ex:
            pe, pb = list(ex.map(lambda a: run(*a), [(qe, ke), (qb, kb)]))
        ce, cb = EV.combine_kv(pe), EV.combine_kv(pb)
        ref = dict(o=np.stack([p["o"] for p in pe]), lse=np.stack([p["lse"] for p in pe]),
                   dq=OR.rope_bwd(np.stack([p["dq"] for p in pe]), table),
                   dk=OR.rope_bwd(ce["dk"], table), dv=ce["dv"])
        rb = dict(o=np.stack([p["o"] for p in pb]), lse=np.stack([p["lse"] for p in pb]),
                  dq=OR.rope_bwd(np.stack([p["dq"] for p in pb]), table),
                  dk=OR.rope_bwd(cb["dk"], table), dv=cb["dv"])
        env = dict(o=np.stack([p["E_o"] for p in pb]), lse=np.stack([p["E_lse"] for p in pb]),
                   dq=EV.rotate_env(np.stack([p["E_dq"] for p in pb])),
                   dk=EV.rotate_env(cb["E_dk"]), dv=cb["E_dv"])
        gotg = dict(o=_np(got["o"][b, hs]), lse=_np(got["lse"][b, hs]),
                    dq=_np(got["dq_in"][b, hs]), dk=_np(got["dk_in"][b, g]),
                    dv=_np(got["dv"][b, g]))
        errs = {}
        for n in ref:
            # envelope on the rounded rotation + what the rounding itself moves
            e = env[n] + np.abs(ref[n] - rb[n])
            errs[n] = check(f"e2e:{n}[b{b},g{g}]", gotg[n], ref[n], env=e, qty=n)
        say(f"  b{b} g{g}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))


def test_long_sequence_parity():
    """T = 16384 (twice the longest workload), GQA 8:1, a window that is not
    a multiple of any tile: the 64-bit offsets, the tile bounds of long
    loops and the dK/dV head loop, against the oracle (every head's o and
    lse on all rows, gradients on sampled rows)."""
    w = synth.Workload("long", "bf16", 1, 8, 1, 16384, 128, window=5000, seed=77)
    say(f"[long] B{w.B} H{w.H}/{w.Hkv} T{w.T} d{w.d} W{w.window}")
    q, k, v, do = synth.draw(w)
    got = _gpu_path(w, q, k, v, do, 0.0)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert torch.isfinite(got[n]).all(), f"{n} has unwritten/non-finite entries"
    rng = np.random.default_rng(1)
    qrows, kvrows = _rows(w.T, w.window, rng, 8), _rows(w.T, w.window, rng, 8)
    kg, vg = synth.to_f64(k[0, 0]), synth.to_f64(v[0, 0])

    def job(h):
        return EV.head_envelopes(synth.to_f64(q[0, h]), kg, vg, synth.to_f64(do[0, h]), w.scale,
                                 w.window, 0.0, q_rows=qrows, kv_rows=kvrows)

    with threadpool_limits(1), ThreadPoolExecutor(WORKERS) as ex:
        parts = list(ex.map(job, range(w.H)))
    errs = _check_group(w, got, parts, 0, 0, qrows, kvrows, "")
    say("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))


def test_forge_f32_every_element():
    w = synth.WORKLOADS["forge-f32"]
    say(f"[workload] forge-f32 B{w.B} H{w.H} T{w.T} d{w.d}")
    q, k, v, do = synth.draw(w)
    got = _gpu_path(w, q, k, v, do, 0.0)
    qf, kf, vf, dof = (synth.to_f64(t) for t in (q, k, v, do))
    o, lse = OA.attn_fwd(qf, kf, vf, w.scale, 0, 0.0)
    dq, dk, dv = OA.attn_bwd(qf, kf, vf, dof, w.scale, 0, 0.0)
    for n, ref in dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv).items():
        e = check(n, got[n].double().numpy(), ref, True)
        say(f"  {n} max-abs {e:.2e}")
