#!/usr/bin/env python3
"""Benchmark of the fused causal attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole path over one batch of synthetic input
already resident in HBM: RoPE (workloads that have it), the attention
forward and backward, RoPE backward.  With --rope fused (default) K is
rotated by rope_apply, q is rotated inside fa_fwd_rope and dq rotated back
inside fa_bwd_rope, dK by rope_apply_bwd; --rope separate runs rope_apply on
Q and K around fa_fwd / fa_bwd.  The default workload is "mistral"
(B4 H32/8 T8192 d128, window 4096): the largest T = 8192 workload, the
sequence length the throughput bars are set at.  Prints ONE JSON line:
effective fwd+bwd TFLOPS (only mask-visible (q, k) pairs count; bwd = 2.5x
fwd) and its fraction of the bf16 dense MFMA peak, per-kernel times from
HIP events recorded by the library between its launches (fa_set_stage_events),
a roofline entry for the dominant kernel, and the float64 CPU oracle timed
on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
METRIC = "attention fwd+bwd TFLOPS (effective FLOPs) & % bf16 MFMA peak, 1×MI355X"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_sources_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "causal_attention_fa_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def cpu_baseline(w, budget_s, seed=0):
    """Time the float64 oracle's fwd+bwd definition on (b, h) heads of the
    workload at full T, one after another until budget_s seconds have passed
    (at least one head); scale to the same effective-FLOP unit."""
    import numpy as np
    from causal_attention_fa_amd import synth
    from oracle import attention as OA
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover
        threads = 1
    q, k, v, do = synth.draw(w, seed=seed)
    G = w.H // w.Hkv
    W = w.window if w.window < w.T else 0
    t0 = time.perf_counter()
    n_heads = 0
    while n_heads < w.B * w.H and (n_heads == 0 or time.perf_counter() - t0 < budget_s):
        b, h = divmod(n_heads, w.H)
        OA.head_backward(synth.to_f64(q[b, h]), synth.to_f64(k[b, h // G]),
                         synth.to_f64(v[b, h // G]), synth.to_f64(do[b, h]), w.scale, W,
                         w.softcap)
        n_heads += 1
    dt = time.perf_counter() - t0
    flops = (w.fwd_flops() + w.bwd_flops()) / (w.B * w.H) * n_heads
    return {"value": flops / dt / 1e12, "unit": "TFLOPS", "cores": int(threads),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{n_heads} of {w.B * w.H} (b,h) heads at full T={w.T}, fwd+bwd "
                      f"(oracle.attention.head_backward, float64, full score matrix); "
                      f"host affinity {len(os.sched_getaffinity(0))} cpus"}


class SclkSampler:
    """Shader clock observed while the timed steps run: a background thread
    reads the driver's current-level line of pp_dpm_sclk (the one marked '*')
    every few milliseconds.  Best effort: null when the file is not exposed."""

    def __init__(self, period_s=0.004):
        import glob
        paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = paths[0] if paths else None
        self.period = period_s
        self.samples = []
        self._stop = False
        self._thread = None

    def _read(self):
        try:
            with open(self.path) as fh:
                for line in fh:
                    if line.rstrip().endswith("*"):
                        return int(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _run(self):
        while not self._stop:
            v = self._read()
            if v is not None:
                self.samples.append(v)
            time.sleep(self.period)

    def start(self):
        if self.path:
            import threading
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def stop(self):
        self._stop = True
        if self._thread:
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        v = sorted(self.samples)
        return {"median": v[len(v) // 2], "min": v[0], "max": v[-1], "samples": len(v),
                "source": self.path}


def kernel_flops_per_pair(kind, d, dv=None):
    """Algorithmic MFMA flops per visible (q, k) pair of one kernel launch
    (d: query/key head size, dv: value head size)."""
    dv = d if dv is None else dv
    return {"fwd": 2 * d + 2 * dv,              # S = QK^T, O += PV
            "bwd_dq": 4 * d + 2 * dv,           # S, dP = dO V^T, dQ += dS K
            "bwd_dkdv": 4 * d + 4 * dv,         # S, dP, dV += P^T dO, dK += dS^T Q
            "bwd_dv": 2 * d + 2 * dv,           # S, dV
            "bwd_dk": 4 * d + 2 * dv}[kind]     # S, dP, dK


def traffic_for(workload, kernel, src_hash):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    try:
        with open(p) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sources_sha") != src_hash:
        return None
    return t.get("kernels", {}).get(kernel, {}).get("hbm_bytes_per_launch")


def decode_leg(name, iters, dev):
    """fa_decode on a decode workload: per-call time from HIP events on the
    launch stream (split and combine kernels separately) and the HBM rate of
    its algorithmic bytes (visible K and V rows once, q, o, lse, lens)."""
    import torch
    from causal_attention_fa_amd import fa, synth
    w = synth.DECODE_WORKLOADS[name]
    q, kc, vc, lens = synth.draw_decode(w, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    for _ in range(3):
        fa.fa_decode(q, kc, vc, lens, o, lse, None, w.B, w.H, w.Hkv, w.S, w.d, w.scale,
                     w.window, w.softcap, sh)
    torch.cuda.synchronize()
    evs = []
    for _ in range(iters):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        for x in e:          # creates the underlying HIP event
            x.record(stream)
        fa.fa_set_stage_events([x.cuda_event for x in e])
        fa.fa_decode(q, kc, vc, lens, o, lse, None, w.B, w.H, w.Hkv, w.S, w.d, w.scale,
                     w.window, w.softcap, sh)
        evs.append(e)
    fa.fa_set_stage_events([])
    torch.cuda.synchronize()
    split = sum(e[0].elapsed_time(e[1]) for e in evs) / iters
    comb = sum(e[1].elapsed_time(e[2]) for e in evs) / iters
    L = lens.cpu().long()
    vis = L.clamp(max=w.window) if w.window > 0 else L
    kv_bytes = int(vis.sum()) * w.Hkv * w.d * 2 * 2
    io_bytes = q.numel() * 2 * 2 + lse.numel() * 4 + lens.numel() * 4
    ms = split + comb
    gbs = (kv_bytes + io_bytes) / (ms * 1e-3) / 1e9
    ns, ch = fa.fa_decode_splits(w.B, w.Hkv, w.S, w.window)
    return {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.Hkv, "S": w.S, "d": w.d,
            "window": w.window, "softcap": w.softcap, "chunks": [ns, ch],
            "ms": round(ms, 4), "split_ms": round(split, 4), "combine_ms": round(comb, 4),
            "algorithmic_bytes": kv_bytes + io_bytes, "gbs": round(gbs, 1),
            "split_gbs": round(kv_bytes / (split * 1e-3) / 1e9, 1),
            "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "iters": iters}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mistral")
    ap.add_argument("--calibrate-copy-mb", type=float, default=0.0,
                    help="only run a plain device copy of this many MiB (5 times) and "
                         "exit: the reference kernel for scaling HBM byte counters")
    ap.add_argument("--rope", choices=["fused", "separate"], default="fused",
                    help="RoPE workloads: fused into the attention (fa_fwd_rope / "
                         "fa_bwd_rope; K rotated by rope_apply) or rope_apply on Q and K "
                         "around fa_fwd / fa_bwd")
    ap.add_argument("--decode-workload", default="qwen25-decode",
                    help="decode workload timed after the main step ('none' to skip)")
    ap.add_argument("--decode-iters", type=int, default=20)
    ap.add_argument("--decode-only", action="store_true",
                    help="time only fa_decode on --decode-workload (one JSON line in GB/s)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU-baseline budget: oracle heads are timed until this many "
                         "seconds have passed (0: skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not "
              "supported (the path shards by (batch, KV-head) groups with no exchange; "
              "see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    from causal_attention_fa_amd import fa, synth

    if args.calibrate_copy_mb > 0:
        n = int(args.calibrate_copy_mb * (1 << 20)) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n * 4, "launches": 5}))
        return

    if args.decode_only:
        r = decode_leg(args.decode_workload, args.decode_iters, torch.device("cuda:0"))
        print(json.dumps({"metric": "decode attention HBM throughput (algorithmic bytes), 1xMI355X",
                          "value": r["gbs"], "unit": "GB/s", "n_gpus": 1,
                          "steps": args.decode_iters, "warmup": 3, "ms_per_step": r["ms"],
                          "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                          "dtype": "bf16", "data": "synthetic",
                          "config": {"workload": r["workload"]},
                          "roofline": {"bound": "hbm", "achieved": r["gbs"],
                                       "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                       "frac": r["frac_hbm"], "traffic": None},
                          "decode": r}), flush=True)
        return

    w = synth.WORKLOADS[args.workload]
    if w.dtype != "bf16":
        raise SystemExit("bench.py times the bf16 path; pick a bf16 workload")
    dev = torch.device("cuda:0")
    B, H, Hkv, T, d = w.B, w.H, w.Hkv, w.T, w.d
    log(f"[bench] workload {w.name}: B{B} H{H}/{Hkv} T{T} d{d} W{w.window} cap{w.softcap}")
    q, k, v, do = (t.to(dev) for t in synth.draw(w))
    o = torch.empty_like(do)
    dvh = w.dv
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    rope = bool(w.rope_theta)
    fused = rope and args.rope == "fused" and dvh == d
    if rope:
        tab = torch.from_numpy(fa.fa_rope_inv_freq(d, w.rope_theta)).to(dev)
        qr, kr = torch.empty_like(q), torch.empty_like(k)
        dqi, dki = torch.empty_like(q), torch.empty_like(k)
    else:
        qr, kr = q, k
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def new_event():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    bwd_names = ["bwd_" + n for n in fa.fa_bwd_kernels(d, dvh)]   # the launches of fa_bwd
    n_bwd = len(bwd_names)

    def step_fused(ev=None):
        # K rotated once; q rotated at the attention's load (rotated q kept
        # for the backward); dq comes back un-rotated; dk rotated back.
        if ev: fa.fa_set_stage_events([ev["rk"][0].cuda_event, ev["rk"][1].cuda_event])
        fa.rope_apply(k, kr, tab, B, Hkv, T, d, sh)
        if ev: fa.fa_set_stage_events([e.cuda_event for e in ev["fwd"]])
        fa.fa_fwd_rope(q, kr, v, o, lse, tab, qr, B, H, Hkv, T, d, w.scale, w.window,
                       w.global_every, w.softcap, sh)
        if ev: fa.fa_set_stage_events([e.cuda_event for e in ev["bwd"]])
        fa.fa_bwd_rope(qr, kr, v, o, lse, do, tab, dqi, dk, dv, B, H, Hkv, T, d, w.scale,
                       w.window, w.global_every, w.softcap, sh)
        if ev: fa.fa_set_stage_events([])
        fa.rope_apply_bwd(dk, dki, tab, B, Hkv, T, d, sh)

    def step(ev=None):
        if fused:
            return step_fused(ev)
        if rope:
            if ev: fa.fa_set_stage_events([ev["rq"][0].cuda_event, ev["rq"][1].cuda_event])
            fa.rope_apply(q, qr, tab, B, H, T, d, sh)
            if ev: fa.fa_set_stage_events([ev["rk"][0].cuda_event, ev["rk"][1].cuda_event])
            fa.rope_apply(k, kr, tab, B, Hkv, T, d, sh)
        if ev: fa.fa_set_stage_events([e.cuda_event for e in ev["fwd"]])
        if dvh == d:
            fa.fa_fwd(qr, kr, v, o, lse, B, H, Hkv, T, d, w.scale, w.window, w.global_every,
                      w.softcap, sh)
        else:
            fa.fa_fwd_vdim(qr, kr, v, o, lse, B, H, Hkv, T, d, dvh, w.scale, w.window,
                           w.global_every, w.softcap, sh)
        if ev: fa.fa_set_stage_events([e.cuda_event for e in ev["bwd"]])
        if dvh == d:
            fa.fa_bwd(qr, kr, v, o, lse, do, dq, dk, dv, B, H, Hkv, T, d, w.scale, w.window,
                      w.global_every, w.softcap, sh)
        else:
            fa.fa_bwd_vdim(qr, kr, v, o, lse, do, dq, dk, dv, B, H, Hkv, T, d, dvh, w.scale,
                           w.window, w.global_every, w.softcap, sh)
        if ev: fa.fa_set_stage_events([])
        if rope:
            fa.rope_apply_bwd(dq, dqi, tab, B, H, T, d, sh)
            fa.rope_apply_bwd(dk, dki, tab, B, Hkv, T, d, sh)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [dict(fwd=[new_event(), new_event()], bwd=[new_event() for _ in range(n_bwd + 1)],
                rq=[new_event(), new_event()], rk=[new_event(), new_event()])
           for _ in range(args.steps)]
    # step boundaries: one event between consecutive steps
    bounds = [new_event() for _ in range(args.steps + 1)]
    t_start, t_end = new_event(), new_event()
    torch.cuda.synchronize()
    sclk = SclkSampler()
    sclk.start()
    wall0 = time.perf_counter()
    t_start.record(stream)
    bounds[0].record(stream)
    for i in range(args.steps):
        step(evs[i])
        bounds[i + 1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    sclk.stop()
    ms = t_start.elapsed_time(t_end) / args.steps
    step_ms = sorted(bounds[i].elapsed_time(bounds[i + 1]) for i in range(args.steps))

    def avg(pairs):
        return sum(a.elapsed_time(b) for a, b in pairs) / len(pairs)

    kern = {"fwd": avg([(e["fwd"][0], e["fwd"][1]) for e in evs])}
    for j, nm in enumerate(bwd_names):
        kern[nm] = avg([(e["bwd"][j], e["bwd"][j + 1]) for e in evs])
    if rope:
        if not fused:
            kern["rope_q"] = avg([(e["rq"][0], e["rq"][1]) for e in evs])
        kern["rope_k"] = avg([(e["rk"][0], e["rk"][1]) for e in evs])

    pairs_total = w.visible_pairs() * B * H
    fwd_f, bwd_f = w.fwd_flops(), w.bwd_flops()
    value = (fwd_f + bwd_f) / (ms * 1e-3) / 1e12
    fwd_tf = fwd_f / (kern["fwd"] * 1e-3) / 1e12
    bwd_ms = sum(kern[n] for n in bwd_names)
    bwd_tf = bwd_f / (bwd_ms * 1e-3) / 1e12
    attn_ms = kern["fwd"] + bwd_ms

    # dominant kernel by time, priced at its own algorithmic flops
    dom = max(["fwd"] + bwd_names, key=lambda n: kern[n])
    dom_flops = kernel_flops_per_pair(dom, d, dvh) * pairs_total
    achieved = dom_flops / (kern[dom] * 1e-3) / 1e12
    src_hash = kernel_sources_hash()
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_for(w.name, dom, src_hash),
                "algorithmic_flops_per_launch": dom_flops,
                "avg_launch_ms": round(kern[dom], 4)}

    sc = sclk.summary()
    if sc:
        # the same fraction against the peak at the observed median shader
        # clock (the published peak assumes 2400 MHz)
        roofline["frac_at_observed_sclk"] = round(achieved / (PEAK_BF16_TFLOPS * sc["median"] / 2400.0), 4)
    extra = {"fwd_tflops": round(fwd_tf, 1), "fwd_pct_peak": round(100 * fwd_tf / PEAK_BF16_TFLOPS, 2),
             "bwd_tflops": round(bwd_tf, 1),
             "attn_fwd_bwd_tflops": round((fwd_f + bwd_f) / (attn_ms * 1e-3) / 1e12, 1),
             "pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
             "kernel_ms": {n: round(t, 4) for n, t in kern.items()},
             "step_ms_median": round(step_ms[len(step_ms) // 2], 4),
             "step_ms_min": round(step_ms[0], 4),
             "sclk_mhz": sc,
             "wall_s": round(wall, 3), "kernel_sources_sha": src_hash}
    if rope:
        extra["rope_mode"] = "fused" if fused else "separate"
        nbytes_k = 2 * k.numel() * 2 + d // 2 * 4
        extra["rope_k_gbs"] = round(nbytes_k / (kern["rope_k"] * 1e-3) / 1e9, 1)
        if not fused:
            nbytes_q = 2 * q.numel() * 2 + d // 2 * 4
            extra["rope_q_gbs"] = round(nbytes_q / (kern["rope_q"] * 1e-3) / 1e9, 1)

    if args.decode_workload != "none":
        del q, k, v, do, o, lse, dq, dk, dv
        if rope:
            del qr, kr, dqi, dki
        torch.cuda.empty_cache()
        log(f"[bench] decode leg: {args.decode_workload}")
        extra["decode"] = decode_leg(args.decode_workload, args.decode_iters, dev)

    cpu = None
    if args.cpu_seconds > 0:
        log(f"[bench] timing the oracle for ~{args.cpu_seconds:g} s (CPU)")
        cpu = cpu_baseline(w, args.cpu_seconds)

    out = {"metric": METRIC, "value": round(value, 2), "unit": "TFLOPS", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": w.name, "B": B, "H": H, "Hkv": Hkv, "T": T, "d": d, "d_v": dvh,
                      "window": w.window, "softcap": w.softcap,
                      "global_every": w.global_every, "rope_theta": w.rope_theta,
                      "visible_pairs_per_head": w.visible_pairs(),
                      "effective_gflop_per_step": round((fwd_f + bwd_f) / 1e9, 1)},
           "roofline": roofline, "cpu_baseline": cpu}
    out.update(extra)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
