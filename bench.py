#!/usr/bin/env python3
"""Benchmark of the fused causal attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole path over one batch of synthetic input
already resident in HBM: RoPE (workloads that have it), the attention
forward and backward, RoPE backward.  With --rope fused (default) K is
rotated by rope_apply, q is rotated inside fa_fwd_rope and dq rotated back
inside fa_bwd_rope, dK by rope_apply_bwd; --rope separate runs rope_apply on
Q and K around fa_fwd / fa_bwd.  The headline workload is "mistral"
(B4 H32/8 T8192 d128, window 4096): the largest T = 8192 workload, the
sequence length the throughput bars are set at.

Prints ONE JSON line: effective fwd+bwd TFLOPS of the headline workload
(only mask-visible (q, k) pairs count; bwd = 2.5x fwd) and its fraction of
the bf16 dense MFMA peak (2516.6 TFLOPS: 256 CUs x 2.4 GHz x 4096
flop/clk), per-kernel times from HIP events recorded by the library
between its own launches (fa_set_stage_events), a roofline entry for the
dominant kernel, the float64 CPU oracle timed on the host cores, and under
"configs" the same figures for every other model shape the pages name
(Forge default, Qwen 2.5, the Gemma 2 local and global layers and their
1:1 step, the Gemma 3 5:1 step), the standalone RoPE kernels in GB/s, and
the decode kernel in GB/s.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CUs x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
METRIC = "attention fwd+bwd TFLOPS (effective FLOPs) & % bf16 MFMA peak, 1×MI355X"

# model steps made of several layers: (name, base workload, window, global_every, layers)
LAYER_STEPS = {
    "gemma2-step": ("gemma-global", 4096, 2, 2),   # Gemma 2: local and global 1:1
    "gemma3-step": ("gemma-global", 1024, 6, 6),   # Gemma 3: 5 local (W1024) : 1 global
}
DEFAULT_CONFIGS = "forge-default,qwen25,gemma-local,gemma-global,gemma2-step,gemma3-step"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_sources_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "causal_attention_fa_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ CPU baseline

def _oracle_head(args):
    """Worker: one (b, h) head of the oracle at full T, one BLAS thread;
    returns (seconds of the forward, seconds of forward + backward)."""
    q, k, v, do, scale, W, cap = args
    from threadpoolctl import threadpool_limits
    from oracle import attention as OA
    with threadpool_limits(1):
        OA.head_forward(q[:256], k[:256], v[:256], scale, W, cap)   # warm-up (BLAS, allocator)
        t0 = time.perf_counter()
        OA.head_forward(q, k, v, scale, W, cap)
        t1 = time.perf_counter()
        OA.head_backward(q, k, v, do, scale, W, cap)
        t2 = time.perf_counter()
    return t1 - t0, t2 - t1


def _mem_available():
    try:
        with open("/proc/meminfo") as fh:
            for line in fh:
                if line.startswith("MemAvailable:"):
                    return int(line.split()[1]) * 1024
    except OSError:
        pass
    return 16 << 30


def cpu_baseline(w, max_workers=16, seed=0):
    """The float64 oracle (head_forward, head_backward: full score matrix) on
    (b, h) heads of the workload at full T, one head per worker process with
    one BLAS thread each, all workers at once; rates in the same effective-
    FLOP unit as the GPU figures.  Runs before the GPU is touched (the pool
    forks)."""
    import multiprocessing as mp
    from causal_attention_fa_amd import synth
    cores = len(os.sched_getaffinity(0))
    per_worker = 6 * w.T * w.T * 8          # a few T x T float64 matrices per head
    workers = max(1, min(cores, max_workers, w.B * w.H,
                         int(0.5 * _mem_available()) // per_worker))
    q, k, v, do = synth.draw(w, seed=seed)
    G = w.H // w.Hkv
    W = w.window if w.window < w.T else 0
    jobs = []
    for n in range(workers):
        b, h = divmod(n, w.H)
        jobs.append((synth.to_f64(q[b, h]), synth.to_f64(k[b, h // G]),
                     synth.to_f64(v[b, h // G]), synth.to_f64(do[b, h]), w.scale, W, w.softcap))
    del q, k, v, do
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(workers) as pool:
        res = pool.map(_oracle_head, jobs, chunksize=1)
    wall = time.perf_counter() - t0
    fwd_s = max(r[0] for r in res)
    fb_s = max(r[1] for r in res)
    per_head_f = w.fwd_flops() / (w.B * w.H)
    per_head_fb = (w.fwd_flops() + w.bwd_flops()) / (w.B * w.H)
    return {"value": round(workers * per_head_fb / fb_s / 1e12, 5), "unit": "TFLOPS",
            "cores": workers, "kind": "oracle",
            "fwd_tflops": round(workers * per_head_f / fwd_s / 1e12, 5),
            "seconds_fwd_per_head": round(fwd_s, 3), "seconds_fwd_bwd_per_head": round(fb_s, 3),
            "seconds_wall": round(wall, 3),
            "sample": f"{workers} of {w.B * w.H} (b,h) heads of {w.name} at full T={w.T}, one "
                      f"head per process (1 BLAS thread each, all at once): "
                      f"oracle.attention.head_forward, then head_backward (fwd+bwd), float64 "
                      f"full score matrix; host affinity {cores} cpus"}


# ------------------------------------------------------------------ GPU timing

def kernel_flops_per_pair(kind, d, dv=None):
    """Algorithmic MFMA flops per visible (q, k) pair of one kernel launch
    (d: query/key head size, dv: value head size)."""
    dv = d if dv is None else dv
    return {"fwd": 2 * d + 2 * dv,              # S = QK^T, O += PV
            "bwd_dq": 4 * d + 2 * dv,           # S, dP = dO V^T, dQ += dS K
            "bwd_dkdv": 4 * d + 4 * dv,         # S, dP, dV += P^T dO, dK += dS^T Q
            "bwd_dkdvq": 6 * d + 4 * dv,        # S, dP, dV, dK and dQ += dS K (atomics)
            "bwd_dqconv": 0}[kind]


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


class Layer:
    """Device tensors and the fwd + bwd calls of one attention layer."""

    def __init__(self, w, window, tensors, dev, rope_mode):
        import torch
        from causal_attention_fa_amd import fa
        self.fa = fa
        self.w, self.window = w, window
        q, k, v, do = (t.to(dev) for t in tensors)
        self.q, self.k, self.v, self.do = q, k, v, do
        self.o = torch.empty_like(do)
        self.lse = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device=dev)
        self.dq, self.dk, self.dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        self.rope = bool(w.rope_theta)
        self.fused = self.rope and rope_mode == "fused" and w.dv == w.d
        if self.rope:
            self.tab = torch.from_numpy(fa.fa_rope_inv_freq(w.d, w.rope_theta)).to(dev)
            self.qr, self.kr = torch.empty_like(q), torch.empty_like(k)
            self.dqi, self.dki = torch.empty_like(q), torch.empty_like(k)
        else:
            self.qr, self.kr = q, k
        self.bwd_names = ["bwd_" + n for n in fa.fa_bwd_kernels(w.d, w.dv)]

    def flops(self):
        w = self.w.replace(window=self.window)
        return w.fwd_flops(), w.bwd_flops(), w.visible_pairs() * w.B * w.H

    def run(self, sh, ev=None):
        """One fwd + bwd.  ev: dict of event lists (fwd, bwd, rq, rk) armed
        as the library's stage events around the matching calls."""
        fa, w, W = self.fa, self.w, self.window
        B, H, Hkv, T, d, dv = w.B, w.H, w.Hkv, w.T, w.d, w.dv
        arm = (lambda key: fa.fa_set_stage_events([e.cuda_event for e in ev[key]])) if ev else \
            (lambda key: None)
        if self.fused:
            # K rotated once; q rotated at the attention's load (rotated q
            # kept for the backward); dq comes back un-rotated; dk rotated back
            arm("rk")
            fa.rope_apply(self.k, self.kr, self.tab, B, Hkv, T, d, sh)
            arm("fwd")
            fa.fa_fwd_rope(self.q, self.kr, self.v, self.o, self.lse, self.tab, self.qr, B, H,
                           Hkv, T, d, w.scale, W, w.global_every, w.softcap, sh)
            arm("bwd")
            fa.fa_bwd_rope(self.qr, self.kr, self.v, self.o, self.lse, self.do, self.tab,
                           self.dqi, self.dk, self.dv, B, H, Hkv, T, d, w.scale, W,
                           w.global_every, w.softcap, sh)
            if ev:
                fa.fa_set_stage_events([])
            fa.rope_apply_bwd(self.dk, self.dki, self.tab, B, Hkv, T, d, sh)
            return
        if self.rope:
            arm("rq")
            fa.rope_apply(self.q, self.qr, self.tab, B, H, T, d, sh)
            arm("rk")
            fa.rope_apply(self.k, self.kr, self.tab, B, Hkv, T, d, sh)
        arm("fwd")
        if dv == d:
            fa.fa_fwd(self.qr, self.kr, self.v, self.o, self.lse, B, H, Hkv, T, d, w.scale, W,
                      w.global_every, w.softcap, sh)
        else:
            fa.fa_fwd_vdim(self.qr, self.kr, self.v, self.o, self.lse, B, H, Hkv, T, d, dv,
                           w.scale, W, w.global_every, w.softcap, sh)
        arm("bwd")
        if dv == d:
            fa.fa_bwd(self.qr, self.kr, self.v, self.o, self.lse, self.do, self.dq, self.dk,
                      self.dv, B, H, Hkv, T, d, w.scale, W, w.global_every, w.softcap, sh)
        else:
            fa.fa_bwd_vdim(self.qr, self.kr, self.v, self.o, self.lse, self.do, self.dq,
                           self.dk, self.dv, B, H, Hkv, T, d, dv, w.scale, W, w.global_every,
                           w.softcap, sh)
        if ev:
            fa.fa_set_stage_events([])
        if self.rope:
            fa.rope_apply_bwd(self.dq, self.dqi, self.tab, B, H, T, d, sh)
            fa.rope_apply_bwd(self.dk, self.dki, self.tab, B, Hkv, T, d, sh)


def time_layers(layers, steps, warmup):
    """Warm up, then time `steps` steps (every layer's fwd + bwd once) with
    HIP events on the launch stream: the whole timed region, each step, and
    each kernel of each layer through the library's stage events."""
    import torch
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def new_event():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)          # creates the underlying HIP event
        return e

    for _ in range(warmup):
        for L in layers:
            L.run(sh)
    torch.cuda.synchronize()
    evs = [[dict(fwd=[new_event(), new_event()],
                 bwd=[new_event() for _ in range(len(L.bwd_names) + 1)],
                 rq=[new_event(), new_event()], rk=[new_event(), new_event()])
            for L in layers] for _ in range(steps)]
    bounds = [new_event() for _ in range(steps + 1)]
    torch.cuda.synchronize()
    bounds[0].record(stream)
    for i in range(steps):
        for L, ev in zip(layers, evs[i]):
            L.run(sh, ev)
        bounds[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = bounds[0].elapsed_time(bounds[-1]) / steps
    step_ms = sorted(bounds[i].elapsed_time(bounds[i + 1]) for i in range(steps))

    def avg(getter):
        return sum(a.elapsed_time(b) for a, b in (getter(e) for e in evs)) / steps

    kern = {}   # kernel name -> ms per step (summed over layers)
    for li, L in enumerate(layers):
        names = [("fwd", lambda e, li=li: (e[li]["fwd"][0], e[li]["fwd"][1]))]
        for j, nm in enumerate(L.bwd_names):
            names.append((nm, lambda e, li=li, j=j: (e[li]["bwd"][j], e[li]["bwd"][j + 1])))
        if L.rope:
            if not L.fused:
                names.append(("rope_q", lambda e, li=li: (e[li]["rq"][0], e[li]["rq"][1])))
            names.append(("rope_k", lambda e, li=li: (e[li]["rk"][0], e[li]["rk"][1])))
        for nm, get in names:
            kern[nm] = kern.get(nm, 0.0) + avg(get)
    return ms, step_ms, kern


def summarize(layers, ms, step_ms, kern):
    fwd_f = sum(L.flops()[0] for L in layers)
    bwd_f = sum(L.flops()[1] for L in layers)
    bwd_names = layers[0].bwd_names
    bwd_ms = sum(kern[n] for n in bwd_names)
    value = (fwd_f + bwd_f) / (ms * 1e-3) / 1e12
    fwd_tf = fwd_f / (kern["fwd"] * 1e-3) / 1e12
    return {"fwd_bwd_tflops": round(value, 2),
            "pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
            "fwd_tflops": round(fwd_tf, 1),
            "fwd_pct_peak": round(100 * fwd_tf / PEAK_BF16_TFLOPS, 2),
            "bwd_tflops": round(bwd_f / (bwd_ms * 1e-3) / 1e12, 1),
            "ms_per_step": round(ms, 4),
            "step_ms_median": round(step_ms[len(step_ms) // 2], 4),
            "step_ms_min": round(step_ms[0], 4),
            "kernel_ms": {n: round(t, 4) for n, t in kern.items()},
            "effective_gflop_per_step": round((fwd_f + bwd_f) / 1e9, 1)}


def build_layers(name, dev, rope_mode):
    """The layers of one configuration: a single workload, or a model step
    of several layers whose windows come from fa_layer_window."""
    from causal_attention_fa_amd import fa, synth
    if name in LAYER_STEPS:
        base, window, every, n = LAYER_STEPS[name]
        w = synth.WORKLOADS[base]
        t = synth.draw(w)
        layers = []
        for layer in range(n):
            W = fa.fa_layer_window(layer, window, every)
            # each layer its own copy of the inputs (distinct memory, as in a model)
            layers.append(Layer(w.replace(window=W, global_every=every), W, t, dev, rope_mode))
        desc = {"workload": name, "layers": [L.window for L in layers], "B": w.B, "H": w.H,
                "Hkv": w.Hkv, "T": w.T, "d": w.d, "softcap": w.softcap,
                "global_every": every}
        return layers, desc
    w = synth.WORKLOADS[name]
    if w.dtype != "bf16":
        raise SystemExit("bench.py times the bf16 path; pick a bf16 workload")
    L = Layer(w, w.window, synth.draw(w), dev, rope_mode)
    desc = {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.Hkv, "T": w.T, "d": w.d,
            "d_v": w.dv, "window": w.window, "softcap": w.softcap,
            "global_every": w.global_every, "rope_theta": w.rope_theta,
            "visible_pairs_per_head": w.visible_pairs()}
    return [L], desc


def rope_leg(name, dev, iters=20):
    """rope_apply alone on the workload's Q and K (bf16 in and out): GB/s
    of its algorithmic bytes (read x, write y, the table) per call."""
    import torch
    from causal_attention_fa_amd import fa, synth
    w = synth.WORKLOADS[name]
    q, k, _, _ = synth.draw(w, need_do=False)
    tab = torch.from_numpy(fa.fa_rope_inv_freq(w.d, w.rope_theta)).to(dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    out = {}
    for nm, x, heads in (("q", q.to(dev), w.H), ("k", k.to(dev), w.Hkv)):
        y = torch.empty_like(x)
        for _ in range(3):
            fa.rope_apply(x, y, tab, w.B, heads, w.T, w.d, sh)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(iters):
            fa.rope_apply(x, y, tab, w.B, heads, w.T, w.d, sh)
        ev[1].record(stream)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / iters
        nbytes = 2 * x.numel() * x.element_size() + w.d // 2 * 4
        out[nm] = {"ms": round(ms, 4), "bytes": nbytes,
                   "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                   "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    return out


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
    ap.add_argument("--workload", default="mistral",
                    help="headline workload (a synth workload, or gemma2-step / gemma3-step)")
    ap.add_argument("--configs", default=DEFAULT_CONFIGS,
                    help="comma-separated further configurations timed after the headline "
                         "one ('none' to skip)")
    ap.add_argument("--config-steps", type=int, default=20)
    ap.add_argument("--config-warmup", type=int, default=5)
    ap.add_argument("--calibrate-copy-mb", type=float, default=0.0,
                    help="only run a plain device copy of this many MiB (5 times) and "
                         "exit: the reference kernel for scaling HBM byte counters")
    ap.add_argument("--rope", choices=["fused", "separate"], default="fused",
                    help="RoPE workloads: fused into the attention (fa_fwd_rope / "
                         "fa_bwd_rope; K rotated by rope_apply) or rope_apply on Q and K "
                         "around fa_fwd / fa_bwd")
    ap.add_argument("--rope-workloads", default="forge-default,qwen25",
                    help="workloads whose standalone RoPE is timed in GB/s ('none' to skip)")
    ap.add_argument("--dq-strategy", type=int, default=1,
                    help="1: time the backward under each dQ strategy (recomputing pass, "
                         "stored dS) beside the dQ-atomics traffic alone")
    ap.add_argument("--decode-workload", default="qwen25-decode",
                    help="decode workload timed after the main step ('none' to skip)")
    ap.add_argument("--decode-iters", type=int, default=20)
    ap.add_argument("--decode-only", action="store_true",
                    help="time only fa_decode on --decode-workload (one JSON line in GB/s)")
    ap.add_argument("--cpu-workers", type=int, default=16,
                    help="CPU baseline: oracle heads run at once, one per process "
                         "(0: skip the baseline)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not "
              "supported (the path shards by (batch, KV-head) groups with no exchange; "
              "see the design notes)", file=sys.stderr)
        sys.exit(2)

    from causal_attention_fa_amd import synth
    head = synth.WORKLOADS.get(args.workload)

    # the CPU baseline first: its worker pool forks, which must happen before
    # this process touches the GPU
    cpu = None
    if args.cpu_workers > 0 and args.calibrate_copy_mb <= 0 and not args.decode_only \
            and head is not None:
        log(f"[bench] timing the oracle on the host ({args.cpu_workers} workers max)")
        cpu = cpu_baseline(head, max_workers=args.cpu_workers)

    import torch
    dev = torch.device("cuda:0")

    if args.calibrate_copy_mb > 0:
        n = int(args.calibrate_copy_mb * (1 << 20)) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n * 4, "launches": 5}))
        return

    if args.decode_only:
        r = decode_leg(args.decode_workload, args.decode_iters, dev)
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

    from causal_attention_fa_amd import fa
    src_hash = kernel_sources_hash()
    log(f"[bench] headline workload {args.workload}")
    layers, desc = build_layers(args.workload, dev, args.rope)
    wall0 = time.perf_counter()
    ms, step_ms, kern = time_layers(layers, args.steps, args.warmup)
    wall = time.perf_counter() - wall0
    s = summarize(layers, ms, step_ms, kern)
    pairs_total = sum(L.flops()[2] for L in layers)
    w0 = layers[0].w
    bwd_names = layers[0].bwd_names
    # dominant kernel by time, priced at its own algorithmic flops
    dom = max(["fwd"] + bwd_names, key=lambda n: kern[n])
    dom_flops = kernel_flops_per_pair(dom, w0.d, w0.dv) * pairs_total
    achieved = dom_flops / (kern[dom] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_for(args.workload, dom, src_hash),
                "algorithmic_flops_per_launch": dom_flops,
                "avg_launch_ms": round(kern[dom], 4)}
    desc["effective_gflop_per_step"] = s["effective_gflop_per_step"]
    if layers[0].rope:
        desc["rope_mode"] = "fused" if layers[0].fused else "separate"
    out = {"metric": METRIC, "value": s["fwd_bwd_tflops"], "unit": "TFLOPS", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": s["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic", "config": desc,
           "roofline": roofline, "cpu_baseline": cpu}
    out.update({k: v for k, v in s.items() if k not in ("ms_per_step", "effective_gflop_per_step",
                                                        "fwd_bwd_tflops")})
    out["wall_s"] = round(wall, 3)
    out["kernel_sources_sha"] = src_hash
    del layers

    configs = {}
    for name in [c for c in args.configs.split(",") if c and c != "none"]:
        if name == args.workload:
            continue
        torch.cuda.empty_cache()
        log(f"[bench] config {name}")
        ls, d = build_layers(name, dev, args.rope)
        ms, step_ms, kern = time_layers(ls, args.config_steps, args.config_warmup)
        d.update(summarize(ls, ms, step_ms, kern))
        configs[name] = d
        del ls
    if configs:
        out["configs"] = configs

    # the dQ strategy, chosen by measurement: per workload the whole
    # backward with dQ recomputed by its own query-parallel pass (mode 1)
    # and with dQ from the dS tiles the dK/dV pass stores (mode 2, where the
    # head size allows), beside only the float atomics that accumulating dQ
    # in the dK/dV pass would issue (a lower bound on that variant's extra
    # cost over the dK/dV pass); the library's default (mode 0) is reported
    # beside the measured choice
    if args.dq_strategy:
        dqs = {}
        for name in [args.workload] + list(configs):
            w = synth.WORKLOADS.get(name)
            if w is None or w.dv != w.d:
                continue
            log(f"[bench] dq strategy {name}")
            r = {}
            for mode, key in ((1, "recompute"), (2, "stored_ds")):
                fa.fa_set_dq_mode(mode)
                try:
                    names = fa.fa_bwd_kernels(w.d)
                    if key == "stored_ds" and "dq_ds" not in names:
                        continue
                    torch.cuda.empty_cache()
                    ls, _ = build_layers(name, dev, args.rope)
                    _, _, km = time_layers(ls, 10, 3)
                    del ls
                finally:
                    fa.fa_set_dq_mode(0)
                r[key + "_bwd_ms"] = round(sum(km["bwd_" + n] for n in names), 4)
                r[key + "_kernel_ms"] = {n: round(km["bwd_" + n], 4) for n in names}
            torch.cuda.empty_cache()
            r["atomics_only_ms"] = round(
                fa.fa_measure_dq_atomics(w.B, w.H, w.Hkv, w.T, w.d, w.window), 4)
            dk = r["recompute_kernel_ms"]["dkdv"]
            cand = {"recompute": r["recompute_bwd_ms"],
                    "atomics (lower bound)": round(dk + r["atomics_only_ms"], 4)}
            if "stored_ds_bwd_ms" in r:
                cand["stored_ds"] = r["stored_ds_bwd_ms"]
            r["choice"] = min(cand, key=cand.get)
            r["library_default"] = "stored_ds" if "dq_ds" in fa.fa_bwd_kernels(w.d) else "recompute"
            # how far the default is from the fastest (run-to-run spread: ~2 %)
            r["default_vs_choice_pct"] = round(
                100 * (cand[r["library_default"]] / cand[r["choice"]] - 1), 2)
            dqs[name] = r
        out["dq_strategy"] = dqs

    rope = {}
    for name in [c for c in args.rope_workloads.split(",") if c and c != "none"]:
        torch.cuda.empty_cache()
        log(f"[bench] rope {name}")
        rope[name] = rope_leg(name, dev)
    if rope:
        out["rope_gbs"] = rope

    if args.decode_workload != "none":
        torch.cuda.empty_cache()
        log(f"[bench] decode leg: {args.decode_workload}")
        out["decode"] = decode_leg(args.decode_workload, args.decode_iters, dev)

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
