"""Seeded synthetic inputs and the workload table.

This module holds no arithmetic of the attention method: it only names the
workloads and draws their random tensors.  Both the HIP path (through the
tests and the benchmark) and the CPU oracle consume what it draws.

Recipe: one ``torch.Generator('cpu')`` seeded per workload; tensors drawn in
the order Q, K, V, dO as float32 ``randn * sigma``; for bf16 workloads each
tensor is then rounded to bfloat16 (round-to-nearest-even, torch's cast).
The oracle receives the exact rounded values upcast to float64.

Workloads (shapes of the models the pages describe; no dataset is used):
  forge-f32     B1 H2/2 T128 d64 fp32, causal               (Forge default
                head size; a case the oracle finishes in seconds)
  forge-default B32 H6/6 T512 d64 bf16, causal, RoPE 1e4    (Forge default
                model: 6 heads, d_model 384, context 512, micro-batch 32)
  qwen25        B8 H28/4 T2048 d128 bf16, causal, RoPE 1e6  (Qwen 2.5 row of
                the ARCHITECTURES.md family table: GQA 28H/4KV, theta 1e6)
  mistral       B4 H32/8 T8192 d128 bf16, window 4096       (Mistral 7B row)
  gemma-local   B2 H8/4 T8192 d256 bf16, window 4096, cap 50 (Gemma 2 row)
  gemma-global  same, full causal, cap 50
  gemma3-local  same, window 1024, cap 50 (Gemma 3 row: 5 local : 1 global,
                window 1024; the global layer is gemma-global)
  mla           B2 H16/16 T8192 d192 d_v128 bf16, causal, scale 1/sqrt(192)
                (DeepSeek-V3 / Kimi K2 MLA with the latent decompressed:
                q, k 128 + 64 rotary dims, v 128; 16 heads = one GPU's
                share of Kimi K2's 64 under 4-way head parallelism)

Decode workloads (one new token per sequence, preallocated 32k bf16 cache,
ragged lengths uniform in [16384, 32768]):
  qwen25-decode        B32 H28/4 S32768 d128, V ~ N(0, 0.5^2)
  mistral-decode       B32 H32/8 S32768 d128, window 4096
  gemma-global-decode  B16 H8/4 S32768 d256, cap 50, Q, K ~ N(0, 2^2)
"""
from __future__ import annotations

import dataclasses
import math

import torch

__all__ = ["Workload", "WORKLOADS", "draw", "to_f64", "DecodeWorkload", "DECODE_WORKLOADS",
           "draw_decode"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16"
    B: int
    H: int
    Hkv: int
    T: int
    d: int
    window: int = 0
    softcap: float = 0.0
    global_every: int = 0
    rope_theta: float = 0.0   # 0: no RoPE pre-step
    sigma_qk: float = 1.0
    sigma_vdo: float = 1.0
    seed: int = 0
    d_v: int = 0              # value head size; 0: same as d

    @property
    def dv(self) -> int:
        return self.d_v or self.d

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def visible_pairs(self) -> int:
        """Number of (query, key) pairs the mask lets through per head."""
        T, W = self.T, self.window
        if W <= 0 or W >= T:
            return T * (T + 1) // 2
        return W * (W + 1) // 2 + (T - W) * W

    def fwd_flops(self) -> float:
        """Effective forward FLOPs: 2*(d + d_v) per visible pair (QK^T and
        PV; 4*d when d_v = d)."""
        return 2.0 * (self.d + self.dv) * self.visible_pairs() * self.B * self.H

    def bwd_flops(self) -> float:
        """Effective backward FLOPs: five products per visible pair -- QK^T
        recompute, dS K, dS^T Q (length d) and dO V^T, P^T dO (length d_v):
        2*(3d + 2d_v), i.e. 2.5x forward when d_v = d."""
        return 2.0 * (3 * self.d + 2 * self.dv) * self.visible_pairs() * self.B * self.H

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    w.name: w for w in [
        Workload("forge-f32", "f32", 1, 2, 2, 128, 64),
        Workload("forge-default", "bf16", 32, 6, 6, 512, 64, rope_theta=1e4),
        Workload("qwen25", "bf16", 8, 28, 4, 2048, 128, rope_theta=1e6,
                 sigma_vdo=0.5),
        Workload("mistral", "bf16", 4, 32, 8, 8192, 128, window=4096),
        Workload("gemma-local", "bf16", 2, 8, 4, 8192, 256, window=4096,
                 softcap=50.0, sigma_qk=2.0),
        Workload("gemma-global", "bf16", 2, 8, 4, 8192, 256, window=0,
                 softcap=50.0, sigma_qk=2.0),
        Workload("gemma3-local", "bf16", 2, 8, 4, 8192, 256, window=1024,
                 softcap=50.0, global_every=6, sigma_qk=2.0),
        Workload("mla", "bf16", 2, 16, 16, 8192, 192, d_v=128),
    ]
}


def draw(w: Workload, seed: int | None = None, need_do: bool = True):
    """Seeded CPU tensors (q, k, v, do) of workload ``w``.

    q: [B, H, T, d]; k: [B, Hkv, T, d]; v: [B, Hkv, T, d_v]; do: [B, H, T, d_v]
    (d_v = d unless the workload sets it); dtype float32 or bfloat16 as
    the workload says.  ``do`` is None when ``need_do`` is False.
    """
    g = torch.Generator("cpu")
    g.manual_seed(w.seed if seed is None else seed)
    shp_q = (w.B, w.H, w.T, w.d)
    shp_k = (w.B, w.Hkv, w.T, w.d)
    q = torch.randn(shp_q, generator=g, dtype=torch.float32) * w.sigma_qk
    k = torch.randn(shp_k, generator=g, dtype=torch.float32) * w.sigma_qk
    v = torch.randn(shp_k[:3] + (w.dv,), generator=g, dtype=torch.float32) * w.sigma_vdo
    do = None
    if need_do:
        do = torch.randn(shp_q[:3] + (w.dv,), generator=g, dtype=torch.float32) * w.sigma_vdo
    dt = w.torch_dtype
    out = [t.to(dt) if t is not None else None for t in (q, k, v, do)]
    return tuple(out)


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """One new token per sequence against a preallocated bf16 KV cache of
    S positions; sequence b holds lens[b] tokens, drawn uniformly from
    [lens_lo, S] (ragged batch)."""
    name: str
    B: int
    H: int
    Hkv: int
    S: int
    d: int
    window: int = 0
    softcap: float = 0.0
    lens_lo: int = 1
    sigma_qk: float = 1.0
    sigma_v: float = 1.0
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def replace(self, **kw) -> "DecodeWorkload":
        return dataclasses.replace(self, **kw)


# Decode counterparts of the training workloads, at a serving batch and a
# 32k cache, so that the cache (>= 0.5 GB read per call) streams from HBM
# rather than the 256 MB last-level cache.
DECODE_WORKLOADS = {
    w.name: w for w in [
        DecodeWorkload("qwen25-decode", 32, 28, 4, 32768, 128, lens_lo=16384,
                       sigma_v=0.5),
        DecodeWorkload("mistral-decode", 32, 32, 8, 32768, 128, window=4096,
                       lens_lo=16384),
        DecodeWorkload("gemma-global-decode", 16, 8, 4, 32768, 256, softcap=50.0,
                       lens_lo=16384, sigma_qk=2.0),
    ]
}


def draw_decode(w: DecodeWorkload, device="cpu", seed: int | None = None):
    """Seeded (q [B,H,d], k_cache, v_cache [B,Hkv,S,d] bf16, lens [B] int32)
    on ``device``.  lens first (CPU generator), then q, K, V as float32
    randn * sigma rounded to bf16, drawn by a generator on ``device`` (the
    caches of the full-size workloads are several GB)."""
    s = w.seed if seed is None else seed
    gc = torch.Generator("cpu")
    gc.manual_seed(s)
    lens = torch.randint(w.lens_lo, w.S + 1, (w.B,), generator=gc, dtype=torch.int32)
    g = torch.Generator(device)
    g.manual_seed(s + 1)
    q = (torch.randn((w.B, w.H, w.d), generator=g, device=device) * w.sigma_qk).to(torch.bfloat16)
    shp = (w.B, w.Hkv, w.S, w.d)
    k = torch.empty(shp, dtype=torch.bfloat16, device=device)
    v = torch.empty(shp, dtype=torch.bfloat16, device=device)
    for b in range(w.B):   # per sequence: bounded float32 temporaries
        k[b] = (torch.randn(shp[1:], generator=g, device=device) * w.sigma_qk).to(torch.bfloat16)
        v[b] = (torch.randn(shp[1:], generator=g, device=device) * w.sigma_v).to(torch.bfloat16)
    return q, k, v, lens.to(device)


def to_f64(t):
    """Exact float64 numpy copy of a CPU tensor (bf16 values upcast)."""
    return t.detach().to("cpu", torch.float64).numpy()
