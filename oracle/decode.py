"""Float64 definition of single-query decode attention over a KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Forge commit "Add HF streaming data pipeline and three research reports",
INFERENCE_RESEARCH.md, section 2 ("KV cache"): the cache is preallocated at
the maximum length, laid out per head along time ([layer][head][seq][d]),
and a dedicated decode kernel serves one query against it, split along the
cache for long contexts; GQA is the largest saving in KV bandwidth.

One layer's cache is k_cache, v_cache [B, Hkv, S, d] (S = preallocated
length); sequence b currently holds lens[b] tokens, the last of which is the
new one, so its query sits at position p = lens[b] - 1.  For head h (KV head g = h // (H // Hkv)):

    s_j  = scale * <q[b,h], k_cache[b,g,j]>,  s'_j = cap*tanh(s_j/cap) or s_j
    vis  = j <= p and (W == 0 or j > p - W)       (j < lens[b])
    lse  = log( sum_{j vis} exp(s'_j) [+ exp(sink_h)] )
    o    = sum_{j vis} exp(s'_j - lse) v_cache[b,g,j]

i.e. exactly the last row of causal attention over the first lens[b]
positions (the same masks, cap and sinks as the training path).

Readings where the pages are silent:
  * cache entries at positions >= lens[b] are never read (they may hold
    anything);
  * lens[b] = 0 (no keys): o = 0 and lse = -inf, or lse = sink with a sink;
  * the pages keep the cache in f16; here it is stored in the dtype of the
    training path (bf16 on the GPU), which changes no arithmetic above.
"""
from __future__ import annotations

import numpy as np

__all__ = ["decode", "merge_partials"]


def decode(q, k_cache, v_cache, lens, scale, window=0, softcap=0.0, sinks=None):
    """q [B,H,d]; k_cache [B,Hkv,S,d]; v_cache [B,Hkv,S,dv]; lens [B].
    Returns (o [B,H,dv], lse [B,H]) in float64.

    Pinned against the independently pinned prefill oracle (last row of
    causal attention over the first lens[b] positions), by closed forms
    (zero query: mean of the visible values; window 1: the newest value)
    and by the empty cache.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k_cache, dtype=np.float64)
    v = np.asarray(v_cache, dtype=np.float64)
    B, H, d = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    if k.shape != (B, Hkv, S, d) or v.shape[:3] != (B, Hkv, S) or H % Hkv:
        raise ValueError("q [B,H,d], caches [B,Hkv,S,d] with H % Hkv == 0 expected")
    grp = H // Hkv
    o = np.zeros((B, H, v.shape[-1]))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        n = int(lens[b])
        if n < 0 or n > S:
            raise ValueError("lens[b] must lie in [0, S]")
        p = n - 1
        j = np.arange(n)
        vis = j > p - window if window > 0 else np.ones(n, dtype=bool)
        for h in range(H):
            g = h // grp
            s = scale * (k[b, g, :n] @ q[b, h])
            if softcap > 0:
                s = softcap * np.tanh(s / softcap)
            s = s[vis]
            terms = list(s)
            if sinks is not None:
                terms.append(float(sinks[h]))
            if not terms:
                continue
            m = max(terms)
            tot = np.exp(np.asarray(terms) - m).sum()
            lse[b, h] = m + np.log(tot)
            o[b, h] = np.exp(s - lse[b, h]) @ v[b, g, :n][vis]
    return o, lse


def merge_partials(os_, lses):
    """Exact merge of attention over disjoint key sets: partial outputs o_r
    (each normalised over its own keys) with log-normalisers lse_r give
    lse = log sum_r exp(lse_r) and o = sum_r exp(lse_r - lse) o_r.  This is
    the identity a split-along-the-cache decode relies on; parts with
    lse_r = -inf (no keys) drop out.  os_ [R, ..., dv], lses [R, ...]."""
    os_ = np.asarray(os_, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    m = np.max(lses, axis=0)
    safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lses - safe)
    tot = w.sum(axis=0)
    lse = np.where(tot > 0, safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    wn = np.where(tot > 0, w / np.where(tot > 0, tot, 1.0), 0.0)
    return np.einsum("r...,r...d->...d", wn, os_), lse
