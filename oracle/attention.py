"""Float64 definition of causal attention with GQA, sliding window and softcap.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, for every batch b and query head h, with the key/value head
g = h // (H // Hkv) (contiguous groups, i.e. K/V heads repeat-interleaved):

    S[i, j]  = scale * <q[b,h,i], k[b,g,j]>
    S'[i, j] = cap * tanh(S[i, j] / cap)      if cap > 0, else S[i, j]
    vis(i,j) = j <= i  and  (W == 0  or  j > i - W)
    lse[i]   = log sum_{j vis} exp(S'[i, j])                (natural log)
    P[i, j]  = exp(S'[i, j] - lse[i])  on visible pairs, 0 elsewhere
    o[i]     = sum_j P[i, j] v[b,g,j]

Backward of L = sum(o * dO):

    dP[i,j] = <dO[i], v[j]>,   D[i] = <dO[i], o[i]>
    dS'     = P * (dP - D[:, None])
    dS      = dS' * (1 - tanh(S/cap)^2)   if cap > 0, else dS'
    dq[i]   = scale * sum_j dS[i,j] k[j]
    dk[g,j] = scale * sum_{h in g} sum_i dS[i,j] q[h,i]
    dv[g,j] = sum_{h in g} sum_i P[i,j] dO[h,i]

Sources: Forge ARCHITECTURES.md, prioritised plan wave 2, item 8 (the causal
mask becomes q-W < k <= q for a window W) and item 9 (cap*tanh(s/cap) on the
pre-softmax scores); Forge attention.h commit log, "Wave 2" (softcap backward
through the exact derivative of tanh); ARCHITECTURES.md family table (GQA, a
query head reads the KV head of its group).  Flash attention reaches exactly
this result (up to rounding order), so the oracle is the plain definition
with the full score matrix, not a replay of a tiled algorithm.

Readings where the pages are silent:
  * softcap acts on the *scaled* score, before masking;
  * window W counts W keys including the query itself (W=1: self only);
    W == 0 or W >= T is full causal;
  * GQA groups are contiguous: head h reads KV head h // (H // Hkv).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "layer_window", "visibility", "capped_scores", "head_forward",
    "head_backward", "attn_fwd", "attn_bwd", "head_forward_rows",
    "head_grads_sampled", "max_logit",
]


def layer_window(layer: int, window: int, global_every: int) -> int:
    """Effective window of one layer of a local:global stack.

    Forge commit log for src/nn/attention.h, "Wave 2": sliding_window with
    sliding_global_every gives the Mistral pattern (every layer windowed)
    and the Gemma 3 pattern (ARCHITECTURES.md family table: 5 local to 1
    global).  Reading: with global_every = n > 0 every n-th layer, counting
    from 1 (0-based layers n-1, 2n-1, ...), is global (returns 0); all other
    layers use ``window``.  global_every = 0 means every layer uses
    ``window``.  So 5 local : 1 global is global_every = 6.

    Pinned: tests/test_oracle_attention.py::test_layer_window_patterns.
    """
    if global_every < 0 or window < 0:
        raise ValueError("window and global_every must be >= 0")
    if global_every > 0 and (layer + 1) % global_every == 0:
        return 0
    return window


def visibility(rows: np.ndarray, cols: np.ndarray, window: int) -> np.ndarray:
    """Boolean mask vis[i, j] for query positions ``rows`` and key positions
    ``cols``: causal (key at or before the query) and, for 0 < window, the
    key is among the ``window`` most recent positions (q - W < k <= q;
    ARCHITECTURES.md, plan wave 2, item 8).

    Pinned: closed forms with window = 1 (self only) and q = 0 (uniform
    weights over min(i+1, W) keys); window >= T equals full causal.
    """
    i = np.asarray(rows)[:, None]
    j = np.asarray(cols)[None, :]
    vis = j <= i
    if window > 0:
        vis &= j > i - window
    return vis


def capped_scores(s: np.ndarray, softcap: float) -> np.ndarray:
    """cap * tanh(s / cap) for cap > 0, identity for cap == 0
    (ARCHITECTURES.md, plan wave 2, item 9).

    Pinned: T = 1 closed form lse = cap*tanh(scale*q.k/cap); cap = 1e8
    equals no cap.
    """
    if softcap > 0:
        return softcap * np.tanh(s / softcap)
    return s


def head_forward_rows(q, k, v, scale, window, softcap, rows=None, sink=None):
    """Forward of one (b, h) pair restricted to query positions ``rows``.

    q: [T, d] (this head's queries), k, v: [T, d_v] (its KV head).  Returns
    (o[rows], lse[rows], P[rows, :]) in float64.  Each output row depends
    only on its own row of S, so evaluating a subset of rows is the same
    definition, not a reordering.

    ``sink`` (a scalar logit, or None): the attention sink of GPT-OSS
    (ARCHITECTURES.md family table, and plan wave 2 item 10: a learned
    per-head logit in the softmax denominator that the online softmax
    starts its (max, sum) from).  It joins every row's normaliser but
    carries no value: lse = log(sum_j exp(S'_ij) + exp(sink)).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T = k.shape[0]
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    s = scale * (q[rows] @ k.T)
    sc = capped_scores(s, softcap)
    vis = visibility(rows, np.arange(T), window)
    sm = np.where(vis, sc, -np.inf)
    m = sm.max(axis=1)
    if sink is not None:
        m = np.maximum(m, sink)
    tot = np.exp(sm - m[:, None]).sum(axis=1)
    if sink is not None:
        tot = tot + np.exp(sink - m)
    lse = m + np.log(tot)
    p = np.exp(sm - lse[:, None])
    o = p @ v
    return o, lse, p


def head_forward(q, k, v, scale, window, softcap, sink=None):
    """Forward of one (b, h): (o [T, d], lse [T], P [T, T])."""
    return head_forward_rows(q, k, v, scale, window, softcap, sink=sink)


def head_backward(q, k, v, do, scale, window, softcap, sink=None):
    """Gradients of L = sum(o * dO) for one (b, h), all in float64.

    Returns (dq, dk, dv), each [T, d]; dk and dv are this query head's
    contribution to its KV head.  The softcap chain multiplies by
    1 - tanh(S/cap)^2, the exact derivative (Forge attention.h commit log,
    "Wave 2").

    With a sink, P is normalised including exp(sink) and the same formulas
    hold; the sink's own gradient is d sink = -sum_i exp(sink - lse_i) D_i
    (returned as a fourth value when ``sink`` is given).

    Pinned: central finite differences of head_forward (also w.r.t. the
    sink); closed forms for window = 1 and q = 0; all keys equal => dq = 0;
    torch.autograd of the library SDPA in the plain causal case.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    o, lse, p = head_forward(q, k, v, scale, window, softcap, sink=sink)
    dp = do @ v.T
    D = (do * o).sum(axis=1)
    dsc = p * (dp - D[:, None])
    if softcap > 0:
        s = scale * (q @ k.T)
        ds = dsc * (1.0 - np.tanh(s / softcap) ** 2)
    else:
        ds = dsc
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    dv = p.T @ do
    if sink is not None:
        dsink = -float((np.exp(sink - lse) * D).sum())
        return dq, dk, dv, dsink
    return dq, dk, dv


def max_logit(q, k, scale, window=0, softcap=0.0):
    """Largest logit entering the softmax, per (b, h): max over visible
    (i, j) of S'_ij (= scale * <q_i, k_j> without a cap).  The per-head
    quantity QK-Clip monitors (ARCHITECTURES.md family table, Kimi K2
    MuonClip; plan wave 3 item 12: the flash kernel already keeps the row
    max, expose it).  Returns [B, H].

    Pinned: brute force over pairs on a tiny case; window = 1 closed form.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, H, T, _ = q.shape
    Hkv = k.shape[1]
    grp = H // Hkv
    out = np.empty((B, H))
    vis = visibility(np.arange(T), np.arange(T), window)
    for b in range(B):
        for h in range(H):
            sc = capped_scores(scale * (q[b, h] @ k[b, h // grp].T), softcap)
            out[b, h] = np.where(vis, sc, -np.inf).max()
    return out


def _check_shapes(q, k, v):
    B, H, T, d = q.shape
    Bk, Hkv, Tk, dk_ = k.shape
    if (Bk, Tk, dk_) != (B, T, d) or v.shape[:3] != k.shape[:3]:
        raise ValueError("q [B,H,T,d], k [B,Hkv,T,d], v [B,Hkv,T,dv] expected")
    if Hkv <= 0 or H % Hkv != 0:
        raise ValueError("H must be a multiple of Hkv")
    return B, H, Hkv, T, d


def attn_fwd(q, k, v, scale, window=0, softcap=0.0, sinks=None):
    """Batched forward.  q [B,H,T,d]; k [B,Hkv,T,d]; v [B,Hkv,T,dv] (d_v may
    differ from d, as in MLA: ARCHITECTURES.md plan wave 3 item 13).
    ``sinks``: optional [H] per-head sink logits.  Returns
    (o [B,H,T,dv], lse [B,H,T]) in float64."""
    B, H, Hkv, T, d = _check_shapes(q, k, v)
    grp = H // Hkv
    o = np.empty((B, H, T, v.shape[-1]))
    lse = np.empty((B, H, T))
    for b in range(B):
        for h in range(H):
            g = h // grp
            sk = None if sinks is None else float(sinks[h])
            o[b, h], lse[b, h], _ = head_forward(q[b, h], k[b, g], v[b, g],
                                                 scale, window, softcap, sink=sk)
    return o, lse


def attn_bwd(q, k, v, do, scale, window=0, softcap=0.0, sinks=None):
    """Batched backward.  Returns (dq [B,H,T,d], dk [B,Hkv,T,d],
    dv [B,Hkv,T,dv]); the KV gradients sum over the query heads of each
    group.  With ``sinks`` ([H]) a fourth value dsinks [H] (summed over the
    batch) is returned."""
    B, H, Hkv, T, d = _check_shapes(q, k, v)
    grp = H // Hkv
    dq = np.empty((B, H, T, d))
    dk = np.zeros((B, Hkv, T, d))
    dv = np.zeros((B, Hkv, T, v.shape[-1]))
    dsinks = np.zeros(H)
    for b in range(B):
        for h in range(H):
            g = h // grp
            sk = None if sinks is None else float(sinks[h])
            res = head_backward(q[b, h], k[b, g], v[b, g], do[b, h],
                                scale, window, softcap, sink=sk)
            dq[b, h] = res[0]
            dk[b, g] += res[1]
            dv[b, g] += res[2]
            if sinks is not None:
                dsinks[h] += res[3]
    if sinks is not None:
        return dq, dk, dv, dsinks
    return dq, dk, dv


def head_grads_sampled(q, k, v, do, scale, window, softcap, q_rows, kv_rows,
                       row_block=1024, sink=None):
    """The backward definition evaluated only where a sampled check needs it.

    For one (b, h): dq at query positions ``q_rows`` and this head's
    contribution to dk, dv at key positions ``kv_rows``.  The statistics that
    those entries depend on -- lse[i] and D[i] = <dO[i], o[i]> for every
    query row i -- come from head_forward_rows evaluated ``row_block`` rows
    at a time (to bound memory at T = 8192); every formula is the one in
    head_backward, restricted to the needed rows or columns.
    Returns (dq [len(q_rows), d], dk, dv [len(kv_rows), d], o, lse [T]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    T = k.shape[0]
    lse = np.empty(T)
    o = np.empty((q.shape[0], v.shape[1]))
    for r0 in range(0, T, row_block):
        rows = np.arange(r0, min(T, r0 + row_block))
        o[rows], lse[rows], _ = head_forward_rows(q, k, v, scale, window,
                                                  softcap, rows, sink=sink)
    D = (do * o).sum(axis=1)
    q_rows = np.asarray(q_rows)
    kv_rows = np.asarray(kv_rows)
    allq = np.arange(T)

    def _ds_p(rows, cols):
        s = scale * (q[rows] @ k[cols].T)
        sc = capped_scores(s, softcap)
        vis = visibility(rows, cols, window)
        p = np.where(vis, np.exp(np.where(vis, sc, 0.0) - lse[rows][:, None]),
                     0.0)
        dp = do[rows] @ v[cols].T
        ds = p * (dp - D[rows][:, None])
        if softcap > 0:
            ds = ds * (1.0 - np.tanh(s / softcap) ** 2)
        return ds, p

    ds_r, _ = _ds_p(q_rows, allq)
    dq = scale * (ds_r @ k)
    ds_c, p_c = _ds_p(allq, kv_rows)
    dk = scale * (ds_c.T @ q)
    dv = p_c.T @ do
    return dq, dk, dv, o, lse
