"""Per-element error envelopes for the bf16 attention path (test code).

A bf16 output X of the GPU path passes when, element by element,

    |X_gpu - X_ref| <= R_BAR * rms(X_ref) + E_X

and rms(X_gpu - X_ref) / rms(X_ref) <= R_BAR, where X_ref is the float64
oracle's value on the exact bf16 inputs and R_BAR = 2e-2 is the stated bf16
tolerance (relative to the output's RMS).  E_X is the largest effect of the
roundings the method's reading allows, propagated to X, and is computed here
from the oracle's inputs and float64 intermediates only; no value computed
on the GPU enters it.  The allowed roundings:

  * every bf16 output is rounded to nearest even: U16 |X_ref|, U16 = 2^-8
    (half an ulp of an 8-bit significand is at most 2^-8 of the value);
  * P is rounded to bf16 before the products P V (forward) and P^T dO (dV);
    dS is rounded to bf16 before dS K (dQ) and, with the factor that
    multiplies (dP - D) rounded first, before dS^T Q (dK);
  * D_i = <dO_i, o_i> is formed from the bf16 o the forward returned (its
    output rounding and its P rounding both enter D);
  * scores, exponentials, sums and lse are float32.

Roundings of different elements are independent and centred: their sum
over a contraction is bounded by Hoeffding's inequality at LAMBDA "sigma"
(probability below 2 exp(-LAMBDA^2 / 2) = 2.5e-14 per element that a
correct kernel exceeds it).  Errors shared by a whole row (D, lse, the
float32 score error) are bounded in the worst case.  Float32 accumulation
over d terms uses the deterministic bound d * 2^-24; over n keys or queries
the probabilistic lambda * sqrt(n) * 2^-24.  The envelope is pinned in
tests/test_envelope.py against an emulation of exactly these roundings
(which must stay inside it with R_BAR = 0) and against planted mistakes
(which must fall outside it).
"""
from __future__ import annotations

import math

import numpy as np

from oracle import attention as OA

R_BAR = 2e-2
LAMBDA = 8.0
U16 = 2.0 ** -8
U32 = 2.0 ** -24


def _abs(x):
    return np.abs(x)


def head_envelopes(q, k, v, do, scale, window, cap, q_rows=None, kv_rows=None, sink=None,
                   row_block=512, rows=None):
    """Oracle values and envelopes for one (b, h).

    q: [T, d] this head's queries; k [T, d], v [T, d_v] its KV head; do
    [T, d_v] or None (forward only).  o and lse (oracle.head_forward_rows)
    on every row (or on ``rows``); with ``do``: dq at ``q_rows`` and this
    head's parts of dk, dv at ``kv_rows`` (oracle.head_grads_sampled), and
    the envelope pieces that combine_kv() sums over a GQA group.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    T, d = k.shape
    dv = v.shape[1]
    sig = 1 if sink is not None else 0
    W = window if 0 < window < T else 0
    all_rows = np.arange(T) if rows is None else np.asarray(rows)
    bwd = do is not None
    if bwd:
        do = np.asarray(do, dtype=np.float64)
        assert rows is None, "the backward envelope needs every query row"
    out = {"o": np.empty((len(all_rows), dv)), "lse": np.empty(len(all_rows)),
           "E_o": np.empty((len(all_rows), dv)), "E_lse": np.empty(len(all_rows))}
    kmax = np.linalg.norm(k, axis=1).max()
    vmax = np.linalg.norm(v, axis=1).max()
    q_rows = np.asarray([] if q_rows is None else q_rows, dtype=int)
    kv_rows = np.asarray([] if kv_rows is None else kv_rows, dtype=int)
    if bwd:
        E_dq = np.zeros((len(q_rows), d))
        kv = dict(var_dk=np.zeros((len(kv_rows), d)), lin_dk=np.zeros((len(kv_rows), d)),
                  abs_dk=np.zeros((len(kv_rows), d)), var_dv=np.zeros((len(kv_rows), dv)),
                  lin_dv=np.zeros((len(kv_rows), dv)), abs_dv=np.zeros((len(kv_rows), dv)),
                  n=np.zeros(len(kv_rows)))
        qpos = {int(r): i for i, r in enumerate(q_rows)}
    for r0 in range(0, len(all_rows), row_block):
        rws_abs = all_rows[r0:r0 + row_block]
        sl = slice(r0, r0 + len(rws_abs))
        # keys the block's rows can see: [klo, khi); the rest contribute
        # exact zeros, so the oracle is evaluated on that key range with
        # positions shifted by klo (visibility depends on differences only)
        khi = int(rws_abs.max()) + 1
        klo = max(0, int(rws_abs.min()) - W + 1) if W > 0 else 0
        kk, vv = k[klo:khi], v[klo:khi]
        rws = rws_abs - klo
        qq = q[klo:]
        cols = np.arange(khi - klo)
        o, lse, P = OA.head_forward_rows(qq, kk, vv, scale, W, cap, rws, sink=sink)
        vis = OA.visibility(rws, cols, W)
        n = vis.sum(1) + sig
        s = scale * (qq[rws] @ kk.T)
        sc = OA.capped_scores(s, cap)
        t = 1.0 - np.tanh(s / cap) ** 2 if cap > 0 else 1.0
        # float32 relative error of one unrounded p: the score's dot product
        # (sum |q_c k_c| <= |q| |k|), the tanh (a few ulps, times the cap),
        # the exp2 argument (|S'| log2 e + |m| in log2 units) and exp2
        smax = np.where(vis, _abs(sc), 0.0).max(1)
        rho = (d * U32 * scale * np.linalg.norm(qq[rws], axis=1) * kmax
               + (8 * U32 * cap if cap > 0 else 0.0) + 4 * U32 * (2 * smax + 16))
        kap = rho + LAMBDA * np.sqrt(n) * U32 + 4 * U32
        Pv = P @ _abs(vv)
        # o: output rounding, P rounded before P V (random over keys), the
        # float32 terms (shared relative error of p, sums over n keys, 1/l)
        e_o = LAMBDA * U16 * np.sqrt((P * P) @ (vv * vv)) + kap[:, None] * (Pv + _abs(o))
        out["o"][sl] = o
        out["lse"][sl] = lse
        out["E_o"][sl] = U16 * _abs(o) + (1 + U16) * e_o
        out["E_lse"][sl] = rho + LAMBDA * np.sqrt(n) * U32 + 4 * U32 * (_abs(lse) + 16)
        if not bwd:
            continue
        dO = do[rws_abs]
        D = (dO * o).sum(1)
        dP = dO @ vv.T
        # error of the kernel's D_i: from the forward's bf16 o (its output
        # rounding and float32 terms, worst case over c; its P rounding,
        # random over keys: sum_j dP_ij dP_ij-weighted), plus D's own dot
        eD = ((_abs(dO) * (U16 * _abs(o) + kap[:, None] * (Pv + _abs(o)))).sum(1)
              + LAMBDA * U16 * np.sqrt(((P * dP) ** 2).sum(1))
              + dv * U32 * (_abs(dO) * _abs(o)).sum(1))
        beta = dv * U32 * np.linalg.norm(dO, axis=1) * vmax     # dP's dot product
        eps = rho + out["E_lse"][sl]       # relative error of the recomputed P
        dSp = P * (dP - D[:, None])        # dS' (before the tanh' factor)
        dS = dSp * t
        Pt = P * t
        # deterministic error of the kernel's dS before its bf16 rounding
        e_dS = eps[:, None] * _abs(dS) + Pt * (eD + beta)[:, None]
        if cap > 0:
            e_dS = e_dS + 2.0 ** -21 * _abs(dSp)   # 1 - tanh^2 in float32
        # dq rows in this block
        sel = np.array([i for i, r in enumerate(rws_abs) if int(r) in qpos], dtype=int)
        if len(sel):
            dsr = dS[sel]
            e = (LAMBDA * U16 * np.sqrt((dsr * dsr) @ (kk * kk)) + e_dS[sel] @ _abs(kk)
                 + (LAMBDA * np.sqrt(n[sel]) * U32)[:, None] * (_abs(dsr) @ _abs(kk)))
            for j, r in enumerate(rws_abs[sel]):
                E_dq[qpos[int(r)]] = scale * e[j]
        inr = np.nonzero((kv_rows >= klo) & (kv_rows < khi))[0]   # sampled keys in range
        if len(inr):
            lc = kv_rows[inr] - klo
            dsc = dS[:, lc]
            pc = P[:, lc]
            qb = q[rws_abs]
            kv["var_dk"][inr] += (dsc * dsc).T @ (qb * qb)
            kv["lin_dk"][inr] += e_dS[:, lc].T @ _abs(qb)
            kv["abs_dk"][inr] += _abs(dsc).T @ _abs(qb)
            kv["var_dv"][inr] += (pc * pc).T @ (dO * dO)
            kv["lin_dv"][inr] += (eps[:, None] * pc).T @ _abs(dO)
            kv["abs_dv"][inr] += pc.T @ _abs(dO)
            kv["n"][inr] += vis[:, lc].sum(0)
    if not bwd:
        return out
    dq, dk, dvv, _, _ = OA.head_grads_sampled(q, k, v, do, scale, W, cap, q_rows, kv_rows,
                                              sink=sink)
    out["dq"] = dq
    out["E_dq"] = U16 * _abs(dq) + (1 + U16) * E_dq
    out["dk_part"], out["dv_part"] = dk, dvv
    out["kv"] = kv
    out["scale"] = scale
    return out


def combine_kv(parts):
    """dk, dv of a KV head (summed over its query heads) and their envelopes
    from head_envelopes() results of every query head of the group."""
    scale = parts[0]["scale"]
    dk = sum(p["dk_part"] for p in parts)
    dv = sum(p["dv_part"] for p in parts)
    acc = {n: sum(p["kv"][n] for p in parts) for n in parts[0]["kv"]}
    nn = acc["n"][:, None]
    # dK: two roundings per element (the bf16 factor, then dS itself)
    e_dk = scale * (LAMBDA * U16 * np.sqrt(2.0 * acc["var_dk"]) + acc["lin_dk"]
                    + LAMBDA * np.sqrt(nn) * U32 * acc["abs_dk"])
    e_dv = (LAMBDA * U16 * np.sqrt(acc["var_dv"]) + acc["lin_dv"]
            + LAMBDA * np.sqrt(nn) * U32 * acc["abs_dv"])
    return {"dk": dk, "dv": dv, "E_dk": U16 * _abs(dk) + (1 + U16) * e_dk,
            "E_dv": U16 * _abs(dv) + (1 + U16) * e_dv}


def full_envelopes(q, k, v, do, scale, window, cap, sinks=None):
    """o, lse, dq, dk, dv of batched tensors (every element) with their
    envelopes: q, do [B, H, T, d(_v)], k, v [B, Hkv, T, d(_v)], float64."""
    B, H, T, d = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    res = {n: [] for n in ("o", "lse", "dq", "E_o", "E_lse", "E_dq")}
    shape_kv = {"dk": np.zeros(k.shape), "dv": np.zeros(v.shape),
                "E_dk": np.zeros(k.shape), "E_dv": np.zeros(v.shape)}
    allr = np.arange(T)
    for b in range(B):
        for g in range(Hkv):
            parts = []
            for h in range(g * G, (g + 1) * G):
                sk = None if sinks is None else float(sinks[h])
                p = head_envelopes(q[b, h], k[b, g], v[b, g], None if do is None else do[b, h],
                                   scale, window, cap, q_rows=allr, kv_rows=allr, sink=sk)
                parts.append(p)
            if do is not None:
                c = combine_kv(parts)
                for n in shape_kv:
                    shape_kv[n][b, g] = c[n]
            for p in parts:
                for n in ("o", "lse", "E_o", "E_lse") + (("dq", "E_dq") if do is not None else ()):
                    res[n].append(p[n])
    out = {}
    for n, xs in res.items():
        if xs:
            out[n] = np.stack(xs).reshape((B, H) + xs[0].shape)
    if do is not None:
        out.update(shape_kv)
    return out


def r_bar_for(name):
    """RMS allowance of an output: R_BAR, except lse, which the kernels
    compute in float32 and which is held to its float32 envelope alone (an
    allowance relative to its RMS, ~8 at T = 8192, would let a row be off
    by a sizeable fraction of a nat)."""
    return 0.0 if name.startswith("lse") else R_BAR


def excess(got, ref, env, r_bar=R_BAR):
    """max over elements of |got - ref| / (r_bar rms(ref) + env); inf if got
    has a non-finite element."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not np.all(np.isfinite(got)):
        return float("inf")
    if got.size == 0:
        return 0.0
    rms = math.sqrt(float(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref) / (r_bar * rms + env + 1e-300)))


def rms_rel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not np.all(np.isfinite(got)):
        return float("inf")
    rms = math.sqrt(float(np.mean(ref * ref))) or 1.0
    return math.sqrt(float(np.mean((got - ref) ** 2))) / rms


def rotate_env(env, pair_axis=-1):
    """Envelope of a pairwise rotation (RoPE backward) of a quantity whose
    elements are bounded by env: each output element of a pair is bounded
    by the sum of the pair's two bounds (|cos|, |sin| <= 1)."""
    e = np.asarray(env)
    ev, od = e[..., 0::2], e[..., 1::2]
    s = ev + od
    out = np.empty_like(e)
    out[..., 0::2] = s
    out[..., 1::2] = s
    return out


def decode_envelopes(q, k, v, lens, scale, window, cap, sinks=None):
    """Envelopes of single-query decode (q [B, H, d]; caches [B, Hkv, S, d],
    float64; sequence b holds lens[b] tokens, its query at position
    lens[b] - 1): E_o [B, H, d], E_lse [B, H] (rows with lens = 0: 0)."""
    B, H, d = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    E_o = np.zeros((B, H, v.shape[-1]))
    E_lse = np.zeros((B, H))
    for b in range(B):
        n = int(lens[b])
        if n <= 0:
            continue
        for h in range(H):
            qq = np.zeros((n, d))
            qq[n - 1] = q[b, h]
            sk = None if sinks is None else float(sinks[h])
            r = head_envelopes(qq, k[b, h // G, :n], v[b, h // G, :n], None, scale, window, cap,
                               rows=[n - 1], sink=sk)
            E_o[b, h] = r["E_o"][0]
            E_lse[b, h] = r["E_lse"][0]
    return E_o, E_lse
