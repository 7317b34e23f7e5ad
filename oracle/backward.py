"""Gradients of exact attention, in fp64 (TEST INFRASTRUCTURE ONLY).

The pages name the backward pass only briefly ("15-operators-attention",
TileLang tutorial, section 5.4: an Ascend example computing dQ, dK and dV
from the forward's saved statistics, with dQ partials accumulated
atomically).  What it computes is the derivative of the forward's definition
(its section 1.1), written out here with every matrix materialised, per
(batch, query head):

    S  = s Q K^T  (masked entries -inf),   P = row-softmax(S),   O = P V
    given dO:
    dV = P^T dO                         (summed over the query heads of a KV head)
    dP = dO V^T
    dS = P * (dP - rowsum(P * dP))      (the softmax Jacobian, row by row)
    dQ = s dS K
    dK = s dS^T Q                       (summed over the query heads of a KV head)

rowsum(P * dP) equals rowsum(dO * O) when O is the exact output.  A row that
sees no key has P = 0 and contributes nothing.  Layout: BHSD, dense; causal
masking bottom-right aligned as in the forward oracle.

With a sliding window W (the tutorial's section 5.2 band, as in the forward
oracle: key j visible to row i iff i + off - W < j <= i + off) only the mask
changes.  With per-head attention sinks (its sections 4.6-4.7: a logit in
the denominator, no value) the row softmax takes one more column, so
P_sink,i = exp(sink - m) / l and the sink's gradient is that column's dS,
dsink_h = sum over rows of P_sink,i (0 - rowsum(P * dP)_i).
"""

from __future__ import annotations

import numpy as np


def _visible(sq: int, skv: int, causal: bool, window: int = 0) -> np.ndarray:
    """[sq, skv] boolean: key j visible to query i."""
    vis = np.ones((sq, skv), dtype=bool)
    i = np.arange(sq)[:, None]
    j = np.arange(skv)[None, :]
    if causal or window > 0:
        vis = j <= i + (skv - sq)
    if window > 0:
        vis = vis & (j > i + (skv - sq) - window)
    return vis


def attention_backward(q, k, v, do, scale: float, causal: bool = False, window: int = 0, sinks=None):
    """dq, dk, dv (fp64) of attention with q [B,H,Sq,d], k/v [B,Hkv,Skv,d]
    and output gradient do [B,H,Sq,d]; with ``sinks`` ([H] logits in the
    units of the scaled scores) also dsinks [H]."""
    q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
    B, H, sq, d = q.shape
    hkv, skv = k.shape[1], k.shape[2]
    group = H // hkv
    vis = _visible(sq, skv, causal, window)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dsinks = np.zeros(H)
    for b in range(B):
        for h in range(H):
            kh = h // group
            s = scale * (q[b, h] @ k[b, kh].T)
            s = np.where(vis, s, -np.inf)
            if sinks is not None:
                # the sink as one more column of the row softmax
                s = np.concatenate([s, np.full((sq, 1), float(sinks[h]))], axis=1)
            m = s.max(axis=1, keepdims=True)
            empty = ~np.isfinite(m)
            m = np.where(empty, 0.0, m)
            p = np.exp(s - m)
            l = p.sum(axis=1, keepdims=True)
            p = np.where(empty, 0.0, p / np.where(empty, 1.0, l))
            if sinks is not None:
                p, p_sink = p[:, :skv], p[:, skv]
            dv[b, kh] += p.T @ do[b, h]
            dp = do[b, h] @ v[b, kh].T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            if sinks is not None:
                dsinks[h] += (p_sink * (0.0 - (p * dp).sum(axis=1))).sum()
            dq[b, h] = scale * (ds @ k[b, kh])
            dk[b, kh] += scale * (ds.T @ q[b, h])
    if sinks is not None:
        return dq, dk, dv, dsinks
    return dq, dk, dv


def delta(o, do):
    """rowsum(dO * O) per row, fp64: [B,H,Sq]."""
    return (np.asarray(o, np.float64) * np.asarray(do, np.float64)).sum(axis=-1)
