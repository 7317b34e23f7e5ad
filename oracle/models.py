"""The pages' companion models, in fp64 (TEST INFRASTRUCTURE ONLY).

* ``online_row`` / ``online_attention``: the online-softmax recurrence of
  "15-operators-attention" (TileLang tutorial) section 2.3, with the
  ``check_inf`` guard of its section 5.1 (1) and the fully-masked-row rule of
  section 5.1 (2).  The same recurrence appears as the three-state update in
  the FlashAttention forward blog post ("TileLang实战"), section 2.3.
* ``split_partials`` / ``split_combine``: split-KV partial results (each
  normalised by its own denominator, with a base-2 log-sum-exp) and their
  combine with weights l_s / sum l, max-subtracted in base 2, from the
  tutorial's section 5.4.
* ``traffic_naive`` / ``traffic_fused``: the element-count traffic model of
  the tutorial's section 1.2 (three passes through HBM) and section 1
  (fused: Q and O once, K and V once per query block).

These follow the pages' steps in their order and notation; they are written
for readability, not speed (pure Python loops for the per-block trace, numpy
for the tensor forms).
"""

from __future__ import annotations

import math

import numpy as np

LOG2E = 1.0 / math.log(2.0)
LN2 = math.log(2.0)


# --------------------------------------------------------------------------
# online softmax recurrence
# --------------------------------------------------------------------------

def online_row(score_blocks, value_blocks):
    """Run the recurrence over one query row.

    ``score_blocks``: list of 1-D sequences of (already scaled) scores; -inf
    marks a masked key.  ``value_blocks``: matching list of [len, dv] arrays.

    Returns ``(o, lse, trace)`` where ``trace`` holds, after each block, the
    running max ``m``, the rescale factor ``alpha`` applied to the old state,
    the running denominator ``ell`` and the unnormalised accumulator ``acc``.
    """
    dv = np.asarray(value_blocks[0]).shape[1]
    m = -math.inf
    ell = 0.0
    acc = np.zeros(dv, dtype=np.float64)
    trace = []
    for s_blk, v_blk in zip(score_blocks, value_blocks):
        s_blk = [float(x) for x in s_blk]
        v_blk = np.asarray(v_blk, dtype=np.float64)
        m_new = max([m] + s_blk)
        # check_inf: with no visible key so far the offset is 0, not -inf
        off = 0.0 if m_new == -math.inf else m_new
        alpha = math.exp(m - off)  # exp(-inf) = 0 on the first visible block
        p = [math.exp(x - off) for x in s_blk]
        ell = alpha * ell + sum(p)
        acc = alpha * acc
        for pj, vj in zip(p, v_blk):
            acc = acc + pj * vj
        m = m_new
        trace.append({"m": m, "alpha": alpha, "ell": ell, "acc": acc.copy()})
    if ell == 0.0:
        return np.zeros(dv), -math.inf, trace
    return acc / ell, m + math.log(ell), trace


def _visible(sq: int, skv: int, causal: bool) -> np.ndarray:
    """Boolean [sq, skv]: key j visible to query i (bottom-right causal)."""
    j = np.arange(skv)[None, :]
    i = np.arange(sq)[:, None]
    if not causal:
        return np.ones((sq, skv), dtype=bool)
    return j <= i + (skv - sq)


def online_attention(q, k, v, scale: float, block_n: int, causal: bool = False):
    """Tiled forward pass for one (batch, head): q [Sq,d], k/v [Skv,d].

    Keys are visited in blocks of ``block_n``; each block updates (m, l, acc)
    as in ``online_row``, written for a whole row block with numpy.
    Returns (o [Sq,d], lse [Sq]) in fp64.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    sq, skv = q.shape[0], k.shape[0]
    vis = _visible(sq, skv, causal)
    m = np.full(sq, -np.inf)
    ell = np.zeros(sq)
    acc = np.zeros((sq, v.shape[1]))
    for j0 in range(0, skv, block_n):
        j1 = min(j0 + block_n, skv)
        s = scale * (q @ k[j0:j1].T)
        s = np.where(vis[:, j0:j1], s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1))
        off = np.where(m_new == -np.inf, 0.0, m_new)           # check_inf
        alpha = np.exp(m - off)
        p = np.exp(s - off[:, None])
        ell = alpha * ell + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ v[j0:j1]
        m = m_new
    empty = ell == 0.0
    o = np.where(empty[:, None], 0.0, acc / np.where(empty, 1.0, ell)[:, None])
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, ell)))
    return o, lse


# --------------------------------------------------------------------------
# split-KV partials and combine
# --------------------------------------------------------------------------

def split_bounds(skv: int, num_splits: int, round_to: int = 1):
    """Contiguous split ranges: ceil(skv / num_splits) keys rounded up to a
    multiple of ``round_to``; trailing splits may be short or empty."""
    chunk = -(-skv // num_splits) if skv else 0
    chunk = -(-chunk // round_to) * round_to
    out = []
    for s in range(num_splits):
        a = min(s * chunk, skv)
        b = min(a + chunk, skv)
        out.append((a, b))
    return out


def split_partials(q, k, v, scale: float, num_splits: int, round_to: int = 1):
    """Per-split partial results for one (batch, head) decode row set.

    q [Sq,d] (no mask), k/v [Skv,d].  For split s over keys [a,b):
    O_s = (1/l_s) sum_j exp(s_j - m_s) v_j  and  glse_s = log2(l_s) + m_s*log2(e)
    (the base-2 log-sum-exp the page's split kernel writes).  An empty split
    has O_s = 0 and glse_s = -inf.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    parts = []
    for a, b in split_bounds(k.shape[0], num_splits, round_to):
        if b <= a:
            parts.append((np.zeros((q.shape[0], v.shape[1])), np.full(q.shape[0], -np.inf)))
            continue
        s = scale * (q @ k[a:b].T)
        m = s.max(axis=1)
        p = np.exp(s - m[:, None])
        ell = p.sum(axis=1)
        o = (p @ v[a:b]) / ell[:, None]
        glse = np.log2(ell) + m * LOG2E
        parts.append((o, glse))
    return parts


def split_combine(parts):
    """Combine split partials: weights 2^(glse_s - glse_tot) with
    glse_tot = log2(sum_s 2^(glse_s - max)) + max, summed in split order.
    Returns (o, lse) with the natural-log LSE."""
    glse = np.stack([g for _, g in parts])           # [S, rows]
    gmax = glse.max(axis=0)
    safe = np.where(gmax == -np.inf, 0.0, gmax)
    tot = np.zeros_like(gmax)
    for g in glse:
        tot = tot + np.exp2(g - safe)
    empty = tot == 0.0
    with np.errstate(divide="ignore"):
        gtot = np.where(empty, -np.inf, np.log2(np.where(empty, 1.0, tot)) + safe)
    o = np.zeros_like(parts[0][0])
    for (o_s, g) in parts:
        w = np.where(empty, 0.0, np.exp2(g - np.where(empty, 0.0, gtot)))
        o = o + w[:, None] * o_s
    return o, gtot * LN2


# --------------------------------------------------------------------------
# HBM traffic model (elements moved per (batch, head))
# --------------------------------------------------------------------------

def traffic_naive(sq: int, skv: int, d: int) -> int:
    """Three passes: S = QK^T reads Q,K writes S; softmax reads S writes P;
    O = PV reads P,V writes O."""
    s_and_p = 4 * sq * skv
    return s_and_p + 2 * sq * d + 2 * skv * d


def traffic_fused(sq: int, skv: int, d: int, block_m: int) -> int:
    """Fused: Q and O once; K and V once per query block."""
    nblocks = -(-sq // block_m)
    return 2 * sq * d + 2 * nblocks * skv * d


def traffic_sp_share(sq: int, skv: int) -> int:
    """Elements of S and P moved by the naive pass structure."""
    return 4 * sq * skv
