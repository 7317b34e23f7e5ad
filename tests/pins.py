"""Pins for the oracle: each function checks the naive fp64 oracle against
something other than itself (values the pages print, closed forms,
invariants, a library routine) and raises AssertionError on a mismatch.

They take the oracle library handle as an argument so that the same checks
can be run against deliberately broken builds of the oracle (see
``test_oracle_mutants.py``): every plausible mistake must trip at least one.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def printed_tol(s: str) -> float:
    """Half a unit in the last printed decimal of the string ``s``."""
    dec = len(s.split(".")[1]) if "." in s else 0
    return 0.5 * 10.0 ** (-dec) + 1e-12


def assert_printed(value: float, printed: str, what: str):
    tol = printed_tol(printed)
    assert abs(value - float(printed)) <= tol, f"{what}: {value!r} vs printed {printed} (tol {tol})"


def rng_tensor(rng, shape):
    return rng.standard_normal(shape).astype(np.float32)


def _example_case(scores, d=64):
    """q = e0, k_j = x_j e0, v_j = e_j, scale 1: row 0 of O is the softmax of
    the scores and LSE is ln(sum exp(x))."""
    n = len(scores)
    q = np.zeros((1, 1, 1, d), np.float32)
    q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, 1, n, d), np.float32)
    k[0, 0, :, 0] = scores
    v = np.zeros((1, 1, n, d), np.float32)
    for j in range(n):
        v[0, 0, j, j] = 1.0
    return q, k, v


# ---------------------------------------------------------------- examples

def pin_four_scores(lib):
    g = golden()["four_scores"]
    scores = [x for b in g["blocks"] for x in b]
    q, k, v = _example_case(scores)
    o, lse = oracle.attention(q, k, v, 1.0, lib=lib)
    for j, w in enumerate(g["weights"]):
        assert_printed(o[0, 0, 0, j], w, f"weight {j}")
    assert np.all(o[0, 0, 0, len(scores):] == 0.0)
    assert_printed(math.exp(lse[0, 0, 0]), g["exp_sum"], "sum of exp")


def pin_three_blocks(lib):
    g = golden()["three_blocks"]
    scores = [x for b in g["blocks"] for x in b]
    q, k, v = _example_case(scores)
    o, lse = oracle.attention(q, k, v, 1.0, lib=lib)
    for j, w in enumerate(g["weights"]):
        assert_printed(o[0, 0, 0, j], w, f"weight {j}")
    # the final denominator relative to the final max is l = sum exp(x - 3)
    assert_printed(math.exp(lse[0, 0, 0] - 3.0), g["ell"][-1], "final l")


# ------------------------------------------------------- library routine

def _sdpa64(q, k, v, scale, causal):
    """torch's CPU scaled_dot_product_attention in float64 (Sq == Skv only,
    where its causal alignment agrees with the bottom-right rule)."""
    H, Hkv = q.shape[1], k.shape[1]
    if H != Hkv:
        k = np.repeat(k, H // Hkv, axis=1)
        v = np.repeat(v, H // Hkv, axis=1)
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), is_causal=causal, scale=scale).numpy()


def pin_sdpa(lib):
    rng = np.random.default_rng(11)
    for (B, H, Hkv, S, d, causal) in [(2, 2, 2, 37, 16, False), (1, 4, 2, 33, 8, True),
                                      (2, 3, 1, 20, 64, True), (1, 2, 2, 65, 128, False)]:
        q = rng_tensor(rng, (B, H, S, d))
        k = rng_tensor(rng, (B, Hkv, S, d))
        v = rng_tensor(rng, (B, Hkv, S, d))
        scale = 1.0 / math.sqrt(d)
        o, _ = oracle.attention(q, k, v, scale, causal, lib=lib)
        ref = _sdpa64(q, k, v, scale, causal)
        err = np.abs(o - ref).max()
        assert err <= 1e-12, f"sdpa mismatch {err} at {(B, H, Hkv, S, d, causal)}"


# ------------------------------------------------------------ closed forms

def pin_closed_forms(lib):
    rng = np.random.default_rng(12)
    d = 16
    # one key: O = v0, LSE = s * q.k0
    q = rng_tensor(rng, (1, 2, 5, d)); k = rng_tensor(rng, (1, 2, 1, d)); v = rng_tensor(rng, (1, 2, 1, d))
    o, lse = oracle.attention(q, k, v, 0.3, lib=lib)
    assert np.abs(o - v.astype(np.float64)).max() <= 1e-15
    want = 0.3 * np.einsum("bhid,bhjd->bhi", q.astype(np.float64), k.astype(np.float64))
    assert np.abs(lse - want).max() <= 1e-12
    # constant scores (q = 0): O = mean(V), LSE = ln n
    n = 7
    q = np.zeros((1, 1, 3, d), np.float32)
    k = rng_tensor(rng, (1, 1, n, d)); v = rng_tensor(rng, (1, 1, n, d))
    o, lse = oracle.attention(q, k, v, 0.25, lib=lib)
    assert np.abs(o - v.astype(np.float64).mean(axis=2, keepdims=True)).max() <= 1e-14
    assert np.abs(lse - math.log(n)).max() <= 1e-14
    # causal, Sq == Skv: row 0 sees key 0 only -> O = v0, LSE = s q0.k0
    q = rng_tensor(rng, (1, 1, 6, d)); k = rng_tensor(rng, (1, 1, 6, d)); v = rng_tensor(rng, (1, 1, 6, d))
    o, lse = oracle.attention(q, k, v, 0.5, causal=True, lib=lib)
    assert np.abs(o[0, 0, 0] - v[0, 0, 0]).max() == 0.0
    assert abs(lse[0, 0, 0] - 0.5 * float(np.dot(q[0, 0, 0].astype(np.float64), k[0, 0, 0].astype(np.float64)))) <= 1e-12
    # causal, last row of Sq == Skv sees every key: equals non-causal row
    o_nc, lse_nc = oracle.attention(q, k, v, 0.5, causal=False, lib=lib)
    assert np.abs(o[0, 0, -1] - o_nc[0, 0, -1]).max() <= 1e-15
    # causal with Sq > Skv: the first Sq - Skv rows see nothing -> O = 0, LSE = -inf
    q = rng_tensor(rng, (1, 1, 9, d)); k = rng_tensor(rng, (1, 1, 4, d)); v = rng_tensor(rng, (1, 1, 4, d))
    o, lse = oracle.attention(q, k, v, 0.5, causal=True, lib=lib)
    assert np.all(o[0, 0, :5] == 0.0) and np.all(np.isneginf(lse[0, 0, :5]))
    assert np.all(np.isfinite(lse[0, 0, 5:]))
    assert np.abs(o[0, 0, 5] - v[0, 0, 0]).max() == 0.0  # row 5 sees key 0 only
    # no keys at all
    o, lse = oracle.attention(q, k[:, :, :0], v[:, :, :0], 0.5, lib=lib)
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))


# -------------------------------------------------------------- invariants

def pin_shift_invariance(lib):
    """Adding c to every score of a row leaves O alone and adds c to LSE.
    Realised exactly with an extra feature: q[..., d] = 1, k[..., d] = c / s."""
    rng = np.random.default_rng(13)
    d = 8
    q = rng_tensor(rng, (1, 2, 10, d)); k = rng_tensor(rng, (1, 2, 12, d)); v = rng_tensor(rng, (1, 2, 12, d))
    s, c = 0.5, 3.0
    o, lse = oracle.attention(q, k, v, s, lib=lib)
    q2 = np.concatenate([q, np.ones((1, 2, 10, 1), np.float32)], axis=-1)
    k2 = np.concatenate([k, np.full((1, 2, 12, 1), c / s, np.float32)], axis=-1)
    v2 = np.concatenate([v, np.zeros((1, 2, 12, 1), np.float32)], axis=-1)
    o2, lse2 = oracle.attention(q2, k2, v2, s, lib=lib)
    assert np.abs(o2[..., :d] - o).max() <= 1e-13
    assert np.abs(lse2 - (lse + c)).max() <= 1e-12


def pin_rows_sum_to_one(lib):
    """V = 1 makes O the row sum of P, which is 1 for every non-empty row."""
    rng = np.random.default_rng(14)
    q = rng_tensor(rng, (2, 2, 9, 16)); k = rng_tensor(rng, (2, 2, 9, 16))
    v = np.ones((2, 2, 9, 16), np.float32)
    for causal in (False, True):
        o, _ = oracle.attention(q, k, v, 0.7, causal=causal, lib=lib)
        assert np.abs(o - 1.0).max() <= 1e-14


def pin_gqa_is_repeated_mha(lib):
    rng = np.random.default_rng(15)
    q = rng_tensor(rng, (2, 6, 11, 8)); k = rng_tensor(rng, (2, 2, 13, 8)); v = rng_tensor(rng, (2, 2, 13, 8))
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, 0.4, causal, lib=lib)
        o2, lse2 = oracle.attention(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), 0.4, causal, lib=lib)
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def pin_causal_is_prefix(lib):
    """Causal row i equals non-causal attention over keys [0, i + Skv - Sq]."""
    rng = np.random.default_rng(16)
    sq, skv, d = 5, 9, 8
    q = rng_tensor(rng, (1, 1, sq, d)); k = rng_tensor(rng, (1, 1, skv, d)); v = rng_tensor(rng, (1, 1, skv, d))
    o, lse = oracle.attention(q, k, v, 0.6, causal=True, lib=lib)
    for i in range(sq):
        n = i + (skv - sq) + 1
        oi, li = oracle.attention(q[:, :, i:i + 1], k[:, :, :n], v[:, :, :n], 0.6, lib=lib)
        assert np.array_equal(o[0, 0, i], oi[0, 0, 0]) and lse[0, 0, i] == li[0, 0, 0]


def pin_varlen_is_dense(lib):
    rng = np.random.default_rng(17)
    lens = [5, 0, 1, 12, 7]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, Hkv, d = int(cu[-1]), 4, 2, 8
    q = rng_tensor(rng, (H, T, d)); k = rng_tensor(rng, (Hkv, T, d)); v = rng_tensor(rng, (Hkv, T, d))
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, 0.3, causal, cu_seqlens=cu, lib=lib)
        for b, L in enumerate(lens):
            a = int(cu[b])
            if L == 0:
                continue
            ob, lb = oracle.attention(q[None, :, a:a + L], k[None, :, a:a + L], v[None, :, a:a + L], 0.3,
                                      causal, lib=lib)
            assert np.array_equal(o[:, a:a + L], ob[0]) and np.array_equal(lse[:, a:a + L], lb[0])


def pin_row_subset(lib):
    rng = np.random.default_rng(18)
    q = rng_tensor(rng, (2, 2, 7, 8)); k = rng_tensor(rng, (2, 1, 9, 8)); v = rng_tensor(rng, (2, 1, 9, 8))
    o, lse = oracle.attention(q, k, v, 0.5, True, lib=lib)
    rows = np.array([[1, 0, 6], [0, 1, 0], [1, 1, 3]])
    orow, lrow = oracle.attention(q, k, v, 0.5, True, rows=rows, lib=lib)
    for r, (b, h, i) in enumerate(rows):
        assert np.array_equal(orow[r], o[b, h, i]) and lrow[r] == lse[b, h, i]


# ----------------------------------------------------- sliding window, sinks

def pin_window_is_key_slice(lib):
    """With a window W, row i equals unmasked attention over the keys
    (i + off - W, i + off], off = Skv - Sq (the tutorial's section 5.2 band,
    bottom-right aligned); rows with no key in the band are empty."""
    rng = np.random.default_rng(19)
    for sq, skv, w in [(9, 9, 3), (5, 12, 4), (12, 7, 2), (6, 6, 1)]:
        q = rng_tensor(rng, (1, 2, sq, 8)); k = rng_tensor(rng, (1, 2, skv, 8)); v = rng_tensor(rng, (1, 2, skv, 8))
        o, lse = oracle.attention(q, k, v, 0.6, True, window=w, lib=lib)
        off = skv - sq
        for i in range(sq):
            lo, hi = max(0, i + off - w + 1), min(skv, i + off + 1)
            if hi <= lo:
                assert np.all(o[0, :, i] == 0.0) and np.all(np.isneginf(lse[0, :, i]))
                continue
            oi, li = oracle.attention(q[:, :, i:i + 1], k[:, :, lo:hi], v[:, :, lo:hi], 0.6, lib=lib)
            assert np.array_equal(o[0, :, i], oi[0, :, 0]) and np.array_equal(lse[0, :, i], li[0, :, 0])


def pin_window_limits(lib):
    """Window 1 keeps only the diagonal key (O = v, LSE = s q.k); a window at
    least Skv long is plain causal attention."""
    rng = np.random.default_rng(20)
    q = rng_tensor(rng, (2, 2, 7, 8)); k = rng_tensor(rng, (2, 2, 10, 8)); v = rng_tensor(rng, (2, 2, 10, 8))
    o, lse = oracle.attention(q, k, v, 0.5, True, window=1, lib=lib)
    for i in range(7):
        j = i + 3
        assert np.array_equal(o[:, :, i], v[:, :, j].astype(np.float64))
        want = 0.5 * np.einsum("bhd,bhd->bh", q[:, :, i].astype(np.float64), k[:, :, j].astype(np.float64))
        assert np.abs(lse[:, :, i] - want).max() <= 1e-12
    oc, lc = oracle.attention(q, k, v, 0.5, True, lib=lib)
    ow, lw = oracle.attention(q, k, v, 0.5, True, window=10, lib=lib)
    assert np.array_equal(oc, ow) and np.array_equal(lc, lw)
    # a window implies the causal bound (the band ends at the diagonal)
    on, ln = oracle.attention(q, k, v, 0.5, False, window=10, lib=lib)
    assert np.array_equal(oc, on) and np.array_equal(lc, ln)


def pin_sink_is_extra_key(lib):
    """A sink is a key that every row sees, whose score is the sink and whose
    value is zero: realised with an extra feature (q[.., d] = 1, key 0 =
    (0, .., 0, sink), value 0) at scale 1, where the products are exact."""
    rng = np.random.default_rng(21)
    B, H, sq, skv, d = 2, 3, 6, 9, 8
    q = rng_tensor(rng, (B, H, sq, d)); k = rng_tensor(rng, (B, H, skv, d)); v = rng_tensor(rng, (B, H, skv, d))
    sinks = np.array([0.75, -2.5, 4.0])
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, 1.0, causal, sinks=sinks, lib=lib)
        q2 = np.concatenate([q, np.ones((B, H, sq, 1), np.float32)], axis=-1)
        k2 = np.zeros((B, H, skv + 1, d + 1), np.float32)
        k2[:, :, 1:, :d] = k
        k2[:, :, 0, d] = sinks[None, :].astype(np.float32)
        v2 = np.zeros((B, H, skv + 1, d + 1), np.float32)
        v2[:, :, 1:, :d] = v
        o2, lse2 = oracle.attention(q2, k2, v2, 1.0, causal, lib=lib)
        assert np.abs(o2[..., :d] - o).max() <= 1e-13 and np.abs(lse2 - lse).max() <= 1e-12


def pin_sink_splits_the_normaliser(lib):
    """With or without a window, the sink only adds exp(sink) to the
    normaliser: LSE' = logaddexp(LSE, sink) and O' = O exp(LSE - LSE'); a
    row with no key gets O' = 0, LSE' = sink; sink = -inf changes nothing;
    a sink far above every score stays finite (the max-with-sink guard)."""
    rng = np.random.default_rng(22)
    q = rng_tensor(rng, (1, 2, 10, 8)); k = rng_tensor(rng, (1, 2, 6, 8)); v = rng_tensor(rng, (1, 2, 6, 8))
    for window in (0, 3):
        o, lse = oracle.attention(q, k, v, 0.5, True, window=window, lib=lib)
        for sk in ([0.3, -1.0], [800.0, 900.0]):
            sinks = np.array(sk)
            o2, lse2 = oracle.attention(q, k, v, 0.5, True, window=window, sinks=sinks, lib=lib)
            assert np.all(np.isfinite(o2)) and np.all(np.isfinite(lse2))
            want = np.logaddexp(lse, sinks[None, :, None])
            assert np.abs(lse2 - want).max() <= 1e-12
            with np.errstate(invalid="ignore"):  # rows without keys: -inf - -inf, masked by the where
                scale = np.where(np.isneginf(lse), 0.0, np.exp(lse - want))
                assert np.abs(o2 - o * scale[..., None]).max() <= 1e-13
        o3, lse3 = oracle.attention(q, k, v, 0.5, True, window=window, sinks=np.array([-np.inf, -np.inf]),
                                    lib=lib)
        assert np.array_equal(o3, o) and np.array_equal(lse3, lse)


ALL_PINS = [pin_four_scores, pin_three_blocks, pin_sdpa, pin_closed_forms, pin_shift_invariance,
            pin_rows_sum_to_one, pin_gqa_is_repeated_mha, pin_causal_is_prefix, pin_varlen_is_dense,
            pin_row_subset, pin_window_is_key_slice, pin_window_limits, pin_sink_is_extra_key,
            pin_sink_splits_the_normaliser]
