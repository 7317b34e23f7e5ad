"""Pins for the backward oracle (``oracle/backward.py``), on the CPU.

* Central finite differences of the pinned forward oracle (``attn_ref.c``):
  with L = sum(O * dO), dL/dq, dL/dk, dL/dv must equal dq, dk, dv.  Inputs
  are multiples of 2^-6 and the step is 2^-12, so every perturbed input is
  exact in the forward's fp32 input format.
* torch's float64 CPU autograd through a masked-softmax attention.
* Closed forms and invariants: one visible key gives dq = dk = 0 and
  dv = sum of dO; every row of dS sums to zero, so dK summed over the keys is
  zero; grouped-query gradients are the per-head gradients summed over the
  group; rowsum(dO * O) is rowsum(P * dP).

* Window and sinks: finite differences of the forward oracle with a window
  and sinks (q, k, v and the sink logits); torch float64 autograd through a
  banded softmax with a sink column; a sink built exactly as one more key
  (score = sink through an extra feature, value 0) whose dK is scale * dsink;
  a window covering every key is plain causal; a sink of -inf is no sink.

Plausible mistakes planted in copies of the backward oracle (sign of the
softmax-Jacobian term, a dropped scale, dV from dP, the row-sum term left
out, a GQA head mapped by modulo, dK from dQ's operand, the window band off
by one or ignored, the sink gradient's sign or its P factor, the sink left
out of the softmax) each trip at least one pin.
"""

import math
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import backward


def dyadic(rng, shape):
    return (rng.integers(-128, 129, size=shape) / 64.0).astype(np.float32)


def fd_pin(bwd):
    rng = np.random.default_rng(31)
    for causal, (sq, skv) in ((False, (4, 6)), (True, (5, 5)), (True, (3, 6))):
        B, H, Hkv, d = 1, 2, 1, 4
        q, k, v, do = (dyadic(rng, s) for s in ((B, H, sq, d), (B, Hkv, skv, d), (B, Hkv, skv, d), (B, H, sq, d)))
        scale = 0.5
        dq, dk, dv = bwd(q, k, v, do, scale, causal)
        eps = 2.0 ** -12

        def loss(qq, kk, vv):
            o, _ = oracle.attention(qq, kk, vv, scale, causal)
            return float((o * do.astype(np.float64)).sum())

        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros(x.shape)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = [q, k, v]
                args_m = [q, k, v]
                pos = "qkv".index(name)
                args_p[pos], args_m[pos] = xp, xm
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            err = np.abs(num - g).max()
            assert err <= 1e-6 * max(1.0, np.abs(g).max()), f"d{name} vs finite differences: {err:.3g}"


def torch_pin(bwd):
    rng = np.random.default_rng(32)
    for causal, (B, H, Hkv, sq, skv, d) in ((False, (2, 4, 2, 7, 9, 8)), (True, (1, 3, 1, 9, 6, 16)),
                                             (True, (1, 2, 2, 8, 8, 8))):
        q, k, v, do = (rng.standard_normal(s).astype(np.float32) for s in
                       ((B, H, sq, d), (B, Hkv, skv, d), (B, Hkv, skv, d), (B, H, sq, d)))
        scale = 1.0 / math.sqrt(d)
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        g = H // Hkv
        kk, vv = tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1)
        s = scale * torch.matmul(tq, kk.transpose(-1, -2))
        if causal:
            i = torch.arange(sq)[:, None]
            j = torch.arange(skv)[None, :]
            s = s.masked_fill(j > i + (skv - sq), float("-inf"))
        p = torch.softmax(s, dim=-1)
        p = torch.nan_to_num(p, nan=0.0)
        o = torch.matmul(p, vv)
        (o * torch.tensor(do, dtype=torch.float64)).sum().backward()
        dq, dk, dv = bwd(q, k, v, do, scale, causal)
        for name, a, b in (("q", dq, tq.grad), ("k", dk, tk.grad), ("v", dv, tv.grad)):
            err = np.abs(a - b.numpy()).max()
            assert err <= 1e-12, f"d{name} vs torch autograd: {err:.3g}"


def closed_form_pin(bwd):
    rng = np.random.default_rng(33)
    q, do = rng.standard_normal((2, 2, 5, 8)), rng.standard_normal((2, 2, 5, 8))
    k, v = rng.standard_normal((2, 1, 1, 8)), rng.standard_normal((2, 1, 1, 8))
    dq, dk, dv = bwd(q, k, v, do, 0.3, False)
    assert np.abs(dq).max() <= 1e-15 and np.abs(dk).max() <= 1e-15
    assert np.abs(dv[:, 0, 0] - do.sum(axis=(1, 2))).max() <= 1e-12


def invariant_pin(bwd):
    rng = np.random.default_rng(34)
    for causal in (False, True):
        q, do = rng.standard_normal((1, 4, 9, 8)), rng.standard_normal((1, 4, 9, 8))
        k, v = rng.standard_normal((1, 2, 11, 8)), rng.standard_normal((1, 2, 11, 8))
        dq, dk, dv = bwd(q, k, v, do, 0.4, causal)
        assert np.abs(dk.sum(axis=2)).max() <= 1e-12, "dK does not sum to zero over the keys"
        # grouped-query = per-head (repeated K/V) gradients summed over the group
        dq2, dk2, dv2 = bwd(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), do, 0.4, causal)
        assert np.abs(dq - dq2).max() <= 1e-12
        assert np.abs(dk - dk2.reshape(1, 2, 2, 11, 8).sum(axis=2)).max() <= 1e-12
        assert np.abs(dv - dv2.reshape(1, 2, 2, 11, 8).sum(axis=2)).max() <= 1e-12


def fd_window_sink_pin(bwd):
    """Central finite differences of the forward oracle with a window and
    sinks, for q, k, v and the sink logits."""
    rng = np.random.default_rng(36)
    for window, with_sinks, (sq, skv) in ((3, True, (6, 6)), (2, False, (4, 7)), (0, True, (5, 5))):
        B, H, Hkv, d = 1, 2, 1, 4
        q, k, v, do = (dyadic(rng, s) for s in ((B, H, sq, d), (B, Hkv, skv, d), (B, Hkv, skv, d), (B, H, sq, d)))
        sinks = (rng.integers(-64, 65, size=H) / 32.0).astype(np.float32) if with_sinks else None
        scale = 0.5
        out = bwd(q, k, v, do, scale, True, window=window, sinks=sinks)
        eps = 2.0 ** -12

        def loss(qq, kk, vv, ss):
            o, _ = oracle.attention(qq, kk, vv, scale, True, window=window, sinks=ss)
            return float((o * do.astype(np.float64)).sum())

        wrt = [("q", 0, q), ("k", 1, k), ("v", 2, v)] + ([("sinks", 3, sinks)] if with_sinks else [])
        for name, pos, x in wrt:
            g = out[pos]
            num = np.zeros(x.shape)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = [q, k, v, sinks]
                args_m = [q, k, v, sinks]
                args_p[pos], args_m[pos] = xp, xm
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            err = np.abs(num - g).max()
            assert err <= 1e-6 * max(1.0, np.abs(g).max()), f"d{name} (window {window}) vs finite differences: {err:.3g}"


def torch_window_sink_pin(bwd):
    """torch float64 autograd through a banded softmax with a sink column."""
    rng = np.random.default_rng(37)
    for causal, window, (B, H, Hkv, sq, skv, d) in ((True, 3, (1, 4, 2, 9, 11, 8)), (True, 0, (2, 2, 1, 7, 7, 16))):
        q, k, v, do = (rng.standard_normal(s).astype(np.float32) for s in
                       ((B, H, sq, d), (B, Hkv, skv, d), (B, Hkv, skv, d), (B, H, sq, d)))
        sinks = rng.standard_normal(H).astype(np.float32) * 2
        scale = 1.0 / math.sqrt(d)
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        ts = torch.tensor(sinks, dtype=torch.float64, requires_grad=True)
        g = H // Hkv
        kk, vv = tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1)
        s = scale * torch.matmul(tq, kk.transpose(-1, -2))
        i = torch.arange(sq)[:, None]
        j = torch.arange(skv)[None, :]
        vis = j <= i + (skv - sq)
        if window > 0:
            vis = vis & (j > i + (skv - sq) - window)
        s = s.masked_fill(~vis, float("-inf"))
        col = ts[None, :, None, None].expand(B, H, sq, 1)
        p = torch.softmax(torch.cat([s, col], dim=-1), dim=-1)[..., :skv]
        o = torch.matmul(p, vv)
        (o * torch.tensor(do, dtype=torch.float64)).sum().backward()
        dq, dk, dv, dsinks = bwd(q, k, v, do, scale, causal, window=window, sinks=sinks)
        for name, a, b in (("q", dq, tq.grad), ("k", dk, tk.grad), ("v", dv, tv.grad), ("sinks", dsinks, ts.grad)):
            err = np.abs(a - b.numpy()).max()
            assert err <= 1e-12, f"d{name} vs torch autograd (window {window}): {err:.3g}"


def sink_as_key_pin(bwd):
    """A sink is a key whose score is the sink and whose value is 0: built
    exactly with one more feature (q_i = 1 there, the extra key sink/scale,
    every other key 0) and the extra key placed first (so that bottom-right
    causal masking keeps the original keys' visibility), its dK in that
    feature is scale * dsink, and the other gradients are the same."""
    rng = np.random.default_rng(38)
    for causal in (False, True):
        B, H, Hkv, sq, skv, d = 1, 2, 2, 5, 6, 4
        q, k, v, do = (dyadic(rng, s) for s in ((B, H, sq, d), (B, Hkv, skv, d), (B, Hkv, skv, d), (B, H, sq, d)))
        sinks = np.array([0.75, -1.5])
        scale = 0.5
        dq, dk, dv, dsinks = bwd(q, k, v, do, scale, causal, sinks=sinks)
        dq2, dk2, dv2 = [], [], []
        for h in range(H):
            qe = np.concatenate([q[:, [h]], np.ones((B, 1, sq, 1))], axis=-1)
            ke = np.zeros((B, 1, skv + 1, d + 1))
            ke[:, :, 1:, :d] = k[:, [h]]
            ke[:, :, 0, d] = sinks[h] / scale
            ve = np.zeros((B, 1, skv + 1, d))
            ve[:, :, 1:] = v[:, [h]]
            gq, gk, gv = bwd(qe, ke, ve, do[:, [h]], scale, causal)
            assert abs(gk[0, 0, 0, d] / scale - dsinks[h]) <= 1e-12, "dsink differs from the extra key's gradient"
            dq2.append(gq[..., :d])
            dk2.append(gk[:, :, 1:, :d])
            dv2.append(gv[:, :, 1:])
        assert np.abs(dq - np.concatenate(dq2, axis=1)).max() <= 1e-12
        assert np.abs(dk - np.concatenate(dk2, axis=1)).max() <= 1e-12
        assert np.abs(dv - np.concatenate(dv2, axis=1)).max() <= 1e-12


def window_invariant_pin(bwd):
    """A window at least as long as the keys is plain causal; a sink of -inf
    is no sink (and gets no gradient)."""
    rng = np.random.default_rng(39)
    q, do = rng.standard_normal((1, 2, 6, 8)), rng.standard_normal((1, 2, 6, 8))
    k, v = rng.standard_normal((1, 1, 9, 8)), rng.standard_normal((1, 1, 9, 8))
    a = bwd(q, k, v, do, 0.4, True)
    b = bwd(q, k, v, do, 0.4, True, window=9)
    for x, y in zip(a, b):
        assert np.abs(x - y).max() <= 1e-12
    c = bwd(q, k, v, do, 0.4, True, window=4, sinks=np.array([-np.inf, -np.inf]))
    w = bwd(q, k, v, do, 0.4, True, window=4)
    for x, y in zip(c[:3], w):
        assert np.abs(x - y).max() <= 1e-12
    assert np.all(c[3] == 0.0)


PINS = [fd_pin, torch_pin, closed_form_pin, invariant_pin, fd_window_sink_pin, torch_window_sink_pin,
        sink_as_key_pin, window_invariant_pin]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_backward_oracle_pin(pin):
    pin(backward.attention_backward)


def test_delta_is_rowsum_p_dp():
    rng = np.random.default_rng(35)
    q, do = rng.standard_normal((1, 2, 6, 8)), rng.standard_normal((1, 2, 6, 8))
    k, v = rng.standard_normal((1, 2, 7, 8)), rng.standard_normal((1, 2, 7, 8))
    o, _ = oracle.attention(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), 0.5, False)
    qf, kf, vf = (x.astype(np.float32).astype(np.float64) for x in (q, k, v))
    s = 0.5 * np.einsum("bhid,bhjd->bhij", qf, kf)
    p = np.exp(s - s.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    dp = np.einsum("bhid,bhjd->bhij", do, vf)
    assert np.abs(backward.delta(o, do) - (p * dp).sum(-1)).max() <= 1e-12


MUTANTS = {
    "jacobian_sign": ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))",
                      "ds = p * (dp + (p * dp).sum(axis=1, keepdims=True))"),
    "rowsum_dropped": ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "ds = p * dp"),
    "dq_no_scale": ("dq[b, h] = scale * (ds @ k[b, kh])", "dq[b, h] = ds @ k[b, kh]"),
    "dk_no_scale": ("dk[b, kh] += scale * (ds.T @ q[b, h])", "dk[b, kh] += ds.T @ q[b, h]"),
    "dv_from_dp": ("dv[b, kh] += p.T @ do[b, h]", "dv[b, kh] += (do[b, h] @ v[b, kh].T).T @ do[b, h]"),
    "gqa_modulo": ("kh = h // group", "kh = h % hkv"),
    "dk_uses_k": ("dk[b, kh] += scale * (ds.T @ q[b, h])", "dk[b, kh] += scale * (ds.T @ k[b, kh][:sq])"),
    "causal_top_left": ("vis = j <= i + (skv - sq)", "vis = j <= i"),
    "window_off_by_one": ("vis = vis & (j > i + (skv - sq) - window)", "vis = vis & (j >= i + (skv - sq) - window)"),
    "window_ignored": ("vis = vis & (j > i + (skv - sq) - window)", "vis = vis"),
    "sink_grad_sign": ("dsinks[h] += (p_sink * (0.0 - (p * dp).sum(axis=1))).sum()",
                       "dsinks[h] += (p_sink * (p * dp).sum(axis=1)).sum()"),
    "sink_grad_no_p": ("dsinks[h] += (p_sink * (0.0 - (p * dp).sum(axis=1))).sum()",
                       "dsinks[h] += (0.0 - (p * dp).sum(axis=1)).sum()"),
    "sink_not_in_softmax": ("s = np.concatenate([s, np.full((sq, 1), float(sinks[h]))], axis=1)",
                            "s = np.concatenate([s, np.full((sq, 1), -np.inf)], axis=1)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_backward_mutant(name):
    src = open(backward.__file__).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType(f"bwd_{name}")
    exec(compile(src.replace(old, new), f"bwd_{name}", "exec"), mod.__dict__)
    caught = []
    for pin in PINS:
        try:
            pin(mod.attention_backward)
        except (AssertionError, ValueError, IndexError, TypeError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches backward mutant {name}"
