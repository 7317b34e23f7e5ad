"""Randomized parity sweep: configurations drawn once from a fixed seed
(layout, batch or packed sequences with empty ones among them, heads and
grouped-query ratio, ragged Sq and Skv, head dim, causal, window, sinks,
decode), forward and backward, each against the fp64 oracles.

The named tests elsewhere pin each feature on chosen shapes; this sweep
mixes them the way a caller would, so that an index or bound that only
breaks in a combination (a window with Sq < Skv in the BSHD layout, sinks on
a packing with an empty sequence, ...) is caught.  The forward bar is the
bf16 rounding bound of check() (few-key rows included), the backward bar
compare_grads()'s.  Sizes keep the oracle to a fraction of a second each.
"""

import math

import numpy as np
import pytest

from exact_attention_09_amd import synth
from exact_attention_09_amd.workloads import host_f32, to_device
from oracle import backward as bwd_oracle
from parity import check, compare_grads, reference, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def draw(rng, backward: bool):
    """One configuration: a dict of the call's options and shapes."""
    layout = "bshd" if rng.random() < 0.5 else "bhsd"
    d = 64 if rng.random() < 0.4 else 128
    H = int(rng.choice([1, 2, 4, 6, 8]))
    Hkv = int(rng.choice([x for x in (1, 2, 3, 4, 6, 8) if H % x == 0]))
    causal = bool(rng.random() < 0.6)
    window = int(rng.integers(1, 300)) if causal and rng.random() < 0.35 else 0
    sinks = bool(causal and rng.random() < 0.35)
    if rng.random() < 0.3:
        nseq = int(rng.integers(1, 6))
        lengths = [int(x) if rng.random() > 0.15 else 0 for x in rng.integers(1, 400, nseq)]
        if sum(lengths) == 0:
            lengths[0] = int(rng.integers(1, 300))
        return dict(layout=layout, d=d, H=H, Hkv=Hkv, causal=causal, window=window, sinks=sinks,
                    lengths=tuple(lengths), B=len(lengths), Sq=sum(lengths), Skv=sum(lengths))
    B = int(rng.integers(1, 4))
    Skv = int(rng.integers(1, 600))
    if not backward and rng.random() < 0.2:
        Sq = 1                                   # decode: the split-KV path
    else:
        Sq = int(rng.integers(1, 400))
    return dict(layout=layout, d=d, H=H, Hkv=Hkv, causal=causal, window=window, sinks=sinks, lengths=None,
                B=B, Sq=Sq, Skv=Skv)


_RNG = np.random.default_rng(20261202)
FORWARD = [draw(_RNG, False) for _ in range(28)]
BACKWARD = [draw(_RNG, True) for _ in range(16)]


def name_of(c):
    parts = [c["layout"], f"d{c['d']}", f"H{c['H']}/{c['Hkv']}"]
    parts.append(f"seqs{'-'.join(map(str, c['lengths']))}" if c["lengths"] else f"B{c['B']}-{c['Sq']}x{c['Skv']}")
    parts += ["causal" if c["causal"] else "full"] + ([f"w{c['window']}"] if c["window"] else [])
    return "_".join(parts + (["sinks"] if c["sinks"] else []))


def inputs(c, seed):
    """BHSD host arrays (bf16 bits) q, k, v, do, the sinks, the device tensors
    in the case's layout, and cu_seqlens (host and device)."""
    H, Hkv, d = c["H"], c["Hkv"], c["d"]
    if c["lengths"]:
        T = c["Sq"]
        qs, ks = (1, H, T, d), (1, Hkv, T, d)
        cu = np.concatenate([[0], np.cumsum(c["lengths"])]).astype(np.int32)
    else:
        qs, ks = (c["B"], H, c["Sq"], d), (c["B"], Hkv, c["Skv"], d)
        cu = None
    q = synth.normal_tensor(seed + 0, qs, "bf16")
    k = synth.normal_tensor(seed + 1, ks, "bf16")
    v = synth.normal_tensor(seed + 2, ks, "bf16")
    do = synth.normal_tensor(seed + 3, qs, "bf16")
    sk = (synth.normal_tensor(seed + 5, (H,), "f32") * np.float32(2.0)).astype(np.float32) if c["sinks"] else None

    def dev(x):
        t = to_device(x, "bf16")
        if c["layout"] == "bhsd":
            return t
        return t[0].transpose(0, 1).contiguous() if cu is not None else t.transpose(1, 2).contiguous()

    devs = tuple(dev(x) for x in (q, k, v, do))
    cut = torch.from_numpy(cu).cuda() if cu is not None else None
    skt = torch.from_numpy(sk).cuda() if sk is not None else None
    return (q, k, v, do), sk, devs, cu, cut, skt


def to_bhsd(t, c):
    """A device tensor of the case's layout back to a BHSD fp64 host array."""
    if c["layout"] == "bshd":
        t = t.transpose(0, 1).unsqueeze(0) if c["lengths"] else t.transpose(1, 2)
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("c", FORWARD, ids=name_of)
def test_random_forward(c):
    import exact_attention_09_amd as ea
    say(f"random forward {name_of(c)}")
    seed = 10 * (FORWARD.index(c) + 7000)
    (q, k, v, _), sk, (qt, kt, vt, _), cu, cut, skt = inputs(c, seed)
    o, lse = ea.attn_fwd_layout(qt, kt, vt, layout=c["layout"], causal=c["causal"], window=c["window"], sinks=skt,
                                cu_seqlens=cut)
    torch.cuda.synchronize()
    og = to_bhsd(o, c)
    lg = lse.cpu().numpy().astype(np.float64).reshape(og.shape[:-1])
    o_ref, lse_ref, a_ref = reference(*(host_f32(x, "bf16") for x in (q, k, v)), 1.0 / math.sqrt(c["d"]),
                                      c["causal"], cu_seqlens=cu, window=c["window"], sinks=sk)
    check(og, lg, o_ref, lse_ref, "bf16", f"random {name_of(c)}", a_ref=a_ref)


@pytest.mark.parametrize("c", BACKWARD, ids=name_of)
def test_random_backward(c):
    import exact_attention_09_amd as ea
    say(f"random backward {name_of(c)}")
    seed = 10 * (BACKWARD.index(c) + 8000)
    (q, k, v, do), sk, (qt, kt, vt, dot), cu, cut, skt = inputs(c, seed)
    o, lse = ea.attn_fwd_layout(qt, kt, vt, layout=c["layout"], causal=c["causal"], window=c["window"], sinks=skt,
                                cu_seqlens=cut)
    dq, dk, dv, ds = ea.attn_bwd_layout(qt, kt, vt, o, lse, dot, layout=c["layout"], causal=c["causal"],
                                        window=c["window"], sinks=skt, cu_seqlens=cut)
    torch.cuda.synchronize()
    got = tuple(to_bhsd(t, c) for t in (dq, dk, dv))
    hq, hk, hv, hdo = (host_f32(x, "bf16") for x in (q, k, v, do))
    scale = 1.0 / math.sqrt(c["d"])
    if cu is None:
        want = bwd_oracle.attention_backward(hq, hk, hv, hdo, scale, c["causal"], window=c["window"], sinks=sk)
        compare_grads(got, want[:3], f"random {name_of(c)}")
    else:
        for i in range(len(c["lengths"])):
            a, e = int(cu[i]), int(cu[i + 1])
            if e == a:
                continue
            sl = slice(a, e)
            want = bwd_oracle.attention_backward(hq[:, :, sl], hk[:, :, sl], hv[:, :, sl], hdo[:, :, sl], scale,
                                                 c["causal"], window=c["window"], sinks=sk)
            compare_grads(tuple(g[:, :, sl] for g in got), want[:3], f"random {name_of(c)} sequence {i}")
    if sk is not None:
        # dsink_h = -sum over the rows of head h of P_sink Delta: against the
        # fp64 forward oracle's P_sink and Delta, within 1e-2 of the sum of
        # the terms' magnitudes (the terms may cancel)
        import oracle
        o_ref, lse_ref = oracle.attention(hq, hk, hv, scale, True, cu_seqlens=cu, window=c["window"], sinks=sk)
        terms = np.exp(sk.astype(np.float64)[None, :, None] - lse_ref) * (o_ref * hdo.astype(np.float64)).sum(-1)
        want_ds = -terms.sum(axis=(0, 2))
        mag = np.abs(terms).sum(axis=(0, 2))
        err = np.abs(ds.cpu().numpy().astype(np.float64) - want_ds)
        say(f"  random {name_of(c)}: dsinks max|err| {err.max():.3g} (terms up to {mag.max():.3g})")
        assert np.all(err <= 1e-2 * mag + 1e-6), f"dsinks error {err.max():.3g}"
