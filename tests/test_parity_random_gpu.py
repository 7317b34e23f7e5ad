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


# ---- fp32 forward (BHSD, no window or sinks: the fp32 path's scope), 1e-5 bar

def draw_f32(rng):
    d = 64 if rng.random() < 0.5 else 128
    H = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([x for x in (1, 2, 4, 8) if H % x == 0]))
    causal = bool(rng.random() < 0.5)
    if rng.random() < 0.3:
        lengths = tuple(int(x) if rng.random() > 0.15 else 0 for x in rng.integers(1, 300, int(rng.integers(1, 5))))
        if sum(lengths) == 0:
            lengths = (int(rng.integers(1, 200)),) + lengths[1:]
        return dict(d=d, H=H, Hkv=Hkv, causal=causal, lengths=lengths, B=len(lengths), Sq=sum(lengths),
                    Skv=sum(lengths))
    B = int(rng.integers(1, 3))
    Sq = 1 if rng.random() < 0.25 else int(rng.integers(1, 300))
    return dict(d=d, H=H, Hkv=Hkv, causal=causal, lengths=None, B=B, Sq=Sq, Skv=int(rng.integers(1, 400)))


F32 = [draw_f32(_RNG) for _ in range(10)]


def name_f32(c):
    shape = f"seqs{'-'.join(map(str, c['lengths']))}" if c["lengths"] else f"B{c['B']}-{c['Sq']}x{c['Skv']}"
    return f"f32_d{c['d']}_H{c['H']}/{c['Hkv']}_{shape}_{'causal' if c['causal'] else 'full'}"


@pytest.mark.parametrize("c", F32, ids=name_f32)
def test_random_forward_f32(c):
    import exact_attention_09_amd as ea
    say(f"random fp32 forward {name_f32(c)}")
    seed = 10 * (F32.index(c) + 9000)
    H, Hkv, d = c["H"], c["Hkv"], c["d"]
    if c["lengths"]:
        qs, ks = (1, H, c["Sq"], d), (1, Hkv, c["Sq"], d)
        cu = np.concatenate([[0], np.cumsum(c["lengths"])]).astype(np.int32)
    else:
        qs, ks = (c["B"], H, c["Sq"], d), (c["B"], Hkv, c["Skv"], d)
        cu = None
    q, k, v = (synth.normal_tensor(seed + i, s, "f32") for i, s in enumerate((qs, ks, ks)))
    cut = torch.from_numpy(cu).cuda() if cu is not None else None
    o, lse = ea.attn_fwd_f32(*(to_device(x, "f32") for x in (q, k, v)), causal=c["causal"], cu_seqlens=cut)
    torch.cuda.synchronize()
    o_ref, lse_ref, _ = reference(q, k, v, 1.0 / math.sqrt(d), c["causal"], cu_seqlens=cu)
    check(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "f32", f"random {name_f32(c)}")


# ---- paged split-KV decode: random page sizes, key counts and scattered pages

def draw_paged(rng):
    d = 64 if rng.random() < 0.4 else 128
    H = int(rng.choice([1, 4, 8, 16]))
    Hkv = int(rng.choice([x for x in (1, 2, 4, 8) if H % x == 0]))
    page = int(rng.choice([16, 32, 64, 128, 256]))
    B = int(rng.integers(1, 5))
    max_pages = int(rng.integers(1, 12))
    seqlens = [int(rng.integers(0, max_pages * page + 1)) for _ in range(B)]
    splits = int(rng.choice([0, 1, 3, 16]))
    return dict(d=d, H=H, Hkv=Hkv, page=page, B=B, max_pages=max_pages, seqlens=tuple(seqlens), splits=splits)


PAGED = [draw_paged(_RNG) for _ in range(10)]


def name_paged(c):
    return (f"paged_d{c['d']}_H{c['H']}/{c['Hkv']}_p{c['page']}_x{c['max_pages']}_lens"
            f"{'-'.join(map(str, c['seqlens']))}_s{c['splits']}")


@pytest.mark.parametrize("c", PAGED, ids=name_paged)
def test_random_paged_decode(c):
    import exact_attention_09_amd as ea
    from oracle import paged as paged_oracle
    say(f"random paged decode {name_paged(c)}")
    seed = 10 * (PAGED.index(c) + 9500)
    rng = np.random.default_rng(seed)
    B, H, Hkv, d, page, mp = c["B"], c["H"], c["Hkv"], c["d"], c["page"], c["max_pages"]
    num_pages = B * mp + 3                                  # a few pages no sequence uses
    table = rng.permutation(num_pages)[:B * mp].reshape(B, mp).astype(np.int32)
    q = synth.normal_tensor(seed + 0, (B, H, 1, d), "bf16")
    kc = synth.normal_tensor(seed + 1, (num_pages, Hkv, page, d), "bf16")
    vc = synth.normal_tensor(seed + 2, (num_pages, Hkv, page, d), "bf16")
    seqlens = np.asarray(c["seqlens"], np.int32)
    o, lse = ea.attn_fwd_paged(to_device(q, "bf16"), to_device(kc, "bf16"), to_device(vc, "bf16"),
                               torch.from_numpy(table).cuda(), torch.from_numpy(seqlens).cuda(),
                               num_splits=c["splits"])
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(d)
    q32, k32, v32 = (host_f32(x, "bf16") for x in (q, kc, vc))
    o_ref, lse_ref = paged_oracle.paged_attention(q32[:, :, 0], k32, v32, table, seqlens, scale)
    a_ref, _ = paged_oracle.paged_attention(q32[:, :, 0], k32, np.abs(v32), table, seqlens, scale)
    check(o.float().cpu().numpy()[:, :, 0], lse.cpu().numpy(), o_ref, lse_ref, "bf16", f"random {name_paged(c)}",
          a_ref=a_ref)


# ---- many short sequences: the paths past the persistent grid's limit (more
# than 1024 sequences, forward) and past the ranked backward order (more than
# 64 sequences)

MANY = [
    # (layout, sequences, max length, H, Hkv, d, causal, backward)
    ("bshd", 1100, 24, 2, 1, 128, True, False),
    ("bhsd", 1100, 24, 4, 2, 64, False, False),
    ("bshd", 100, 90, 2, 1, 128, True, True),
    ("bhsd", 100, 90, 4, 4, 64, False, True),
]


@pytest.mark.parametrize("c", MANY, ids=lambda c: "-".join(map(str, c)))
def test_many_sequences(c):
    import exact_attention_09_amd as ea
    layout, nseq, maxlen, H, Hkv, d, causal, backward = c
    say(f"many sequences {c}")
    rng = np.random.default_rng(nseq * 7 + maxlen)
    lengths = tuple(int(x) for x in rng.integers(0, maxlen + 1, nseq))
    cfg = dict(layout=layout, d=d, H=H, Hkv=Hkv, causal=causal, window=0, sinks=False, lengths=lengths, B=nseq,
               Sq=sum(lengths), Skv=sum(lengths))
    seed = 10 * (MANY.index(c) + 9900)
    (q, k, v, do), _, (qt, kt, vt, dot), cu, cut, _ = inputs(cfg, seed)
    o, lse = ea.attn_fwd_layout(qt, kt, vt, layout=layout, causal=causal, cu_seqlens=cut)
    hq, hk, hv = (host_f32(x, "bf16") for x in (q, k, v))
    scale = 1.0 / math.sqrt(d)
    if not backward:
        torch.cuda.synchronize()
        og = to_bhsd(o, cfg)
        lg = lse.cpu().numpy().astype(np.float64).reshape(og.shape[:-1])
        o_ref, lse_ref, a_ref = reference(hq, hk, hv, scale, causal, cu_seqlens=cu)
        check(og, lg, o_ref, lse_ref, "bf16", f"many sequences {c}", a_ref=a_ref)
        return
    dq, dk, dv, _ = ea.attn_bwd_layout(qt, kt, vt, o, lse, dot, layout=layout, causal=causal, cu_seqlens=cut)
    torch.cuda.synchronize()
    got = tuple(to_bhsd(t, cfg) for t in (dq, dk, dv))
    hdo = host_f32(do, "bf16")
    for i in range(nseq):
        a, e = int(cu[i]), int(cu[i + 1])
        if e == a:
            continue
        sl = slice(a, e)
        want = bwd_oracle.attention_backward(hq[:, :, sl], hk[:, :, sl], hv[:, :, sl], hdo[:, :, sl], scale, causal)
        for g, w, name in zip(got, want[:3], ("dq", "dk", "dv")):
            gs = g[:, :, sl]
            scale_w = max(np.abs(w).max(), 1e-30)
            err = np.abs(gs - w).max()
            assert err <= 1e-2 * scale_w + 1e-4, f"{c} sequence {i} {name}: max|err| {err:.3g} of {scale_w:.3g}"
    say(f"  many sequences {c}: {nseq} sequences within the backward bar")
