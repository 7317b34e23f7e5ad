"""GPU parity for the backward in the BSHD and packed-THD layouts
(attn_bwd_layout).

A layout changes where rows live, not what is computed: every kernel reads
the same values and sums them in the same order, so the BSHD gradients must
equal the BHSD ones bit for bit once transposed back, and the BHSD path is
itself held to the fp64 backward oracle (test_parity_bwd_gpu.py).  Each case
checks that equality, and a few also compare the BSHD gradients with the
oracle directly.  The forward outputs that feed the backward come from
attn_fwd_layout in the same layout.
"""

import math
import zlib

import numpy as np
import pytest

from exact_attention_09_amd import synth
from exact_attention_09_amd.workloads import host_f32, to_device
from oracle import backward as bwd_oracle
from parity import compare_grads, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_09_amd as ea
    ea.load_library()
    return ea


def to_bshd(x):
    """[B, H, S, d] -> [B, S, H, d], contiguous."""
    return x.transpose(1, 2).contiguous()


def assert_same(a, b, what):
    assert a.shape == b.shape, f"{what}: shapes {tuple(a.shape)} and {tuple(b.shape)}"
    same = torch.equal(a, b)
    if not same:
        diff = (a.float() - b.float()).abs().max().item()
        raise AssertionError(f"{what}: BSHD and BHSD differ (max |diff| {diff:.3g})")


def sinks_for(seed, H):
    return torch.from_numpy(synth.normal_tensor(seed, (H,), "f32") * np.float32(2.0)).cuda()


DENSE = [
    # (B, H, Hkv, Sq, Skv, d, causal, window, with_sinks, oracle check)
    (2, 4, 2, 200, 200, 128, True, 0, False, True),
    (1, 8, 2, 256, 256, 128, False, 0, False, False),   # GQA group 4, whole tiles
    (1, 4, 1, 77, 300, 128, True, 0, False, False),     # Sq < Skv, MQA
    (1, 2, 2, 300, 130, 128, True, 0, False, False),    # Sq > Skv: rows with no key
    (2, 4, 4, 333, 333, 64, True, 0, False, True),
    (1, 6, 3, 129, 257, 64, False, 0, False, False),
    (1, 4, 2, 300, 300, 128, True, 64, True, True),     # window and sinks
    (1, 4, 4, 257, 257, 64, True, 100, False, False),   # window only
]


@pytest.mark.parametrize("case", DENSE, ids=lambda c: "-".join(map(str, c[:9])))
def test_bwd_bshd_dense(gpu, case):
    ea = gpu
    B, H, Hkv, Sq, Skv, d, causal, window, with_sinks, check_oracle = case
    say(f"backward BSHD {case}")
    seed = zlib.crc32(repr(case).encode()) % 10000
    q = synth.normal_tensor(seed * 10 + 0, (B, H, Sq, d), "bf16")
    k = synth.normal_tensor(seed * 10 + 1, (B, Hkv, Skv, d), "bf16")
    v = synth.normal_tensor(seed * 10 + 2, (B, Hkv, Skv, d), "bf16")
    do = synth.normal_tensor(seed * 10 + 3, (B, H, Sq, d), "bf16")
    qt, kt, vt, dot = (to_device(x, "bf16") for x in (q, k, v, do))
    sk = sinks_for(seed * 10 + 5, H) if with_sinks else None

    # BHSD: the forward and the backward through the general entry points
    o, lse = ea.attn_fwd_layout(qt, kt, vt, layout="bhsd", causal=causal, window=window, sinks=sk)
    ref = ea.attn_bwd_layout(qt, kt, vt, o, lse, dot, layout="bhsd", causal=causal, window=window, sinks=sk)
    # the BHSD call is the plain entry points' call
    if window > 0 or sk is not None:
        plain = ea.attn_bwd_window_sink(qt, kt, vt, o, lse, dot, window=window, sinks=sk)
    else:
        plain = ea.attn_bwd(qt, kt, vt, o, lse, dot, causal=causal) + (None,)
    for name, a, b in zip(("dq", "dk", "dv", "dsinks"), ref, plain):
        if a is not None:
            assert_same(a, b, f"{case} {name} (attn_bwd_layout BHSD vs the plain entry point)")

    # BSHD: forward and backward on the transposed tensors
    qb, kb, vb, dob = (to_bshd(x) for x in (qt, kt, vt, dot))
    ob, lseb = ea.attn_fwd_layout(qb, kb, vb, layout="bshd", causal=causal, window=window, sinks=sk)
    assert_same(ob, to_bshd(o), f"{case} forward o")
    assert_same(lseb, lse, f"{case} forward lse")
    got = ea.attn_bwd_layout(qb, kb, vb, ob, lseb, dob, layout="bshd", causal=causal, window=window, sinks=sk)
    torch.cuda.synchronize()
    for name, g, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        assert_same(g, to_bshd(r), f"{case} {name}")
    if sk is not None:
        assert_same(got[3], ref[3], f"{case} dsinks")

    if check_oracle:
        sinks_np = sk.cpu().numpy() if sk is not None else None
        want = bwd_oracle.attention_backward(*(host_f32(x, "bf16") for x in (q, k, v, do)), 1.0 / math.sqrt(d),
                                             causal, window=window, sinks=sinks_np)
        grads = tuple(g.transpose(1, 2).float().cpu().numpy().astype(np.float64) for g in got[:3])
        compare_grads(grads, want[:3], f"BSHD {case}")


VARLEN = [
    # (sequence lengths, H, Hkv, d, causal, window, with_sinks, oracle check)
    ((1, 130, 77, 300, 64, 129), 4, 2, 64, True, 0, False, True),
    ((257, 1, 128, 500), 4, 4, 128, False, 0, False, False),
    ((200, 333, 1000, 64), 8, 2, 128, True, 0, False, True),
    ((0, 96, 0, 129), 2, 1, 128, True, 0, False, False),       # empty sequences in the list
    ((300, 77, 513), 4, 2, 128, True, 64, True, False),         # window and sinks
]


@pytest.mark.parametrize("case", VARLEN, ids=lambda c: "-".join(map(str, c[0])) + "-" + "-".join(map(str, c[1:7])))
def test_bwd_thd_varlen(gpu, case):
    """Packed sequences as [T, H, d]: the THD gradients equal the BHSD
    varlen ones ([1, H, T, d]) bit for bit, and (some cases) each sequence's
    equal the oracle's for that sequence alone."""
    ea = gpu
    lengths, H, Hkv, d, causal, window, with_sinks, check_oracle = case
    say(f"backward THD varlen {case}")
    T = sum(lengths)
    seed = zlib.crc32(repr(case).encode()) % 10000
    q = synth.normal_tensor(seed * 10 + 0, (1, H, T, d), "bf16")
    k = synth.normal_tensor(seed * 10 + 1, (1, Hkv, T, d), "bf16")
    v = synth.normal_tensor(seed * 10 + 2, (1, Hkv, T, d), "bf16")
    do = synth.normal_tensor(seed * 10 + 3, (1, H, T, d), "bf16")
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)).cuda()
    qt, kt, vt, dot = (to_device(x, "bf16") for x in (q, k, v, do))
    sk = sinks_for(seed * 10 + 5, H) if with_sinks else None

    o, lse = ea.attn_fwd_layout(qt, kt, vt, layout="bhsd", causal=causal, window=window, sinks=sk, cu_seqlens=cu)
    ref = ea.attn_bwd_layout(qt, kt, vt, o, lse, dot, layout="bhsd", causal=causal, window=window, sinks=sk,
                             cu_seqlens=cu)

    def thd(x):  # [1, H, T, d] -> [T, H, d]
        return x[0].transpose(0, 1).contiguous()

    qp, kp, vp, dop = (thd(x) for x in (qt, kt, vt, dot))
    op, lsep = ea.attn_fwd_layout(qp, kp, vp, layout="bshd", causal=causal, window=window, sinks=sk, cu_seqlens=cu)
    assert_same(op, thd(o), f"{case} forward o")
    assert_same(lsep, lse[0], f"{case} forward lse")
    got = ea.attn_bwd_layout(qp, kp, vp, op, lsep, dop, layout="bshd", causal=causal, window=window, sinks=sk,
                             cu_seqlens=cu)
    torch.cuda.synchronize()
    for name, g, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        assert_same(g, thd(r), f"{case} {name}")
    if sk is not None:
        assert_same(got[3], ref[3], f"{case} dsinks")

    if check_oracle:
        grads = tuple(g.transpose(0, 1).unsqueeze(0).float().cpu().numpy().astype(np.float64) for g in got[:3])
        s0 = 0
        for i, n in enumerate(lengths):
            if n > 0:
                sl = slice(s0, s0 + n)
                want = bwd_oracle.attention_backward(*(host_f32(x, "bf16")[:, :, sl] for x in (q, k, v, do)),
                                                     1.0 / math.sqrt(d), causal)
                compare_grads(tuple(g[:, :, sl] for g in grads), want[:3], f"THD {case} sequence {i}")
            s0 += n


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_bshd_workload_shape(gpu, causal):
    """The 8K workload shape (B=1, H=32, S=8192, d=128) in BSHD: row strides
    of 8 KB and offsets past 2^26 bytes, gradients bit for bit those of BHSD
    (whose parity at this shape test_parity_bwd_gpu.py checks on a full
    head)."""
    ea = gpu
    B, H, S, d = 1, 32, 8192, 128
    say(f"backward BSHD at the workload shape, causal={causal}")
    q, k, v, do = (to_device(synth.normal_tensor(4100 + 10 * int(causal) + i, (B, H, S, d), "bf16"), "bf16")
                   for i in range(4))
    o, lse = ea.attn_fwd_layout(q, k, v, layout="bhsd", causal=causal)
    ref = ea.attn_bwd_layout(q, k, v, o, lse, do, layout="bhsd", causal=causal)
    qb, kb, vb, dob, ob = (to_bshd(x) for x in (q, k, v, do, o))
    got = ea.attn_bwd_layout(qb, kb, vb, ob, lse, dob, layout="bshd", causal=causal)
    torch.cuda.synchronize()
    for name, g, r in zip(("dq", "dk", "dv"), got[:3], ref[:3]):
        assert_same(g, to_bshd(r), f"8K causal={causal} {name}")
