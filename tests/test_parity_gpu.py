"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle on
the same seeded inputs (bars in ``parity.py``: the raw 1e-2 workload bar on
every element of the benchmark workloads, the bf16 rounding bound everywhere,
1e-5 for fp32, 1e-3 for the LSE).
"""

import math
import zlib

import numpy as np
import pytest

from exact_attention_09_amd import synth
from exact_attention_09_amd.workloads import WORKLOADS, host_f32, to_device
from parity import bf16_half_spacing, check, oracle_threads, reference, say
from pins import assert_printed, golden

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_09_amd as ea
    ea.load_library()  # fails loudly if the library was not built
    return ea


def gpu_run(q, k, v, dtype, causal, scale, cu=None, num_splits=0, flags=0):
    import exact_attention_09_amd as ea
    qt, kt, vt = (to_device(x, dtype) for x in (q, k, v))
    cut = torch.from_numpy(np.asarray(cu, np.int32)).cuda() if cu is not None else None
    o, lse = ea.attn_fwd_ex(qt, kt, vt, causal=causal, scale=scale, cu_seqlens=cut,
                            num_splits=num_splits, flags=flags)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def oracle_dense(q, k, v, dtype, scale, causal, cu=None, rows=None):
    """(O, LSE, A) of the oracle for host inputs (bf16 bits or fp32)."""
    return reference(host_f32(q, dtype), host_f32(k, dtype), host_f32(v, dtype), scale, causal,
                     cu_seqlens=cu, rows=rows)


# ------------------------------------------------------------ worked examples

def _example_inputs(scores, d, rows):
    n = len(scores)
    q = np.zeros((1, 1, rows, d), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, n, d), np.float32)
    k[0, 0, :, 0] = scores
    v = np.zeros((1, 1, n, d), np.float32)
    for j in range(n):
        v[0, 0, j, j] = 1.0
    return q, k, v


@pytest.mark.parametrize("example", ["four_scores", "three_blocks"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,num_splits", [(1, 1), (1, 2), (1, 3), (2, 0), (130, 0)])
def test_worked_examples_through_api(example, dtype, rows, num_splits):
    """The pages' worked examples run through attn_fwd: q = e0, k_j = x_j e0,
    v_j = e_j, scale 1, so O's first entries are the softmax weights.  One row
    takes the split-KV path (2 splits of the four scores is the LLM course's
    two-block example), more rows take the tiled path."""
    g = golden()[example]
    scores = [x for b in g["blocks"] for x in b]
    q, k, v = _example_inputs(scores, 64, rows)
    if dtype == "bf16":
        q, k, v = (synth.f32_to_bf16_bits(x) for x in (q, k, v))  # all values exact in bf16
    say(f"worked example {example} {dtype} rows={rows} splits={num_splits}")
    o, lse = gpu_run(q, k, v, dtype, False, 1.0, num_splits=num_splits)
    o_ref, lse_ref, a_ref = oracle_dense(q, k, v, dtype, 1.0, False)
    check(o, lse, o_ref, lse_ref, dtype, f"{example}/{dtype}", a_ref=a_ref, workload=True)
    for r in range(rows):
        for j, w in enumerate(g["weights"]):
            got = o[0, 0, r, j]
            if dtype == "f32":
                assert_printed(got, w, f"weight {j}")
            else:  # bf16 output: printed value within its own rounding plus one bf16 spacing
                assert abs(got - float(w)) <= 0.5 * 10 ** -(len(w.split('.')[1])) + 2 * bf16_half_spacing(got)
        assert np.all(o[0, 0, r, len(scores):] == 0.0)
    if example == "four_scores":
        assert_printed(math.exp(lse[0, 0, 0]), g["exp_sum"], "sum of exp")


# ------------------------------------------------------------ the workloads

# the benchmark workloads (the five configurations, the 8K one with and
# without the causal mask), compared on every output element
CONFIG_WORKLOADS = ["single_head_f32", "mha_causal_s2048_d64", "mha_s8192_d128", "mha_causal_s8192_d128",
                    "varlen_gqa_causal_d128", "decode_gqa_s16384_d128"]


@pytest.mark.parametrize("name", CONFIG_WORKLOADS)
def test_workload_parity(name):
    """Every row of the workload against the oracle: the raw 1e-2 bar (1e-5
    for fp32) and the rounding bound on each element, 1e-3 on each LSE."""
    wl = WORKLOADS[name]
    say(f"workload {name}: B={wl.B} H={wl.H} Hkv={wl.Hkv} Sq={wl.Sq} Skv={wl.Skv} d={wl.d} "
        f"{wl.dtype} causal={wl.causal} (oracle on {oracle_threads()} threads)")
    x = wl.make_inputs()
    o, lse = gpu_run(x["q"], x["k"], x["v"], wl.dtype, wl.causal, wl.scale, cu=x["cu_seqlens"],
                     num_splits=wl.num_splits)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    vmax = float(np.abs(host_f32(x["v"], wl.dtype)).max())
    assert np.abs(o).max() <= vmax * (1 + 2 ** -7)  # a convex combination of V rows
    q, k, v = (host_f32(x[t], wl.dtype) for t in ("q", "k", "v"))
    if wl.varlen:
        q, k, v, o, lse = q[0], k[0], v[0], o[0], lse[0]
    o_ref, lse_ref, a_ref = reference(q, k, v, wl.scale, wl.causal, cu_seqlens=x["cu_seqlens"])
    check(o, lse, o_ref, lse_ref, wl.dtype, name, a_ref=a_ref if wl.dtype == "bf16" else None, workload=True)


# ------------------------------------------------------------ edge shapes

EDGE = [
    # dtype, B, H, Hkv, Sq, Skv, d, causal, num_splits
    ("bf16", 1, 2, 2, 100, 100, 64, False, 0),      # one partial tile
    ("bf16", 1, 2, 2, 257, 257, 128, False, 0),     # ragged tail, several tiles
    ("bf16", 2, 4, 1, 77, 200, 128, True, 0),       # Sq < Skv causal (bottom right), MQA
    ("bf16", 1, 2, 2, 300, 130, 128, True, 0),      # Sq > Skv causal: 170 rows see nothing
    ("bf16", 1, 2, 2, 300, 130, 64, True, 0),
    ("bf16", 1, 3, 3, 129, 1, 64, False, 0),        # one key
    ("bf16", 2, 6, 3, 200, 200, 64, True, 0),       # GQA group 2, d = 64
    ("bf16", 2, 4, 2, 77, 300, 64, True, 0),        # d = 64, Sq < Skv causal, ragged key tail
    ("bf16", 1, 2, 2, 257, 333, 64, False, 0),      # d = 64 non-causal, ragged tails in both
    ("bf16", 1, 4, 4, 150, 150, 64, True, 0),       # d = 64 causal, diagonals inside 16-key chunks
    ("bf16", 1, 4, 4, 128, 0, 128, False, 0),       # no keys at all
    ("bf16", 1, 2, 1, 1, 1000, 128, False, 0),      # decode, heuristic split
    ("bf16", 2, 8, 2, 1, 333, 64, True, 3),         # decode d = 64 (causal is moot at Sq = 1)
    ("bf16", 1, 4, 4, 1, 5, 128, False, 16),        # more splits than keys
    ("bf16", 2, 40, 2, 1, 700, 128, False, 7),      # group of 20 heads: two head groups
    ("bf16", 1, 2, 2, 1, 0, 64, False, 0),          # decode with an empty cache
    ("f32", 1, 2, 2, 100, 100, 64, False, 0),
    ("f32", 2, 4, 1, 77, 200, 128, True, 0),
    ("f32", 1, 2, 2, 300, 130, 64, True, 0),
    ("f32", 1, 2, 1, 1, 1000, 128, False, 0),
    ("f32", 2, 6, 2, 1, 99, 64, False, 4),
    ("f32", 1, 2, 2, 64, 0, 64, True, 0),
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "-".join(map(str, c)))
def test_edge_shapes(case):
    dtype, B, H, Hkv, Sq, Skv, d, causal, ns = case
    say(f"edge case {case}")
    seed = zlib.crc32(repr(case).encode()) % 10000
    q = synth.normal_tensor(seed * 10 + 0, (B, H, Sq, d), dtype)
    k = synth.normal_tensor(seed * 10 + 1, (B, Hkv, Skv, d), dtype)
    v = synth.normal_tensor(seed * 10 + 2, (B, Hkv, Skv, d), dtype)
    scale = 1.0 / math.sqrt(d)
    o, lse = gpu_run(q, k, v, dtype, causal, scale, num_splits=ns)
    o_ref, lse_ref, a_ref = oracle_dense(q, k, v, dtype, scale, causal)
    check(o, lse, o_ref, lse_ref, dtype, str(case), a_ref=a_ref)


VARLEN_EDGE = [
    ("bf16", (5, 0, 1, 127, 128, 129, 300), 4, 2, 128, True),
    ("bf16", (5, 0, 1, 127, 128, 129, 300), 4, 4, 64, False),
    ("bf16", (0,), 2, 1, 64, True),
    ("bf16", (1000, 3), 8, 2, 128, True),
    ("f32", (5, 0, 1, 33, 64, 100), 4, 2, 64, True),
    ("f32", (70, 31), 2, 2, 128, False),
]


@pytest.mark.parametrize("case", VARLEN_EDGE, ids=lambda c: "-".join(map(str, c)))
def test_varlen_edges(case):
    dtype, lengths, H, Hkv, d, causal = case
    say(f"varlen case {case}")
    T = sum(lengths)
    cu = synth.cu_seqlens_from_lengths(lengths)
    seed = zlib.crc32(repr(case).encode()) % 10000
    q = synth.normal_tensor(seed * 10 + 0, (1, H, T, d), dtype)
    k = synth.normal_tensor(seed * 10 + 1, (1, Hkv, T, d), dtype)
    v = synth.normal_tensor(seed * 10 + 2, (1, Hkv, T, d), dtype)
    scale = 1.0 / math.sqrt(d)
    o, lse = gpu_run(q, k, v, dtype, causal, scale, cu=cu)
    if T == 0:
        return
    o_ref, lse_ref, a_ref = reference(host_f32(q, dtype)[0], host_f32(k, dtype)[0], host_f32(v, dtype)[0],
                                      scale, causal, cu_seqlens=cu)
    check(o[0], lse[0], o_ref, lse_ref, dtype, str(case), a_ref=a_ref)


BASIC_FLAG = 1  # ATTN_FLAG_BASIC_PREFILL
BASIC = [
    ("dense", 1, 2, 2, 257, 257, True, 128),
    ("dense", 2, 4, 1, 77, 200, True, 128),
    ("dense", 1, 2, 2, 300, 130, False, 128),
    ("dense", 2, 6, 3, 200, 200, True, 64),
    ("dense", 1, 2, 2, 300, 130, True, 64),
    ("varlen", (5, 0, 127, 128, 300), 4, 2, 0, 0, True, 128),
    ("varlen", (5, 0, 127, 128, 300), 4, 4, 0, 0, False, 64),
]


@pytest.mark.parametrize("case", BASIC, ids=lambda c: "-".join(map(str, c)))
def test_basic_kernel(case):
    """bf16 prefill normally runs the ping-pong kernel; ATTN_FLAG_BASIC_PREFILL
    selects the basic tiled kernel, which must meet the same bar."""
    say(f"basic kernel case {case}")
    seed = zlib.crc32(repr(case).encode()) % 10000
    d = case[-1]
    scale = 1.0 / math.sqrt(d)
    if case[0] == "varlen":
        _, lengths, H, Hkv, _, _, causal, _ = case
        T = sum(lengths)
        cu = synth.cu_seqlens_from_lengths(lengths)
        q, k, v = (synth.normal_tensor(seed * 10 + i, (1, h, T, d), "bf16") for i, h in enumerate((H, Hkv, Hkv)))
        o, lse = gpu_run(q, k, v, "bf16", causal, scale, cu=cu, flags=BASIC_FLAG)
        o_ref, lse_ref, a_ref = reference(host_f32(q, "bf16")[0], host_f32(k, "bf16")[0],
                                          host_f32(v, "bf16")[0], scale, causal, cu_seqlens=cu)
        check(o[0], lse[0], o_ref, lse_ref, "bf16", str(case), a_ref=a_ref)
        return
    _, B, H, Hkv, Sq, Skv, causal, _ = case
    q = synth.normal_tensor(seed * 10 + 0, (B, H, Sq, d), "bf16")
    k = synth.normal_tensor(seed * 10 + 1, (B, Hkv, Skv, d), "bf16")
    v = synth.normal_tensor(seed * 10 + 2, (B, Hkv, Skv, d), "bf16")
    o, lse = gpu_run(q, k, v, "bf16", causal, scale, flags=BASIC_FLAG)
    o_ref, lse_ref, a_ref = oracle_dense(q, k, v, "bf16", scale, causal)
    check(o, lse, o_ref, lse_ref, "bf16", str(case), a_ref=a_ref)


@pytest.mark.parametrize("varlen", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_dispatched_grid_matches_persistent(causal, varlen):
    """bf16 prefill runs a persistent grid when the query tiles divide evenly
    over the CUs (dense) or when the sequence scan is short (varlen); the
    one-workgroup-per-tile grid (ATTN_FLAG_NO_PERSIST) must give bitwise the
    same result."""
    import exact_attention_09_amd as ea
    say(f"persistent vs dispatched, causal={causal} varlen={varlen}")
    d = 128
    if varlen:
        lengths = (700, 1, 0, 2100, 256, 513, 3000)
        cu = torch.from_numpy(np.asarray(synth.cu_seqlens_from_lengths(lengths), np.int32)).cuda()
        T = sum(lengths)
        q = to_device(synth.normal_tensor(9200, (1, 16, T, d), "bf16"), "bf16")
        k, v = (to_device(synth.normal_tensor(9201 + i, (1, 4, T, d), "bf16"), "bf16") for i in range(2))
    else:
        cu = None
        q, k, v = (to_device(synth.normal_tensor(9100 + i, (1, 32, 2048, d), "bf16"), "bf16") for i in range(3))
    o1, l1 = ea.attn_fwd(q, k, v, causal=causal, cu_seqlens=cu)
    o2, l2 = ea.attn_fwd(q, k, v, causal=causal, cu_seqlens=cu, flags=ea.ATTN_FLAG_NO_PERSIST)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


PERSISTENT = [
    # (B, H, Hkv, Sq, Skv, d, causal): 256 query tiles of 256 rows, so on a
    # 256-CU part the persistent grid runs them
    (2, 16, 4, 2048, 1024, 128, True),    # Sq > Skv: the first 1024 rows see no key
    (2, 16, 16, 2048, 3000, 128, True),   # Sq < Skv, ragged key tail
    (1, 32, 8, 2048, 2048, 64, False),
    (4, 8, 2, 2048, 777, 64, True),
]


def _edge_and_random_rows(B, H, Sq, rng, n=192):
    fixed = sorted({0, 1, 255, 256, 1023, 1024, Sq // 2, Sq - 2, Sq - 1})
    rows = [(int(rng.integers(B)), int(rng.integers(H)), i) for i in fixed if 0 <= i < Sq]
    while len(rows) < n:
        rows.append((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(Sq))))
    return np.array(rows, np.int64)


@pytest.mark.parametrize("case", PERSISTENT, ids=lambda c: "-".join(map(str, c)))
def test_persistent_shapes(case):
    """Persistent-grid prefill (heavy/light pairing, GQA, Sq != Skv, d = 64)
    against the oracle on sampled rows."""
    B, H, Hkv, Sq, Skv, d, causal = case
    say(f"persistent case {case}")
    seed = zlib.crc32(repr(case).encode()) % 10000
    q = synth.normal_tensor(seed * 10 + 0, (B, H, Sq, d), "bf16")
    k = synth.normal_tensor(seed * 10 + 1, (B, Hkv, Skv, d), "bf16")
    v = synth.normal_tensor(seed * 10 + 2, (B, Hkv, Skv, d), "bf16")
    scale = 1.0 / math.sqrt(d)
    o, lse = gpu_run(q, k, v, "bf16", causal, scale)
    rows = _edge_and_random_rows(B, H, Sq, np.random.default_rng(seed))
    o_ref, lse_ref, a_ref = oracle_dense(q, k, v, "bf16", scale, causal, rows=rows)
    og = np.stack([o[b, h, i] for b, h, i in rows])
    lg = np.array([lse[b, h, i] for b, h, i in rows])
    check(og, lg, o_ref, lse_ref, "bf16", str(case), a_ref=a_ref)


def test_persistent_varlen_many_sequences():
    """Varlen with 40 sequences (empty, one-token and long ones) on the
    persistent listed order, against the oracle on sampled rows."""
    rng = np.random.default_rng(4242)
    lengths = [0, 1, 2, 255, 256, 257] + [int(x) for x in rng.integers(1, 1500, 34)]
    H, Hkv, d = 16, 4, 128
    say(f"persistent varlen, {len(lengths)} sequences, T={sum(lengths)}")
    T = sum(lengths)
    cu = synth.cu_seqlens_from_lengths(lengths)
    q = synth.normal_tensor(5100, (1, H, T, d), "bf16")
    k = synth.normal_tensor(5101, (1, Hkv, T, d), "bf16")
    v = synth.normal_tensor(5102, (1, Hkv, T, d), "bf16")
    scale = 1.0 / math.sqrt(d)
    o, lse = gpu_run(q, k, v, "bf16", True, scale, cu=cu)
    rows = []
    for b, L in enumerate(lengths):
        for i in sorted({0, L // 2, L - 1}):
            if 0 <= i < L:
                rows.append((b, int(rng.integers(H)), i))
    rows = np.array(rows, np.int64)
    rf, lf, af = reference(host_f32(q, "bf16")[0], host_f32(k, "bf16")[0], host_f32(v, "bf16")[0],
                           scale, True, cu_seqlens=cu, rows=rows)
    og = np.stack([o[0, h, cu[b] + i] for b, h, i in rows])
    lg = np.array([lse[0, h, cu[b] + i] for b, h, i in rows])
    check(og, lg, rf, lf, "bf16", "persistent varlen", a_ref=af)


# ------------------------------------------------------------ determinism, canaries

@pytest.mark.parametrize("Sq,ns", [(1, 16), (300, 0)])
def test_bitwise_repeatable(Sq, ns):
    import exact_attention_09_amd as ea
    say(f"repeatability Sq={Sq} splits={ns}")
    q = to_device(synth.normal_tensor(71, (2, 8, Sq, 128), "bf16"), "bf16")
    k = to_device(synth.normal_tensor(72, (2, 2, 4000, 128), "bf16"), "bf16")
    v = to_device(synth.normal_tensor(73, (2, 2, 4000, 128), "bf16"), "bf16")
    o1, l1 = ea.attn_fwd(q, k, v, num_splits=ns)
    o2, l2 = ea.attn_fwd(q, k, v, num_splits=ns)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype,Sq,causal", [("bf16", 200, True), ("bf16", 1, False), ("f32", 70, False),
                                             ("f32", 1, False)])
def test_guard_bands_untouched(dtype, Sq, causal):
    """Outputs written through views inside larger buffers: the bytes around
    them keep their canary values."""
    import exact_attention_09_amd as ea
    say(f"guard bands {dtype} Sq={Sq}")
    B, H, Hkv, Skv, d = 2, 4, 2, 150, 64
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = to_device(synth.normal_tensor(81, (B, H, Sq, d), dtype), dtype)
    k = to_device(synth.normal_tensor(82, (B, Hkv, Skv, d), dtype), dtype)
    v = to_device(synth.normal_tensor(83, (B, Hkv, Skv, d), dtype), dtype)
    n, pad = B * H * Sq * d, 256
    obuf = torch.full((n + 2 * pad,), 7.0, dtype=tdt, device="cuda")
    lbuf = torch.full((B * H * Sq + 2 * pad,), 9.0, dtype=torch.float32, device="cuda")
    o = obuf[pad:pad + n].view(B, H, Sq, d)
    lse = lbuf[pad:pad + B * H * Sq].view(B, H, Sq)
    ea.attn_fwd_ex(q, k, v, o, lse, causal=causal)
    torch.cuda.synchronize()
    assert torch.all(obuf[:pad] == 7.0) and torch.all(obuf[pad + n:] == 7.0)
    assert torch.all(lbuf[:pad] == 9.0) and torch.all(lbuf[pad + B * H * Sq:] == 9.0)
    assert torch.all(torch.isfinite(o.float()))


def test_caller_workspace_matches_internal():
    import exact_attention_09_amd as ea
    say("caller workspace")
    q = to_device(synth.normal_tensor(91, (3, 8, 1, 128), "bf16"), "bf16")
    k = to_device(synth.normal_tensor(92, (3, 2, 2000, 128), "bf16"), "bf16")
    v = to_device(synth.normal_tensor(93, (3, 2, 2000, 128), "bf16"), "bf16")
    nbytes = ea.attn_workspace_bytes(3, 8, 128, 5)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    o1, l1 = ea.attn_fwd(q, k, v, num_splits=5)
    o2, l2 = ea.attn_fwd(q, k, v, num_splits=5, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
