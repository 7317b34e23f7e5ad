"""GPU parity for split-KV decode over a paged KV cache (attn_fwd_paged)
against the paged oracle (``oracle/paged.py``: gather through the block
table, then naive fp64 attention).

The bar is the one of the other bf16 tests: |dO| <= 1e-2 plus half the bf16
spacing at the exact value, |dLSE| <= 1e-3, O = 0 and LSE = -inf exactly for
a sequence without keys.  Because a paged cache only changes where the bytes
are read from, the paged kernel must also give bitwise the output of the
contiguous decode path on the same keys with the same split count.
"""

import math
import zlib

import numpy as np
import pytest

from exact_attention_09_amd import synth
from exact_attention_09_amd.workloads import WORKLOADS, host_f32, to_device
from oracle import paged as paged_oracle
from parity import check, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_09_amd as ea
    ea.load_library()
    return ea


def run_paged(q, kc, vc, table, seqlens, scale, num_splits=0):
    import exact_attention_09_amd as ea
    qt = to_device(q, "bf16")
    kt, vt = to_device(kc, "bf16"), to_device(vc, "bf16")
    bt = torch.from_numpy(np.ascontiguousarray(table, np.int32)).cuda()
    sl = torch.from_numpy(np.ascontiguousarray(seqlens, np.int32)).cuda()
    o, lse = ea.attn_fwd_paged(qt, kt, vt, bt, sl, scale=scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return o, lse


def test_paged_workload_parity_and_equals_contiguous():
    import exact_attention_09_amd as ea
    wl = WORKLOADS["decode_paged_gqa_s16384_d128"]
    say(f"paged workload: B={wl.B} H={wl.H} Hkv={wl.Hkv} Skv={wl.Skv} page={wl.page_size} "
        f"splits={wl.num_splits}")
    x = wl.make_inputs()
    o, lse = run_paged(x["q"], x["k"], x["v"], x["block_table"], x["seqlens_k"], wl.scale, wl.num_splits)
    og = o.float().cpu().numpy().astype(np.float64)[:, :, 0, :]
    lg = lse.cpu().numpy().astype(np.float64)
    q32 = host_f32(x["q"], "bf16")[:, :, 0, :]
    kc, vc = host_f32(x["k"], "bf16"), host_f32(x["v"], "bf16")
    o_ref, lse_ref = paged_oracle.paged_attention(q32, kc, vc, x["block_table"], x["seqlens_k"], wl.scale)
    a_ref, _ = paged_oracle.paged_attention(q32, kc, np.abs(vc), x["block_table"], x["seqlens_k"], wl.scale)
    check(og, lg, o_ref, lse_ref, "bf16", "paged decode workload", a_ref=a_ref, workload=True)
    # the same keys laid out contiguously through the dense decode path
    kd = np.stack([paged_oracle.gather(x["k"], x["block_table"][b], wl.Skv) for b in range(wl.B)])
    vd = np.stack([paged_oracle.gather(x["v"], x["block_table"][b], wl.Skv) for b in range(wl.B)])
    qt, kt, vt = to_device(x["q"], "bf16"), to_device(kd, "bf16"), to_device(vd, "bf16")
    o2, l2 = ea.attn_fwd(qt, kt, vt, num_splits=wl.num_splits)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), "paged and contiguous decode differ"
    assert torch.equal(lse, l2[:, :, 0])


PAGED_EDGE = [
    # (B, H, Hkv, d, page_size, seqlens, num_splits)
    (3, 8, 2, 128, 16, (0, 1, 17), 0),
    (4, 8, 8, 64, 16, (15, 16, 33, 200), 3),
    (2, 40, 2, 128, 32, (700, 65), 7),          # group of 20 heads: two head groups
    (2, 4, 1, 128, 64, (1000, 1), 16),
    (1, 4, 4, 64, 256, (513,), 0),
    (5, 8, 2, 128, 16, (5, 0, 1, 1024, 31), 40),  # more splits than some sequences' keys
    (2, 8, 2, 128, 1024, (3000, 2048), 2),
]


@pytest.mark.parametrize("case", PAGED_EDGE, ids=lambda c: "-".join(map(str, c)))
def test_paged_edges(case):
    B, H, Hkv, d, ps, lens, ns = case
    say(f"paged case {case}")
    seed = zlib.crc32(repr(case).encode()) % 10000
    max_pages = max(1, -(-max(lens) // ps)) + 1       # one unused table column
    num_pages = B * max_pages + 3
    q = synth.normal_tensor(seed * 10 + 0, (B, H, 1, d), "bf16")
    kc = synth.normal_tensor(seed * 10 + 1, (num_pages, Hkv, ps, d), "bf16")
    vc = synth.normal_tensor(seed * 10 + 2, (num_pages, Hkv, ps, d), "bf16")
    table = synth.page_table(seed * 10 + 4, B, max_pages, num_pages)
    seqlens = np.array(lens, np.int32)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_paged(q, kc, vc, table, seqlens, scale, ns)
    og = o.float().cpu().numpy().astype(np.float64)[:, :, 0, :]
    lg = lse.cpu().numpy().astype(np.float64)
    q32, k32, v32 = host_f32(q, "bf16")[:, :, 0, :], host_f32(kc, "bf16"), host_f32(vc, "bf16")
    o_ref, lse_ref = paged_oracle.paged_attention(q32, k32, v32, table, seqlens, scale)
    a_ref, _ = paged_oracle.paged_attention(q32, k32, np.abs(v32), table, seqlens, scale)
    check(og, lg, o_ref, lse_ref, "bf16", str(case), a_ref=a_ref)


def test_paged_malformed_table_stays_in_bounds():
    """Table entries outside [0, num_pages) and lengths beyond the table are
    clamped on the device: the call completes and the outputs are finite."""
    B, H, Hkv, d, ps, max_pages, num_pages = 2, 8, 2, 128, 16, 4, 6
    q = to_device(synth.normal_tensor(61, (B, H, 1, d), "bf16"), "bf16")
    kc = to_device(synth.normal_tensor(62, (num_pages, Hkv, ps, d), "bf16"), "bf16")
    vc = to_device(synth.normal_tensor(63, (num_pages, Hkv, ps, d), "bf16"), "bf16")
    bt = torch.tensor([[0, 5, 99, -7], [1 << 30, 2, 3, 4]], dtype=torch.int32, device="cuda")
    sl = torch.tensor([10 ** 6, -5], dtype=torch.int32, device="cuda")
    import exact_attention_09_amd as ea
    o, lse = ea.attn_fwd_paged(q, kc, vc, bt, sl)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(o[0].float())) and torch.all(torch.isfinite(lse[0]))
    assert torch.all(o[1].float() == 0.0) and torch.all(torch.isneginf(lse[1]))
