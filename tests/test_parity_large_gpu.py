"""Tensors past 2^31 elements: every K/V offset in the kernels must be 64-bit.

K and V hold 2^24 + 64 keys of d = 128, that is 2^31 + 8192 elements each
(4.3 GB).  The inputs are the two-kind structure of tests/closed_forms.py
with c = 8: keys below 2^24 have k = 0 and v = e1, the 64 keys past the
2^31-element boundary have k = 8 e0 and v = e2, every query row is e0 and,
for the backward, every row of dO is e2.  The expected outputs and
gradients are those closed forms in fp64 (pinned to the oracle on a small
instance in test_closed_forms.py).  A 32-bit wrap of a row offset would
read or write the first rows in place of the last ones and lose the e2
weight.
"""

import pytest
import torch

import exact_attention_09_amd as ea

import closed_forms

pytestmark = pytest.mark.gpu

N0 = 1 << 24  # keys of score 0, value e1
N1 = 64       # keys past element 2^31: score 8, value e2
D = 128
H, HKV = 4, 1


@pytest.fixture(scope="module")
def kv():
    skv = N0 + N1
    assert skv * D > 2 ** 31
    k = torch.zeros((1, HKV, skv, D), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    k[:, :, N0:, 0] = 8.0
    v[:, :, :N0, 1] = 1.0
    v[:, :, N0:, 2] = 1.0
    torch.cuda.synchronize()
    yield k, v
    del k, v
    torch.cuda.empty_cache()


def query(sq):
    q = torch.zeros((1, H, sq, D), dtype=torch.bfloat16, device="cuda")
    q[..., 0] = 1.0
    return q


def check(o, lse, n1_of_row):
    """o [1, H, Sq, D], lse [1, H, Sq]; row i sees N0 keys of score 0 and
    n1_of_row(i) of score 8."""
    o = o.float().cpu()
    lse = lse.cpu()
    sq = o.shape[2]
    for i in range(sq):
        e1, e2, l = closed_forms.forward(N0, n1_of_row(i), 8.0)
        row = o[0, :, i, :]
        assert (row[:, 1] - e1).abs().max().item() <= 1e-2, (i, row[:, 1], e1)
        assert (row[:, 2] - e2).abs().max().item() <= 1e-2, (i, row[:, 2], e2)
        assert row[:, 0].abs().max().item() == 0.0
        assert row[:, 3:].abs().max().item() == 0.0
        assert (lse[0, :, i].double() - l).abs().max().item() <= 1e-3, (i, lse[0, :, i], l)


@pytest.mark.parametrize("num_splits", [0, ea.ATTN_MAX_SPLITS])
def test_decode_past_2_31_elements(kv, num_splits):
    k, v = kv
    print(f"decode, Skv = {N0 + N1}, num_splits = {num_splits}", flush=True)
    o, lse = ea.attn_fwd_ex(query(1), k, v, scale=1.0, num_splits=num_splits)
    torch.cuda.synchronize()
    check(o, lse, lambda i: N1)


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_past_2_31_elements(kv, causal):
    k, v = kv
    sq = N1  # causal, bottom-right aligned: row i sees keys up to N0 + i
    print(f"prefill, Sq = {sq}, Skv = {N0 + N1}, causal = {causal}", flush=True)
    o, lse = ea.attn_fwd(query(sq), k, v, scale=1.0, causal=causal)
    torch.cuda.synchronize()
    check(o, lse, (lambda i: i + 1) if causal else (lambda i: N1))


def rel_close(t, want, rtol=2e-2):
    """every element of the GPU tensor t within rtol of the scalar want"""
    err = (t.float() - want).abs().max().item()
    assert err <= rtol * abs(want), (err, want)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_past_2_31_elements(kv, causal):
    k, v = kv
    sq = N1  # causal, bottom-right aligned: row i sees keys up to N0 + i
    print(f"backward, Sq = {sq}, Skv = {N0 + N1}, causal = {causal}", flush=True)
    q = query(sq)
    o, lse = ea.attn_fwd(q, k, v, scale=1.0, causal=causal)
    dout = torch.zeros_like(q)
    dout[..., 2] = 1.0
    dq, dk, dv = ea.attn_bwd(q, k, v, o, lse, dout, causal=causal, scale=1.0)
    torch.cuda.synchronize()
    m_rows = [(i + 1) if causal else N1 for i in range(sq)]
    dq0, dk0_first, dk0_second, dv2_first, dv2_second = closed_forms.backward(N0, m_rows, H, 8.0)
    for i in range(sq):
        rel_close(dq[0, :, i, 0], dq0[i])  # every head alike
    assert dq[..., 1:].abs().max().item() == 0.0
    # the first kind of key: one value for all 2^24 rows
    rel_close(dk[0, 0, :N0, 0], dk0_first)
    rel_close(dv[0, 0, :N0, 2], dv2_first)
    # the second kind, past element 2^31
    for t in range(N1):
        rel_close(dk[0, 0, N0 + t, 0], dk0_second[t])
        rel_close(dv[0, 0, N0 + t, 2], dv2_second[t])
    assert dk[..., 1:].abs().max().item() == 0.0
    assert dv[..., :2].abs().max().item() == 0.0
    assert dv[..., 3:].abs().max().item() == 0.0
    del dq, dk, dv, o, lse, dout
    torch.cuda.empty_cache()
