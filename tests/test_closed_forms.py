"""The two-kind closed forms (tests/closed_forms.py) against the fp64 oracle
on a small instance of the same structure, so that the large-tensor GPU
tests compare with a formula that is itself pinned."""

import numpy as np
import pytest

import oracle
from oracle.backward import attention_backward

import closed_forms

N0, N1, D, H, C = 50, 6, 8, 2, 3.0


def inputs():
    skv = N0 + N1
    q = np.zeros((1, H, N1, D))
    q[..., 0] = 1.0
    k = np.zeros((1, 1, skv, D))
    k[0, 0, N0:, 0] = C
    v = np.zeros((1, 1, skv, D))
    v[0, 0, :N0, 1] = 1.0
    v[0, 0, N0:, 2] = 1.0
    do = np.zeros((1, H, N1, D))
    do[..., 2] = 1.0
    return q, k, v, do


@pytest.mark.parametrize("causal", [False, True])
def test_forward_closed_form(causal):
    q, k, v, _ = inputs()
    o, lse = oracle.attention(q, k, v, 1.0, causal=causal)
    for i in range(N1):
        m = i + 1 if causal else N1  # bottom-right: row i sees keys up to N0 + i
        e1, e2, lz = closed_forms.forward(N0, m, C)
        want = np.zeros(D)
        want[1], want[2] = e1, e2
        np.testing.assert_allclose(o[0, :, i, :], np.broadcast_to(want, (H, D)), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, :, i], lz, rtol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_closed_form(causal):
    q, k, v, do = inputs()
    dq, dk, dv = attention_backward(q, k, v, do, 1.0, causal=causal)
    m_rows = [(i + 1) if causal else N1 for i in range(N1)]
    dq0, dk0_first, dk0_second, dv2_first, dv2_second = closed_forms.backward(N0, m_rows, H, C)
    for i in range(N1):
        np.testing.assert_allclose(dq[0, :, i, 0], dq0[i], rtol=1e-12)
    assert np.abs(dq[..., 1:]).max() < 1e-15
    np.testing.assert_allclose(dk[0, 0, :N0, 0], dk0_first, rtol=1e-12)
    np.testing.assert_allclose(dv[0, 0, :N0, 2], dv2_first, rtol=1e-12)
    np.testing.assert_allclose(dk[0, 0, N0:, 0], dk0_second, rtol=1e-12)
    np.testing.assert_allclose(dv[0, 0, N0:, 2], dv2_second, rtol=1e-12)
    assert np.abs(dk[..., 1:]).max() < 1e-15
    assert np.abs(dv[..., [0, 1, 3, 4, 5, 6, 7]]).max() < 1e-15
