"""The companion models (online recurrence, split-KV combine, traffic model)
against the pages' printed numbers, and against the naive oracle."""

import math

import numpy as np
import pytest

import oracle
from oracle import models
from pins import assert_printed, golden, rng_tensor


def _identity_values(n):
    return np.eye(n)


def test_four_scores_trace():
    """LLM course ch.19, section 19.5: two blocks [1,2], [3,4]."""
    g = golden()["four_scores"]
    blocks = g["blocks"]
    n = sum(len(b) for b in blocks)
    eye = _identity_values(n)
    vb, j = [], 0
    for b in blocks:
        vb.append(eye[j:j + len(b)]); j += len(b)
    o, lse, trace = models.online_row(blocks, vb)
    for t, m in zip(trace, g["m_after_block"]):
        assert t["m"] == float(m)
    assert_printed(trace[0]["ell"], g["ell_after_block1"], "l after block 1")
    assert_printed(trace[0]["ell"] * trace[1]["alpha"], g["ell_block1_rescaled"], "rescaled l")
    assert_printed(trace[1]["ell"], g["ell_final"], "final l")
    for jj, w in enumerate(g["weights"]):
        assert_printed(o[jj], w, f"weight {jj}")
    for jj, e in enumerate(g["exp_values"]):
        assert_printed(math.exp(blocks[jj // 2][jj % 2]), e, "exp value")
    assert_printed(math.exp(lse), g["exp_sum"], "sum of exp")


def test_three_blocks_trace():
    """TileLang forward blog, section 2.3: blocks {1}, {2}, {3} from m = -inf."""
    g = golden()["three_blocks"]
    blocks = g["blocks"]
    eye = _identity_values(3)
    o, lse, trace = models.online_row(blocks, [eye[i:i + 1] for i in range(3)])
    for t, m, a, l, c in zip(trace, g["m_after_block"], g["alpha"], g["ell"], g["v1_coefficient"]):
        assert t["m"] == float(m)
        assert_printed(t["alpha"], a, "alpha")
        assert_printed(t["ell"], l, "l")
        assert_printed(t["acc"][0], c, "v1 coefficient")
    for jj, w in enumerate(g["weights"]):
        assert_printed(o[jj], w, f"weight {jj}")


def test_traffic_model():
    """TileLang tutorial ch.15, section 1: N = 8192, 64 query blocks."""
    g = golden()["traffic_model"]
    N, d, bm = g["N"], g["d"], g["block_m"]
    assert -(-N // bm) == g["q_blocks"]
    naive = models.traffic_naive(N, N, d)
    fused = models.traffic_fused(N, N, d, bm)
    assert naive == g["naive_elements"]
    assert fused == g["fused_elements"]
    assert models.traffic_sp_share(N, N) == g["sp_elements"]
    assert naive - models.traffic_sp_share(N, N) == g["qkvo_elements"]
    assert_printed(100.0 * g["qkvo_elements"] / naive, g["qkvo_share_percent"], "Q/K/V/O share")
    assert_printed(naive / fused, g["ratio"], "naive / fused")


def test_traffic_model_decode_is_about_one():
    """Same page: at Sq = 1 the fused form saves almost nothing (the page says
    1x; the model gives 1 + 2/d up to O(1/N))."""
    for d in (64, 128):
        r = models.traffic_naive(1, 16384, d) / models.traffic_fused(1, 16384, d, 128)
        assert 1.0 < r <= 1.0 + 2.0 / d + 1e-9


@pytest.mark.parametrize("shape", [(16, 16, 8), (128, 128, 64), (5, 9, 8), (9, 4, 8)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block_n", [1, 2, 3, 4, 64])
def test_online_equals_naive(shape, causal, block_n, oracle_lib):
    """TileLang tutorial section 2.4: the recurrence gives exactly the naive
    result (fp64: within 1e-12, the bound the LLM course's simulator uses)."""
    sq, skv, d = shape
    rng = np.random.default_rng(sq * 1000 + skv + block_n)
    q = rng_tensor(rng, (sq, d)); k = rng_tensor(rng, (skv, d)); v = rng_tensor(rng, (skv, d))
    scale = 1.0 / math.sqrt(d)
    o, lse = models.online_attention(q, k, v, scale, block_n, causal)
    o_ref, lse_ref = oracle.attention(q[None, None], k[None, None], v[None, None], scale, causal,
                                      lib=oracle_lib)
    assert np.abs(o - o_ref[0, 0]).max() <= 1e-12
    fin = np.isfinite(lse_ref[0, 0])
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.abs(lse[fin] - lse_ref[0, 0][fin]).max(initial=0.0) <= 1e-12


@pytest.mark.parametrize("num_splits,round_to", [(1, 1), (2, 1), (3, 1), (16, 1), (7, 64), (40, 1)])
def test_split_combine_equals_unsplit(num_splits, round_to, oracle_lib):
    """TileLang tutorial section 5.4: partials normalised per split, combined
    with weights l_s / sum l, give the unsplit result (some splits may be
    empty when the split count exceeds the keys or rounding leaves a tail)."""
    rng = np.random.default_rng(num_splits)
    skv, d = 37, 16
    q = rng_tensor(rng, (4, d)); k = rng_tensor(rng, (skv, d)); v = rng_tensor(rng, (skv, d))
    scale = 0.25
    parts = models.split_partials(q, k, v, scale, num_splits, round_to)
    o, lse = models.split_combine(parts)
    o_ref, lse_ref = oracle.attention(q[None, None], k[None, None], v[None, None], scale, lib=oracle_lib)
    assert np.abs(o - o_ref[0, 0]).max() <= 1e-12
    assert np.abs(lse - lse_ref[0, 0]).max() <= 1e-12


def test_split_single_is_identity():
    rng = np.random.default_rng(3)
    q = rng_tensor(rng, (2, 8)); k = rng_tensor(rng, (10, 8)); v = rng_tensor(rng, (10, 8))
    parts = models.split_partials(q, k, v, 0.5, 1)
    o, lse = models.split_combine(parts)
    assert np.array_equal(o, parts[0][0])
    assert np.abs(lse - parts[0][1] * models.LN2).max() <= 1e-15


def test_split_worked_example_two_blocks():
    """The four-score example split in two halves is the page's two-block
    computation: combined weights equal the printed ones."""
    g = golden()["four_scores"]
    scores = np.array([x for b in g["blocks"] for x in b], np.float64)
    q = np.array([[1.0]])
    k = scores[:, None]
    v = np.eye(4)
    parts = models.split_partials(q, k, v, 1.0, 2)
    o, lse = models.split_combine(parts)
    for j, w in enumerate(g["weights"]):
        assert_printed(o[0, j], w, f"weight {j}")
    assert_printed(math.exp(lse[0]), g["exp_sum"], "sum of exp")


def test_split_bounds_partition():
    for skv in (0, 1, 63, 64, 1000, 16384):
        for ns in (1, 2, 3, 16, 17):
            for r in (1, 64):
                b = models.split_bounds(skv, ns, r)
                assert len(b) == ns and b[0][0] == 0 and b[-1][1] == skv
                for (a0, b0), (a1, b1) in zip(b, b[1:]):
                    assert b0 == a1 and a0 <= b0
