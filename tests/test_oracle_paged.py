"""Pins for the paged-KV oracle (``oracle/paged.py``), on the CPU.

The tutorial's section 4.8 (2) says a paged cache changes where the key and
value bytes come from, not the mathematics.  So:

* a cache whose pages hold a contiguous K/V in order gives exactly the dense
  oracle's result;
* shuffling the physical pages (and the table with them) changes nothing,
  bit for bit;
* a brute-force walk over (page, offset) pairs written from the CUDA course's
  address formula (section 12.9.4) reproduces the gathered keys;
* closed forms: a sequence with no key gives O = 0, LSE = -inf; with one key
  O = v_0 and LSE = scale * q . k_0.

Plausible mistakes planted in copies of the gather (offset and page index
swapped, the head-major page read as token-major, an off-by-one page, the
length ignored) each trip at least one of these pins.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import paged
from exact_attention_09_amd import synth


def _dense_to_pages(k, page_size, perm):
    """Store dense k [B, Hkv, S, d] (S a multiple of page_size) in pages:
    logical block p of sequence b goes to physical page perm[b * P + p]."""
    B, Hkv, S, d = k.shape
    P = S // page_size
    cache = np.zeros((B * P + 3, Hkv, page_size, d), k.dtype)  # 3 unused pages
    table = np.zeros((B, P), np.int32)
    for b in range(B):
        for p in range(P):
            phys = int(perm[b * P + p])
            cache[phys] = k[b, :, p * page_size:(p + 1) * page_size, :]
            table[b, p] = phys
    return cache, table


def _case(seed=7, B=3, H=4, Hkv=2, S=64, d=16, page_size=16, shuffle=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, d)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, S, d)).astype(np.float32)
    n = B * (S // page_size) + 3
    perm = synth.page_permutation(seed, n) if shuffle else np.arange(n)
    kc, table = _dense_to_pages(k, page_size, perm)
    vc, _ = _dense_to_pages(v, page_size, perm)
    return q, k, v, kc, vc, table


def pin_paged_is_dense(gather_fn):
    q, k, v, kc, vc, table = _case()
    B, H, d = q.shape
    S = k.shape[2]
    lens = np.array([S, S - 5, 17])
    for b in range(B):
        kk = gather_fn(kc, table[b], int(lens[b]))
        vv = gather_fn(vc, table[b], int(lens[b]))
        assert kk.shape == (k.shape[1], lens[b], d)
        assert np.array_equal(kk, k[b, :, :lens[b]]), "gathered keys differ from the dense keys"
        assert np.array_equal(vv, v[b, :, :lens[b]]), "gathered values differ from the dense values"


def pin_brute_force_walk(gather_fn):
    """Key t of sequence b read as K_blocks + block_id * (page_size * d) +
    (t % page_size) * d inside KV head h's slice of the page."""
    q, k, v, kc, vc, table = _case(seed=11, B=2, S=48, page_size=16)
    num_pages, Hkv, ps, d = kc.shape
    flat = kc.reshape(-1)
    for b in range(2):
        got = gather_fn(kc, table[b], 40)
        for h in range(Hkv):
            for t in range(40):
                block_id = int(table[b][t // ps])
                base = (block_id * Hkv + h) * ps * d + (t % ps) * d
                assert np.array_equal(got[h, t], flat[base:base + d]), f"key {t} of head {h} misread"


def test_paged_equals_dense_attention():
    q, k, v, kc, vc, table = _case()
    lens = np.array([64, 59, 17])
    o, lse = paged.paged_attention(q, kc, vc, table, lens, 0.25)
    for b in range(3):
        L = int(lens[b])
        od, ld = oracle.attention(q[b][None, :, None, :], k[b:b + 1, :, :L], v[b:b + 1, :, :L], 0.25)
        assert np.array_equal(o[b], od[0, :, 0]) and np.array_equal(lse[b], ld[0, :, 0])


def test_page_shuffle_changes_nothing():
    a = _case(seed=3, shuffle=False)
    b = _case(seed=3, shuffle=True)
    lens = np.array([64, 33, 1])
    oa, la = paged.paged_attention(a[0], a[3], a[4], a[5], lens, 0.3)
    ob, lb = paged.paged_attention(b[0], b[3], b[4], b[5], lens, 0.3)
    assert not np.array_equal(a[5], b[5])
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_paged_pins_hold():
    pin_paged_is_dense(paged.gather)
    pin_brute_force_walk(paged.gather)


def test_paged_closed_forms():
    q, k, v, kc, vc, table = _case(seed=5)
    scale = 0.125
    o, lse = paged.paged_attention(q, kc, vc, table, np.array([0, 1, 0]), scale)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0]))
    H, Hkv = q.shape[1], k.shape[1]
    for h in range(H):
        kvh = h // (H // Hkv)
        np.testing.assert_allclose(o[1, h], v[1, kvh, 0], rtol=0, atol=1e-12)
        assert abs(lse[1, h] - scale * float(np.dot(q[1, h].astype(np.float64), k[1, kvh, 0]))) < 1e-9


def test_paged_table_out_of_range_raises():
    q, k, v, kc, vc, table = _case(seed=9)
    bad = table.copy()
    bad[0, 0] = kc.shape[0]
    with pytest.raises(ValueError):
        paged.paged_attention(q, kc, vc, bad, np.array([5, 5, 5]), 0.2)


def _mutant_swap(cache, row, length):
    num_pages, hkv, ps, d = cache.shape
    out = np.empty((hkv, length, d), cache.dtype)
    for t in range(length):
        page = int(row[min(t % ps, len(row) - 1)])
        out[:, t, :] = cache[page, :, min(t // ps, ps - 1), :]
    return out


def _mutant_token_major(cache, row, length):
    num_pages, hkv, ps, d = cache.shape
    view = cache.reshape(num_pages, ps, hkv, d)  # page read as [token, head, d]
    out = np.empty((hkv, length, d), cache.dtype)
    for t in range(length):
        out[:, t, :] = view[int(row[t // ps]), t % ps, :, :]
    return out


def _mutant_page_off_by_one(cache, row, length):
    num_pages, hkv, ps, d = cache.shape
    out = np.empty((hkv, length, d), cache.dtype)
    for t in range(length):
        out[:, t, :] = cache[int(row[min(t // ps + 1, len(row) - 1)]), :, t % ps, :]
    return out


def _mutant_ignores_length(cache, row, length):
    num_pages, hkv, ps, d = cache.shape
    full = len(row) * ps
    return paged.gather(cache, row, full)


@pytest.mark.parametrize("mutant", [_mutant_swap, _mutant_token_major, _mutant_page_off_by_one,
                                    _mutant_ignores_length])
def test_pins_catch_gather_mutants(mutant):
    caught = []
    for pin in (pin_paged_is_dense, pin_brute_force_walk):
        try:
            pin(mutant)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches {mutant.__name__}"
