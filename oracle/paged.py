"""Attention over a paged KV cache, in fp64 (TEST INFRASTRUCTURE ONLY).

A paged cache does not change what attention computes, only where the key and
value bytes live ("15-operators-attention", TileLang tutorial, section 4.8
(2)): the cache is cut into fixed-size pages and a per-sequence block table
maps logical block k to a physical page.  The indirection is the one of
"learn-cuda-from-scratch" ch.12, section 12.9.4: logical key t of a sequence
lives in page ``block_table[t // page_size]`` at offset ``t % page_size``.

Cache layout (this library's reading; the tutorial's paged example is a BHSD
kernel): ``k_cache`` and ``v_cache`` are [num_pages, Hkv, page_size, d], so a
page holds ``page_size`` consecutive keys of every KV head, head-major.

The oracle gathers each sequence's keys and values through the table into a
contiguous [Hkv, L, d] array, in logical order, and runs the naive oracle of
``attn_ref.c`` on them.  No blocking, no reordering.
"""

from __future__ import annotations

import numpy as np

from . import attention


def gather(cache, table_row, length: int):
    """Keys (or values) 0 .. length-1 of one sequence as [Hkv, length, d]:
    logical block j (keys j*page_size ..) is physical page table_row[j]."""
    cache = np.asarray(cache)
    num_pages, hkv, page_size, d = cache.shape
    out = np.empty((hkv, length, d), cache.dtype)
    for j in range(-(-length // page_size)):
        page = int(table_row[j])
        if not 0 <= page < num_pages:
            raise ValueError(f"block table entry {page} outside [0, {num_pages})")
        t0 = j * page_size
        t1 = min(length, t0 + page_size)
        out[:, t0:t1, :] = cache[page, :, :t1 - t0, :]
    return out


def paged_attention(q, k_cache, v_cache, block_table, seqlens, scale: float, lib=None):
    """One query row per head attending to its sequence's cached keys.

    q [B, H, d]; k_cache, v_cache [num_pages, Hkv, page_size, d];
    block_table [B, max_pages] (int); seqlens [B] keys per sequence.
    Returns ``(o [B, H, d], lse [B, H])`` in fp64; a sequence without keys
    gives O = 0 and LSE = -inf (the tutorial's section 5.1 (2)).
    """
    q = np.asarray(q, np.float32)
    B, H, d = q.shape
    o = np.empty((B, H, d), np.float64)
    lse = np.empty((B, H), np.float64)
    for b in range(B):
        length = int(seqlens[b])
        k = gather(k_cache, block_table[b], length)
        v = gather(v_cache, block_table[b], length)
        ob, lb = attention(q[b][None, :, None, :], k[None], v[None], scale, False, lib=lib)
        o[b] = ob[0, :, 0, :]
        lse[b] = lb[0, :, 0]
    return o, lse
