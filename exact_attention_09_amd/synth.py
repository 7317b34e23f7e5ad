"""Seeded synthetic inputs for attention workloads.

This module is the one piece shared by the oracle side and the GPU side: it
produces input bytes and nothing else.  It holds none of the attention
arithmetic.

Generator (counter based, so any slice can be produced independently):

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): output i of the stream with seed s is
  ``mix(s + (i + 1) * 0x9E3779B97F4A7C15)`` where ``mix`` is the published
  finaliser (xor-shift 30, multiply, xor-shift 27, multiply, xor-shift 31).
* Uniforms in (0, 1]: ``((x >> 11) + 1) * 2**-53``.
* Normals by the Box-Muller transform (Box and Muller, 1958): uniforms
  ``u[2j], u[2j+1]`` give ``r cos(2 pi u[2j+1])`` and ``r sin(2 pi u[2j+1])``
  with ``r = sqrt(-2 ln u[2j])``, as normals ``2j`` and ``2j+1``.
* The fp64 normals are rounded to fp32 (round to nearest even) and, for bf16
  workloads, from fp32 to bf16 (round to nearest even on the fp32 bit pattern).

Seeds: ``1000 * workload_id + tensor_id`` with tensor ids Q=0, K=1, V=2,
sequence lengths=3, page tables=4, attention sinks=5 (N(0,1) times 2), output gradients=6.

Page tables (paged KV caches): the physical pages are a seeded random
permutation (the order of the stream outputs ``0 .. num_pages-1``, ties broken
by index), dealt out to the sequences in order, so that consecutive logical
blocks of a sequence sit in scattered physical pages.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_LENGTHS, TENSOR_PAGES, TENSOR_SINKS, TENSOR_DOUT = 0, 1, 2, 3, 4, 5, 6

_CHUNK = 1 << 22  # normals per work item


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs ``start .. start+count-1`` of the SplitMix64 stream ``seed``."""
    with np.errstate(over="ignore"):
        idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + idx * GOLDEN_GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniforms(seed: int, start: int, count: int) -> np.ndarray:
    """Uniform doubles in (0, 1] from stream outputs ``start ..``."""
    x = splitmix64(seed, start, count)
    return ((x >> np.uint64(11)) + np.uint64(1)).astype(np.float64) * (2.0 ** -53)


def _normals_f64(seed: int, start: int, count: int) -> np.ndarray:
    """Normals ``start .. start+count-1`` (``start`` even) in fp64."""
    assert start % 2 == 0
    npairs = (count + 1) // 2
    u = uniforms(seed, start, 2 * npairs)
    r = np.sqrt(-2.0 * np.log(u[0::2]))
    t = (2.0 * np.pi) * u[1::2]
    out = np.empty(2 * npairs, dtype=np.float64)
    out[0::2] = r * np.cos(t)
    out[1::2] = r * np.sin(t)
    return out[:count]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_tensor(seed: int, shape, dtype: str) -> np.ndarray:
    """N(0,1) tensor of ``shape``.

    ``dtype`` is ``"f32"`` (returns float32) or ``"bf16"`` (returns the uint16
    bit patterns).  Large tensors are produced chunk by chunk on a thread pool;
    the bytes do not depend on the chunking.
    """
    n = int(np.prod(shape)) if len(shape) else 1
    if dtype == "f32":
        out = np.empty(n, dtype=np.float32)
    elif dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
    else:
        raise ValueError(f"unknown dtype {dtype!r}")

    def work(start: int) -> None:
        cnt = min(_CHUNK, n - start)
        z = _normals_f64(seed, start, cnt).astype(np.float32)
        out[start:start + cnt] = z if dtype == "f32" else f32_to_bf16_bits(z)

    starts = list(range(0, n, _CHUNK))
    if len(starts) <= 1:
        for s in starts:
            work(s)
    else:
        workers = max(1, min(16, os.cpu_count() or 1, len(starts)))
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(work, starts))
    return out.reshape(shape)


def varlen_lengths(seed: int, count: int, lo: int = 256, hi: int = 4096) -> np.ndarray:
    """``count`` lengths ``lo + (u64 mod (hi - lo + 1))`` from stream ``seed``."""
    x = splitmix64(seed, 0, count)
    return (np.uint64(lo) + x % np.uint64(hi - lo + 1)).astype(np.int64)


def cu_seqlens_from_lengths(lengths) -> np.ndarray:
    """int32 prefix sums ``[0, L0, L0+L1, ...]``."""
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    if cu[-1] > np.iinfo(np.int32).max:
        raise ValueError("total length does not fit int32")
    return cu.astype(np.int32)


def page_permutation(seed: int, num_pages: int) -> np.ndarray:
    """A seeded random permutation of ``0 .. num_pages-1`` (int64)."""
    x = splitmix64(seed, 0, num_pages)
    return np.argsort(x, kind="stable").astype(np.int64)


def page_table(seed: int, B: int, max_pages: int, num_pages: int) -> np.ndarray:
    """int32 [B, max_pages] block table: row b holds the physical pages
    ``perm[b * max_pages .. (b + 1) * max_pages)`` of a random permutation."""
    if B * max_pages > num_pages:
        raise ValueError("not enough physical pages for the table")
    perm = page_permutation(seed, num_pages)
    return perm[:B * max_pages].reshape(B, max_pages).astype(np.int32)
