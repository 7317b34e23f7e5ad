"""Oracle for the attention forward pass: plain, slow, fp64, on the CPU.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the smoke check and the CPU
baseline leg of the benchmark may import this package.  It shares no code
with the GPU library and never imports it.

* ``attention`` -- naive materialised attention (``attn_ref.c``, built with
  gcc into ``liboracle_attn.so`` beside it).
* ``models`` -- the pages' companion models in fp64: the online-softmax
  recurrence (with per-block state), split-KV partials and their
  log-sum-exp combine, and the HBM traffic model.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_ref.c")
LIB_PATH = os.path.join(_HERE, "liboracle_attn.so")

_lib = None


def build(out: str = LIB_PATH, src: str = _SRC) -> str:
    """Compile ``attn_ref.c`` with gcc (fp-contract off so every product and
    sum rounds as written)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-pthread", src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load(path: str = LIB_PATH):
    global _lib
    if path == LIB_PATH and _lib is not None:
        return _lib
    if not os.path.exists(path):
        build(path)
    lib = ctypes.CDLL(path)
    fn = lib.oracle_attn_f64
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 6 + [ctypes.c_double, ctypes.c_int,
                                                                ctypes.c_void_p, ctypes.c_void_p,
                                                                ctypes.c_int64, ctypes.c_void_p,
                                                                ctypes.c_void_p, ctypes.c_int,
                                                                ctypes.c_int, ctypes.c_void_p]
    if path == LIB_PATH:
        _lib = lib
    return lib


def _f32(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32)


def attention(q, k, v, scale: float, causal: bool = False, cu_seqlens=None, rows=None,
              nthreads: int | None = None, lib=None, window: int = 0, sinks=None):
    """Exact attention in fp64.

    Dense: q [B,H,Sq,d], k/v [B,Hkv,Skv,d].  Varlen (``cu_seqlens`` given, B+1
    int32): q [H,T,d] (or [1,H,T,d]), k/v [Hkv,T,d].  Inputs are any float
    arrays whose values fp32 holds exactly (fp32 or widened bf16).
    ``window`` > 0 keeps the last ``window`` keys up to the (bottom-right)
    diagonal; ``sinks`` ([H] logits) adds exp(sink - m) to each row's
    denominator.

    Returns ``(o, lse)`` as fp64 in the output layout, or for ``rows`` (an
    [n,3] array of (b, h, i)) as [n,d] and [n].
    """
    lib = lib or load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    d = q.shape[-1]
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        B = len(cu) - 1
        H, Hkv = q.shape[-3], k.shape[-3]
        T = int(cu[-1])
        if q.shape[-2] != T or k.shape[-2] != T or v.shape[-2] != T:
            raise ValueError("varlen tensors must have T = cu_seqlens[-1] rows")
        Sq = Skv = T
        out_shape, lse_shape = q.shape, q.shape[:-1]
        cu_ptr = cu.ctypes.data
    else:
        cu = None
        B, H, Sq, _ = q.shape
        Hkv, Skv = k.shape[1], k.shape[2]
        out_shape, lse_shape = q.shape, q.shape[:-1]
        cu_ptr = None
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
        n = rows.shape[0]
        o = np.empty((n, d), np.float64)
        lse = np.empty((n,), np.float64)
        rows_ptr = rows.ctypes.data
    else:
        n = 0
        o = np.empty(out_shape, np.float64)
        lse = np.empty(lse_shape, np.float64)
        rows_ptr = None
    nthreads = nthreads or (os.cpu_count() or 1)
    sk = None if sinks is None else np.ascontiguousarray(sinks, dtype=np.float64).reshape(-1)
    if sk is not None and sk.shape[0] != H:
        raise ValueError("sinks must hold one value per query head")
    st = lib.oracle_attn_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, Hkv, Sq, Skv, d,
                             float(scale), int(bool(causal)), cu_ptr, rows_ptr, n,
                             o.ctypes.data, lse.ctypes.data, int(nthreads), int(window),
                             None if sk is None else sk.ctypes.data)
    if st != 0:
        raise ValueError(f"oracle_attn_f64 failed with status {st}")
    return o, lse
