"""Exact attention forward (FlashAttention) for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI in ``include/attn.h`` (``libattn09.so``
beside this file, built by ``exact_attention_09_amd.build``).  The functions
here only marshal arguments: shapes, pointers, the stream.  Every step of the
attention computation runs in the library's HIP kernels; there is no Python
or CPU fallback.  Calling into the library without it being built raises.

Names mirror the C entry points:

* ``attn_fwd`` (bf16), ``attn_fwd_f32`` (fp32), ``attn_fwd_ex`` (either, with
  split-KV options) take torch tensors on the GPU in BHSD layout and return
  ``(o, lse)``; ``attn_fwd_noalloc`` is ``attn_fwd_ex`` for callers that
  cannot allocate (decode partials in a static per-GPU scratch array);
* ``attn_fwd_window_sink`` is causal attention with a sliding window and/or
  per-head attention sinks;
* ``attn_fwd_layout`` is the general bf16 call: BHSD or BSHD (packed THD for
  varlen) tensors, plus the window and sinks;
* ``attn_bwd`` computes dq, dk, dv from the forward's o and lse (dense or
  packed varlen), ``attn_bwd_window_sink`` the same for the window/sink
  forward (plus the sink gradients), ``attn_bwd_layout`` either of them in
  the layouts of ``attn_fwd_layout``;
* ``flash_attention`` is the forward and backward as one differentiable
  torch op (``attn_fwd_layout`` forward, ``attn_bwd_layout`` gradients);
* ``attn_fwd_paged`` runs split-KV decode over a paged KV cache (block
  table and per-sequence key counts) and returns ``(o, lse)``;
* ``attn_workspace_bytes``, ``attn_decode_num_splits``,
  ``attn_status_string``, ``attn_last_error`` are the helpers.
"""

from __future__ import annotations

import ctypes
import math
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn09.so")

ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_ENOMEM, ATTN_EHIP = range(5)
ATTN_BF16, ATTN_F32 = 0, 1
ATTN_BHSD, ATTN_BSHD = 0, 1
ATTN_MAX_SPLITS = 256

ATTN_NOALLOC_SCRATCH_BYTES = 16 << 20

EXPORTED = ("attn_fwd", "attn_fwd_f32", "attn_fwd_ex", "attn_fwd_noalloc", "attn_fwd_window_sink", "attn_fwd_layout",
            "attn_fwd_paged", "attn_bwd", "attn_bwd_window_sink", "attn_bwd_layout", "attn_bwd_workspace_bytes",
            "attn_workspace_bytes",
            "attn_decode_num_splits", "attn_status_string", "attn_last_error")


ATTN_FLAG_BASIC_PREFILL = 1
ATTN_FLAG_NO_PERSIST = 2


class AttnOpts(ctypes.Structure):
    _fields_ = [("num_splits", ctypes.c_int), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("flags", ctypes.c_uint)]


class AttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"attn: {status_string(status)} ({status}): {detail}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m exact_attention_09_amd.build` "
                           "(there is no fallback path)")
    lib = ctypes.CDLL(path)
    fwd_args = [ctypes.c_void_p] * 4 + [ctypes.c_void_p] + [ctypes.c_int] * 6 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    for name in ("attn_fwd", "attn_fwd_f32"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = fwd_args
    lib.attn_fwd_ex.restype = ctypes.c_int
    lib.attn_fwd_ex.argtypes = fwd_args + [ctypes.c_int, ctypes.POINTER(AttnOpts)]
    lib.attn_fwd_noalloc.restype = ctypes.c_int
    lib.attn_fwd_noalloc.argtypes = fwd_args + [ctypes.c_int, ctypes.POINTER(AttnOpts)]
    lib.attn_fwd_window_sink.restype = ctypes.c_int
    lib.attn_fwd_window_sink.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + [
        ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(AttnOpts)]
    lib.attn_fwd_layout.restype = ctypes.c_int
    lib.attn_fwd_layout.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.POINTER(AttnOpts)]
    lib.attn_fwd_paged.restype = ctypes.c_int
    lib.attn_fwd_paged.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int] * 7 + [
        ctypes.c_float, ctypes.c_void_p, ctypes.POINTER(AttnOpts)]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int] * 6 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(AttnOpts)]
    lib.attn_bwd_window_sink.restype = ctypes.c_int
    lib.attn_bwd_window_sink.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 6 + [
        ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(AttnOpts)]
    lib.attn_bwd_layout.restype = ctypes.c_int
    lib.attn_bwd_layout.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 6 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.POINTER(AttnOpts)]
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_bwd_workspace_bytes.argtypes = [ctypes.c_int] * 3
    lib.attn_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_workspace_bytes.argtypes = [ctypes.c_int] * 4
    lib.attn_decode_num_splits.restype = ctypes.c_int
    lib.attn_decode_num_splits.argtypes = [ctypes.c_int] * 3
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    _lib = lib
    return lib


def status_string(s: int) -> str:
    return load_library().attn_status_string(int(s)).decode()


attn_status_string = status_string


def attn_last_error() -> str:
    return load_library().attn_last_error().decode()


def attn_workspace_bytes(B: int, H: int, d: int, num_splits: int) -> int:
    return int(load_library().attn_workspace_bytes(B, H, d, num_splits))


def attn_decode_num_splits(B: int, Hkv: int, Skv: int) -> int:
    return int(load_library().attn_decode_num_splits(B, Hkv, Skv))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _shapes(q, k, cu_seqlens):
    if cu_seqlens is not None:
        if q.dim() == 3:
            q, k = q.unsqueeze(0), k.unsqueeze(0)
        if q.shape[0] != 1 or k.shape[0] != 1:
            raise ValueError("varlen tensors have batch dimension 1")
        B = cu_seqlens.numel() - 1
        _, H, T, d = q.shape
        _, Hkv, Tk, dk = k.shape
        if Tk != T:
            raise ValueError("varlen q and k must hold the same tokens")
        return B, H, Hkv, T, T, d, dk
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("dense tensors are [B, H, S, d]")
    B, H, Sq, d = q.shape
    Bk, Hkv, Skv, dk = k.shape
    if Bk != B:
        raise ValueError("q and k batch sizes differ")
    return B, H, Hkv, Sq, Skv, d, dk


def attn_fwd_ex(q, k, v, o=None, lse=None, *, causal: bool = False, scale: float | None = None,
                cu_seqlens=None, stream=None, dtype: int | None = None, num_splits: int = 0,
                workspace=None, want_lse: bool = True, flags: int = 0):
    """Run the forward pass through ``attn_fwd_ex``.

    q [B,H,Sq,d], k/v [B,Hkv,Skv,d] (varlen: [1,H,T,d], [1,Hkv,T,d] with an
    int32 ``cu_seqlens`` of B+1 prefix sums on the GPU).  ``o``/``lse`` are
    allocated when not given (``lse`` only if ``want_lse``).  ``scale``
    defaults to 1/sqrt(d).  ``stream`` defaults to torch's current stream.
    ``flags`` are the ``ATTN_FLAG_*`` kernel selection bits.
    Returns ``(o, lse)``.
    """
    import torch
    lib = load_library()
    B, H, Hkv, Sq, Skv, d, dk = _shapes(q, k, cu_seqlens)
    if dk != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must have the shape [.., Hkv, Skv, d] with q's d")
    if dtype is None:
        dtype = {torch.bfloat16: ATTN_BF16, torch.float32: ATTN_F32}.get(q.dtype)
        if dtype is None:
            raise ValueError(f"unsupported dtype {q.dtype}")
    want = torch.bfloat16 if dtype == ATTN_BF16 else torch.float32
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != want or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous {want} tensor on the GPU")
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda):
        raise ValueError("cu_seqlens must be an int32 tensor on the GPU")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    opts = AttnOpts(int(num_splits), workspace.data_ptr() if workspace is not None else None,
                    workspace.numel() * workspace.element_size() if workspace is not None else 0, int(flags))
    st = lib.attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, Sq, Skv, d,
                         float(scale), int(bool(causal)), _ptr(cu_seqlens), ctypes.c_void_p(stream),
                         int(dtype), ctypes.byref(opts))
    if st != ATTN_OK:
        raise AttnError(st, attn_last_error())
    return o, lse


def attn_fwd_noalloc(q, k, v, o, lse, *, causal: bool = False, scale: float | None = None, cu_seqlens=None,
                     stream=None, dtype: int | None = None, num_splits: int = 0, flags: int = 0):
    """``attn_fwd_ex`` through ``attn_fwd_noalloc``: the library allocates
    nothing (decode partials in its static per-GPU scratch array).  The
    caller passes the outputs ``o`` and ``lse`` (``lse`` may be None)."""
    import torch
    lib = load_library()
    B, H, Hkv, Sq, Skv, d, dk = _shapes(q, k, cu_seqlens)
    if dk != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must have the shape [.., Hkv, Skv, d] with q's d")
    if dtype is None:
        dtype = {torch.bfloat16: ATTN_BF16, torch.float32: ATTN_F32}.get(q.dtype)
        if dtype is None:
            raise ValueError(f"unsupported dtype {q.dtype}")
    want = torch.bfloat16 if dtype == ATTN_BF16 else torch.float32
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if t.dtype != want or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous {want} tensor on the GPU")
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda):
        raise ValueError("cu_seqlens must be an int32 tensor on the GPU")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    opts = AttnOpts(int(num_splits), None, 0, int(flags))
    st = lib.attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, Sq, Skv, d,
                              float(scale), int(bool(causal)), _ptr(cu_seqlens), ctypes.c_void_p(stream),
                              int(dtype), ctypes.byref(opts))
    if st != ATTN_OK:
        raise AttnError(st, attn_last_error())
    return o, lse


def attn_fwd_window_sink(q, k, v, o=None, lse=None, *, window: int = 0, sinks=None, scale: float | None = None,
                         cu_seqlens=None, stream=None, num_splits: int = 0, workspace=None, want_lse: bool = True):
    """Causal bf16 attention with a sliding window (``window`` > 0 keys up to
    the diagonal) and/or per-head sinks (``sinks``: fp32 [H] on the GPU)
    through ``attn_fwd_window_sink``.  Shapes as for ``attn_fwd_ex``.
    Returns ``(o, lse)``."""
    import torch
    lib = load_library()
    B, H, Hkv, Sq, Skv, d, dk = _shapes(q, k, cu_seqlens)
    if dk != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must have the shape [.., Hkv, Skv, d] with q's d")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous bfloat16 tensor on the GPU")
    if sinks is not None and (sinks.dtype != torch.float32 or sinks.numel() != H or not sinks.is_cuda
                              or not sinks.is_contiguous()):
        raise ValueError("sinks must be a contiguous float32 tensor of H values on the GPU")
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda):
        raise ValueError("cu_seqlens must be an int32 tensor on the GPU")
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    opts = AttnOpts(int(num_splits), workspace.data_ptr() if workspace is not None else None,
                    workspace.numel() * workspace.element_size() if workspace is not None else 0)
    st = lib.attn_fwd_window_sink(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, Sq, Skv, d,
                                  float(scale), _ptr(cu_seqlens), int(window), _ptr(sinks),
                                  ctypes.c_void_p(stream), ctypes.byref(opts))
    if st != ATTN_OK:
        raise AttnError(st, attn_last_error())
    return o, lse


def attn_fwd_layout(q, k, v, o=None, lse=None, *, layout: str = "bshd", causal: bool = False, window: int = 0,
                    sinks=None, scale: float | None = None, cu_seqlens=None, stream=None, num_splits: int = 0,
                    workspace=None, want_lse: bool = True):
    """bf16 forward through ``attn_fwd_layout``.

    ``layout="bshd"``: q [B,Sq,H,d], k/v [B,Skv,Hkv,d]; with ``cu_seqlens``
    the packed-token form q [T,H,d], k/v [T,Hkv,d].  ``layout="bhsd"``: the
    shapes of ``attn_fwd_ex``.  lse is [B,H,Sq] ([H,T] varlen) either way.
    ``window``/``sinks`` as for ``attn_fwd_window_sink`` (need ``causal``).
    Returns ``(o, lse)``.
    """
    import torch
    lib = load_library()
    lay = {"bhsd": ATTN_BHSD, "bshd": ATTN_BSHD}[layout]
    if lay == ATTN_BSHD:
        if cu_seqlens is not None:
            if q.dim() != 3 or k.dim() != 3:
                raise ValueError("packed varlen tensors are [T, H, d]")
            T, H, d = q.shape
            Tk, Hkv, dk = k.shape
            if Tk != T:
                raise ValueError("varlen q and k must hold the same tokens")
            B, Sq, Skv = cu_seqlens.numel() - 1, T, T
            lse_shape = (H, T)
        else:
            if q.dim() != 4 or k.dim() != 4:
                raise ValueError("BSHD tensors are [B, S, H, d]")
            B, Sq, H, d = q.shape
            Bk, Skv, Hkv, dk = k.shape
            if Bk != B:
                raise ValueError("q and k batch sizes differ")
            lse_shape = (B, H, Sq)
    else:
        B, H, Hkv, Sq, Skv, d, dk = _shapes(q, k, cu_seqlens)
        lse_shape = q.shape[:-1]
    if dk != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must have the same shape, with q's d")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous bfloat16 tensor on the GPU")
    if sinks is not None and (sinks.dtype != torch.float32 or sinks.numel() != H or not sinks.is_cuda
                              or not sinks.is_contiguous()):
        raise ValueError("sinks must be a contiguous float32 tensor of H values on the GPU")
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda):
        raise ValueError("cu_seqlens must be an int32 tensor on the GPU")
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    opts = AttnOpts(int(num_splits), workspace.data_ptr() if workspace is not None else None,
                    workspace.numel() * workspace.element_size() if workspace is not None else 0)
    st = lib.attn_fwd_layout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, Sq, Skv, d, float(scale),
                             int(bool(causal)), _ptr(cu_seqlens), lay, int(window), _ptr(sinks),
                             ctypes.c_void_p(stream), ctypes.byref(opts))
    if st != ATTN_OK:
        raise AttnError(st, attn_last_error())
    return o, lse


def attn_fwd_paged(q, k_cache, v_cache, block_table, seqlens_k, o=None, lse=None, *,
                   scale: float | None = None, num_splits: int = 0, workspace=None, stream=None,
                   want_lse: bool = True):
    """Split-KV decode over a paged KV cache through ``attn_fwd_paged``.

    q [B,H,1,d] (or [B,H,d]) bf16; k_cache/v_cache [num_pages,Hkv,page_size,d]
    bf16; block_table [B,max_pages] int32 and seqlens_k [B] int32 on the GPU.
    Returns ``(o, lse)`` with o shaped like q and lse [B,H] (or None).
    """
    import torch
    lib = load_library()
    if q.dim() == 3:
        q = q.unsqueeze(2)
    if q.dim() != 4 or q.shape[2] != 1:
        raise ValueError("q is [B, H, 1, d]")
    B, H, _, d = q.shape
    if k_cache.dim() != 4 or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache and v_cache are [num_pages, Hkv, page_size, d]")
    num_pages, Hkv, page_size, dk = k_cache.shape
    if dk != d:
        raise ValueError("cache head dim differs from q's")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous bfloat16 tensor on the GPU")
    for name, t in (("block_table", block_table), ("seqlens_k", seqlens_k)):
        if t.dtype != torch.int32 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous int32 tensor on the GPU")
    if block_table.dim() != 2 or block_table.shape[0] != B or seqlens_k.numel() != B:
        raise ValueError("block_table is [B, max_pages] and seqlens_k is [B]")
    max_pages = block_table.shape[1]
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    opts = AttnOpts(int(num_splits), workspace.data_ptr() if workspace is not None else None,
                    workspace.numel() * workspace.element_size() if workspace is not None else 0)
    st = lib.attn_fwd_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), _ptr(block_table),
                            _ptr(seqlens_k), B, H, Hkv, d, page_size, max_pages, num_pages, float(scale),
                            ctypes.c_void_p(stream), ctypes.byref(opts))
    if st != ATTN_OK:
        raise AttnError(st, attn_last_error())
    return o, lse


def attn_bwd(q, k, v, o, lse, dout, *, causal: bool = False, scale: float | None = None, cu_seqlens=None,
             dq=None, dk=None, dv=None, stream=None, workspace=None):
    """Gradients through ``attn_bwd``: q [B,H,Sq,d], k/v [B,Hkv,Skv,d], the
    forward's o and lse, and dout [B,H,Sq,d] (bf16 on the GPU); with
    ``cu_seqlens`` (int32 on the GPU) the packed varlen layout of
    ``attn_fwd_ex``.  Returns ``(dq, dk, dv)``."""
    import torch
    lib = load_library()
    B, H, Hkv, Sq, Skv, d, dk_ = _shapes(q, k, cu_seqlens)
    if dk_ != d or tuple(v.shape) != tuple(k.shape) or tuple(o.shape) != tuple(q.shape) \
            or tuple(dout.shape) != tuple(q.shape) or tuple(lse.shape) != tuple(q.shape[:-1]):
        raise ValueError("shapes: q, o, dout [B,H,Sq,d]; k, v [B,Hkv,Skv,d]; lse [B,H,Sq]")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous bfloat16 tensor on the GPU")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or not lse.is_cuda:
        raise ValueError("lse must be a contiguous float32 tensor on the GPU")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    opts = AttnOpts(0, workspace.data_ptr() if workspace is not None else None,
                    workspace.numel() * workspace.element_size() if workspace is not None else 0)
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda):
        raise ValueError("cu_seqlens must be an int32 tensor on the GPU")
    st = lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                      B, H, Hkv, Sq, Skv, d, float(scale), int(bool(causal)),
                      _ptr(cu_seqlens) if cu_seqlens is not None else None, ctypes.c_void_p(stream),
                      ctypes.byref(opts))
    if st != ATTN_OK:
        raise AttnError(st, attn_last_error())
    return dq, dk, dv


def attn_bwd_window_sink(q, k, v, o, lse, dout, *, window: int = 0, sinks=None, scale: float | None = None,
                         cu_seqlens=None, dq=None, dk=None, dv=None, dsinks=None, stream=None, workspace=None):
    """Gradients of ``attn_fwd_window_sink`` (causal, sliding ``window``,
    per-head ``sinks`` fp32 [H]) through ``attn_bwd_window_sink``; shapes as
    for ``attn_bwd``.  Returns ``(dq, dk, dv, dsinks)`` (``dsinks`` None
    without sinks)."""
    import torch
    lib = load_library()
    B, H, Hkv, Sq, Skv, d, dk_ = _shapes(q, k, cu_seqlens)
    if dk_ != d or tuple(v.shape) != tuple(k.shape) or tuple(o.shape) != tuple(q.shape) \
            or tuple(dout.shape) != tuple(q.shape) or tuple(lse.shape) != tuple(q.shape[:-1]):
        raise ValueError("shapes: q, o, dout [B,H,Sq,d]; k, v [B,Hkv,Skv,d]; lse [B,H,Sq]")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous bfloat16 tensor on the GPU")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or not lse.is_cuda:
        raise ValueError("lse must be a contiguous float32 tensor on the GPU")
    if sinks is not None and (sinks.dtype != torch.float32 or not sinks.is_cuda or sinks.numel() != H):
        raise ValueError("sinks must be a float32 tensor of H values on the GPU")
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda):
        raise ValueError("cu_seqlens must be an int32 tensor on the GPU")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if sinks is not None and dsinks is None:
        dsinks = torch.empty(H, dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    opts = AttnOpts(0, workspace.data_ptr() if workspace is not None else None,
                    workspace.numel() * workspace.element_size() if workspace is not None else 0)
    st = lib.attn_bwd_window_sink(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                                  _ptr(dv), _ptr(dsinks) if sinks is not None else None, B, H, Hkv, Sq, Skv, d,
                                  float(scale), _ptr(cu_seqlens), int(window), _ptr(sinks), ctypes.c_void_p(stream),
                                  ctypes.byref(opts))
    if st != ATTN_OK:
        raise AttnError(st, attn_last_error())
    return dq, dk, dv, (dsinks if sinks is not None else None)


def attn_bwd_layout(q, k, v, o, lse, dout, *, layout: str = "bshd", causal: bool = False, window: int = 0,
                    sinks=None, scale: float | None = None, cu_seqlens=None, dq=None, dk=None, dv=None, dsinks=None,
                    stream=None, workspace=None):
    """Gradients through ``attn_bwd_layout``, the inverse of
    ``attn_fwd_layout``: the same layouts and shapes (``layout="bshd"``: q,
    o, dout [B,Sq,H,d], k, v [B,Skv,Hkv,d], packed [T,H,d] / [T,Hkv,d] with
    ``cu_seqlens``; ``layout="bhsd"``: those of ``attn_bwd``), lse as the
    forward wrote it, ``window``/``sinks`` as for ``attn_bwd_window_sink``
    (need ``causal``).  Returns ``(dq, dk, dv, dsinks)`` (``dsinks`` None
    without sinks)."""
    import torch
    lib = load_library()
    lay = {"bhsd": ATTN_BHSD, "bshd": ATTN_BSHD}[layout]
    if lay == ATTN_BSHD:
        if cu_seqlens is not None:
            if q.dim() != 3 or k.dim() != 3:
                raise ValueError("packed varlen tensors are [T, H, d]")
            T, H, d = q.shape
            Tk, Hkv, dk_ = k.shape
            if Tk != T:
                raise ValueError("varlen q and k must hold the same tokens")
            B, Sq, Skv = cu_seqlens.numel() - 1, T, T
            lse_shape = (H, T)
        else:
            if q.dim() != 4 or k.dim() != 4:
                raise ValueError("BSHD tensors are [B, S, H, d]")
            B, Sq, H, d = q.shape
            Bk, Skv, Hkv, dk_ = k.shape
            if Bk != B:
                raise ValueError("q and k batch sizes differ")
            lse_shape = (B, H, Sq)
    else:
        B, H, Hkv, Sq, Skv, d, dk_ = _shapes(q, k, cu_seqlens)
        lse_shape = tuple(q.shape[:-1])
    if dk_ != d or tuple(v.shape) != tuple(k.shape) or tuple(o.shape) != tuple(q.shape) \
            or tuple(dout.shape) != tuple(q.shape) or tuple(lse.shape) != tuple(lse_shape):
        raise ValueError("shapes: o and dout as q, v as k, lse [B,H,Sq] ([H,T] varlen)")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous bfloat16 tensor on the GPU")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or not lse.is_cuda:
        raise ValueError("lse must be a contiguous float32 tensor on the GPU")
    if sinks is not None and (sinks.dtype != torch.float32 or not sinks.is_cuda or sinks.numel() != H
                              or not sinks.is_contiguous()):
        raise ValueError("sinks must be a contiguous float32 tensor of H values on the GPU")
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda):
        raise ValueError("cu_seqlens must be an int32 tensor on the GPU")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if sinks is not None and dsinks is None:
        dsinks = torch.empty(H, dtype=torch.float32, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    opts = AttnOpts(0, workspace.data_ptr() if workspace is not None else None,
                    workspace.numel() * workspace.element_size() if workspace is not None else 0)
    st = lib.attn_bwd_layout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                             _ptr(dsinks) if sinks is not None else None, B, H, Hkv, Sq, Skv, d, float(scale),
                             int(bool(causal)), _ptr(cu_seqlens), lay, int(window), _ptr(sinks),
                             ctypes.c_void_p(stream), ctypes.byref(opts))
    if st != ATTN_OK:
        raise AttnError(st, attn_last_error())
    return dq, dk, dv, (dsinks if sinks is not None else None)


def attn_bwd_workspace_bytes(B: int, H: int, Sq: int) -> int:
    return int(load_library().attn_bwd_workspace_bytes(B, H, Sq))


def attn_fwd(q, k, v, o=None, lse=None, **kw):
    """bf16 forward (``attn_fwd``); see ``attn_fwd_ex`` for the arguments."""
    return attn_fwd_ex(q, k, v, o, lse, dtype=ATTN_BF16, **kw)


def attn_fwd_f32(q, k, v, o=None, lse=None, **kw):
    """fp32 forward (``attn_fwd_f32``); see ``attn_fwd_ex`` for the arguments."""
    return attn_fwd_ex(q, k, v, o, lse, dtype=ATTN_F32, **kw)


def raw_call(name: str, *args):
    """Call a C entry point with already-marshalled arguments (used by the
    ABI tests to drive the validation paths with raw pointers)."""
    return getattr(load_library(), name)(*args)


_FLASH_FN = None


def _flash_function():
    """The torch.autograd.Function behind ``flash_attention`` (built on first
    use, so that importing the package does not import torch)."""
    global _FLASH_FN
    if _FLASH_FN is not None:
        return _FLASH_FN
    import torch

    class FlashAttention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, sinks, causal, window, scale, cu_seqlens, layout):
            o, lse = attn_fwd_layout(q, k, v, layout=layout, causal=causal, window=window, sinks=sinks, scale=scale,
                                     cu_seqlens=cu_seqlens)
            ctx.save_for_backward(q, k, v, o, lse, sinks, cu_seqlens)
            ctx.args = (causal, window, scale, layout)
            ctx.mark_non_differentiable(lse)
            return o, lse

        @staticmethod
        def backward(ctx, do, _dlse):
            q, k, v, o, lse, sinks, cu_seqlens = ctx.saved_tensors
            causal, window, scale, layout = ctx.args
            dq, dk, dv, ds = attn_bwd_layout(q, k, v, o, lse, do.to(torch.bfloat16).contiguous(), layout=layout,
                                             causal=causal, window=window, sinks=sinks, scale=scale,
                                             cu_seqlens=cu_seqlens)
            if sinks is None or not ctx.needs_input_grad[3]:
                ds = None
            return dq, dk, dv, ds, None, None, None, None, None

    _FLASH_FN = FlashAttention
    return _FLASH_FN


def flash_attention(q, k, v, *, causal: bool = False, window: int = 0, sinks=None, scale: float | None = None,
                    cu_seqlens=None, layout: str = "bshd", return_lse: bool = False):
    """Exact attention as a differentiable torch op: ``attn_fwd_layout`` in
    the forward, ``attn_bwd_layout`` for the gradients of q, k, v (and of
    ``sinks`` when it requires them).  Tensors and options as for
    ``attn_fwd_layout`` (bf16 q, k, v on the GPU, contiguous; ``layout``
    "bshd" [B,S,H,d] or "bhsd" [B,H,S,d]; packed [T,H,d] with ``cu_seqlens``).
    Returns o, or ``(o, lse)`` with ``return_lse`` (lse carries no gradient).
    """
    o, lse = _flash_function().apply(q, k, v, sinks, bool(causal), int(window), scale, cu_seqlens, layout)
    return (o, lse) if return_lse else o
