"""attn_fwd_noalloc: attn_fwd_ex without any device allocation (decode
partials in the library's static per-GPU scratch array).  Called through the
C ABI and compared with attn_fwd_ex, which allocates its workspace, on two
decode calls in a row (the second smaller), an fp32 decode, a prefill call,
and the rejections (oversized partials, a workspace argument)."""

import ctypes
import math

import numpy as np
import pytest

from exact_attention_09_amd import synth
from exact_attention_09_amd.workloads import to_device
from parity import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_09_amd as ea
    ea.load_library()
    return ea


def inputs(seed, B, H, Hkv, Sq, Skv, d, dtype):
    q = to_device(synth.normal_tensor(seed, (B, H, Sq, d), dtype), dtype)
    k = to_device(synth.normal_tensor(seed + 1, (B, Hkv, Skv, d), dtype), dtype)
    v = to_device(synth.normal_tensor(seed + 2, (B, Hkv, Skv, d), dtype), dtype)
    return q, k, v


def noalloc_raw(q, k, v, o, lse, causal, num_splits, dtype_code):
    """attn_fwd_noalloc through the C ABI with raw pointers."""
    import exact_attention_09_amd as ea
    B, H, Sq, d = q.shape
    _, Hkv, Skv, _ = k.shape
    opts = ea.AttnOpts(num_splits, None, 0, 0)
    return ea.raw_call("attn_fwd_noalloc", ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                       ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(o.data_ptr()),
                       ctypes.c_void_p(lse.data_ptr()) if lse is not None else None, B, H, Hkv, Sq, Skv, d,
                       ctypes.c_float(1.0 / math.sqrt(d)), int(causal), None,
                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), dtype_code, ctypes.byref(opts))


def same_as_allocating_call(q, k, v, causal, num_splits, dtype):
    import exact_attention_09_amd as ea
    code = ea.ATTN_BF16 if dtype == "bf16" else ea.ATTN_F32
    o = torch.full_like(q, 7.0)
    lse = torch.full(q.shape[:-1], 9.0, dtype=torch.float32, device="cuda")
    st = noalloc_raw(q, k, v, o, lse, causal, num_splits, code)
    assert st == ea.ATTN_OK, ea.attn_last_error()
    o_ref, lse_ref = ea.attn_fwd_ex(q, k, v, causal=causal, num_splits=num_splits, dtype=code)
    torch.cuda.synchronize()
    err = (o.float() - o_ref.float()).abs().max().item()
    lerr = (lse - lse_ref).abs().max().item()
    say(f"  noalloc vs attn_fwd_ex: max|dO| {err:.3g} max|dLSE| {lerr:.3g}")
    assert err <= (1e-2 if dtype == "bf16" else 1e-5) and lerr <= 1e-3
    # the same kernels run, so the results agree bit for bit
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)


def test_decode_twice_second_smaller():
    say("noalloc decode: B=32 H=32 Hkv=8 Skv=16384 d=128, 16 splits, then B=3 H=8 Hkv=2 Skv=1000 d=64, 5 splits")
    same_as_allocating_call(*inputs(8100, 32, 32, 8, 1, 16384, 128, "bf16"), False, 16, "bf16")
    same_as_allocating_call(*inputs(8110, 3, 8, 2, 1, 1000, 64, "bf16"), False, 5, "bf16")


def test_decode_f32_and_prefill():
    say("noalloc fp32 decode and bf16 prefill")
    same_as_allocating_call(*inputs(8120, 2, 6, 2, 1, 999, 64, "f32"), False, 4, "f32")
    same_as_allocating_call(*inputs(8130, 2, 4, 2, 300, 300, 128, "bf16"), True, 0, "bf16")


def test_rejects_what_does_not_fit():
    import exact_attention_09_amd as ea
    say("noalloc rejections")
    # 64 * 64 * 256 splits * 129 * 4 bytes of partials: more than the scratch
    q, k, v = inputs(8140, 64, 64, 64, 1, 256, 128, "bf16")
    o = torch.full_like(q, 7.0)
    lse = torch.full(q.shape[:-1], 9.0, dtype=torch.float32, device="cuda")
    assert ea.attn_workspace_bytes(64, 64, 128, 256) > ea.ATTN_NOALLOC_SCRATCH_BYTES
    st = noalloc_raw(q, k, v, o, lse, False, 256, ea.ATTN_BF16)
    assert st == ea.ATTN_EINVAL and "scratch" in ea.attn_last_error()
    # a workspace argument is refused
    opts = ea.AttnOpts(4, 0x100, 1 << 20, 0)
    B, H, Sq, d = q.shape
    st = ea.raw_call("attn_fwd_noalloc", ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                     ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
                     B, H, 64, 1, 256, d, ctypes.c_float(0.1), 0, None, None, ea.ATTN_BF16, ctypes.byref(opts))
    assert st == ea.ATTN_EINVAL
    torch.cuda.synchronize()
    assert torch.all(o == 7.0) and torch.all(lse == 9.0)  # nothing was launched
