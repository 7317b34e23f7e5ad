"""flash_attention, the differentiable torch op over attn_fwd_layout and
attn_bwd_layout: its forward output and the gradients torch's autograd
computes through it equal the direct C-ABI calls bit for bit (the op only
marshals arguments; the backward parity against the fp64 oracle is tested
for those calls in test_parity_bwd_gpu.py and test_parity_bwd_layout_gpu.py)."""

import zlib

import numpy as np
import pytest

from exact_attention_09_amd import synth
from exact_attention_09_amd.workloads import to_device
from parity import say

torch = pytest.importorskip("torch")


def test_flash_attention_rejects_host_tensors():
    """Validation happens in the binding before any GPU call (runs without a
    GPU)."""
    import exact_attention_09_amd as ea
    x = torch.zeros((1, 8, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ea.flash_attention(x, x, x)


CASES = [
    # (layout, B, H, Hkv, Sq, Skv, d, causal, window, with_sinks, lengths)
    ("bshd", 2, 4, 2, 200, 200, 128, True, 0, False, None),
    ("bhsd", 1, 8, 2, 256, 300, 64, False, 0, False, None),
    ("bshd", 1, 4, 4, 300, 300, 128, True, 64, True, None),
    ("bshd", 0, 4, 2, 0, 0, 128, True, 0, False, (130, 1, 300, 77)),    # packed [T, H, d]
    ("bhsd", 0, 4, 2, 0, 0, 64, True, 0, False, (64, 257, 0, 129)),     # packed [1, H, T, d]
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c[:10])) + ("-varlen" if c[10] else ""))
def test_flash_attention_autograd_equals_direct_calls(case):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_09_amd as ea
    layout, B, H, Hkv, Sq, Skv, d, causal, window, with_sinks, lengths = case
    say(f"flash_attention autograd {case}")
    seed = zlib.crc32(repr(case).encode()) % 10000
    if lengths is not None:
        T = sum(lengths)
        shapes = ((1, H, T, d), (1, Hkv, T, d))
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)).cuda()
    else:
        shapes = ((B, H, Sq, d), (B, Hkv, Skv, d))
        cu = None
    q, k, v, w = (to_device(synth.normal_tensor(seed * 10 + i, shapes[1 if i in (1, 2) else 0], "bf16"), "bf16")
                  for i in range(4))

    def lay(x):  # BHSD -> the case's layout
        if layout == "bhsd":
            return x.contiguous()
        return x[0].transpose(0, 1).contiguous() if lengths is not None else x.transpose(1, 2).contiguous()

    q, k, v, w = (lay(x) for x in (q, k, v, w))
    sk = (torch.from_numpy(synth.normal_tensor(seed * 10 + 5, (H,), "f32")).cuda() if with_sinks else None)

    # through autograd
    qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
    ska = sk.clone().requires_grad_(True) if sk is not None else None
    o, lse = ea.flash_attention(qa, ka, va, causal=causal, window=window, sinks=ska, cu_seqlens=cu, layout=layout,
                                return_lse=True)
    (o * w).sum().backward()    # dL/do = w, exactly (bf16)

    # the direct calls
    o2, lse2 = ea.attn_fwd_layout(q, k, v, layout=layout, causal=causal, window=window, sinks=sk, cu_seqlens=cu)
    dq, dk, dv, ds = ea.attn_bwd_layout(q, k, v, o2, lse2, w, layout=layout, causal=causal, window=window, sinks=sk,
                                        cu_seqlens=cu)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2) and torch.equal(lse, lse2), "forward differs"
    for name, g, r in (("dq", qa.grad, dq), ("dk", ka.grad, dk), ("dv", va.grad, dv)):
        assert g is not None and torch.equal(g, r), f"{case}: {name} through autograd differs"
    if sk is not None:
        assert ska.grad is not None and torch.equal(ska.grad, ds), f"{case}: dsinks through autograd differs"
