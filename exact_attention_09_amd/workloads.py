"""The attention workloads: shapes, seeded inputs and work counts.

Shapes are the ones the pages' discussion is built around (a single head for
the worked examples, multi-head prefill at 2K and 8K tokens, packed
variable-length grouped-query prefill, and split-KV decode over a 16K cache,
contiguous or paged).
Inputs are synthetic i.i.d. N(0, 1) from ``synth`` with seed
``1000 * workload_id + tensor_id``.

Work counts (used for throughput, not by the computation):
* FLOPs: 4 * B * H * Sq * Skv * d, halved when causal (the TileLang forward
  blog post's TFLOPs formula, section 6); varlen sums 4 * H * L^2 * d / 2 over
  the sequences.
* Algorithmic HBM bytes: Q + K + V + O once each plus the fp32 LSE; the
  decode path adds its fp32 split partials, written once and read once.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np

from . import synth


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # seed base: 1000 * wid + tensor id
    B: int
    H: int
    Hkv: int
    Sq: int
    Skv: int
    d: int
    dtype: str               # "bf16" or "f32"
    causal: bool
    lengths: tuple = field(default=())   # varlen sequence lengths (then B = len)
    num_splits: int = 0      # decode path split count (0 = library heuristic)
    page_size: int = 0       # > 0: decode over a paged KV cache of Skv keys per sequence
    window: int = 0          # > 0: causal sliding window of this many keys
    sinks: bool = False      # per-head attention sinks (seeded inputs)
    backward: bool = False   # time the backward pass (dq, dk, dv) instead

    @property
    def paged(self) -> bool:
        return self.page_size > 0

    @property
    def max_pages(self) -> int:
        return -(-self.Skv // self.page_size) if self.paged else 0

    @property
    def num_pages(self) -> int:
        # one spare page per sequence, so the table is not the whole cache
        return self.B * (self.max_pages + 1) if self.paged else 0

    def cache_shape(self):
        return (self.num_pages, self.Hkv, self.page_size, self.d)

    @property
    def varlen(self) -> bool:
        return len(self.lengths) > 0

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def total_tokens(self) -> int:
        return int(sum(self.lengths)) if self.varlen else self.Sq

    def q_shape(self):
        return (1, self.H, self.total_tokens, self.d) if self.varlen else (self.B, self.H, self.Sq, self.d)

    def kv_shape(self):
        if self.paged:
            return self.cache_shape()
        return (1, self.Hkv, self.total_tokens, self.d) if self.varlen else (self.B, self.Hkv, self.Skv, self.d)

    def cu_seqlens(self):
        return synth.cu_seqlens_from_lengths(self.lengths) if self.varlen else None

    def visible_pairs(self) -> float:
        """(query, key) pairs a causal (optionally windowed) dense head sees."""
        off = self.Skv - self.Sq
        i = np.arange(self.Sq, dtype=np.int64)
        hi = np.minimum(self.Skv, i + off + 1)
        lo = np.maximum(0, i + off - self.window + 1) if self.window > 0 else np.zeros_like(i)
        return float(np.maximum(0, hi - lo).sum())

    def flops(self) -> float:
        if self.backward:
            # the usual count for the backward: five products of the forward's
            # size (S recomputed, dP, dV, dQ, dK), 2.5 times the forward
            return 2.5 * dataclasses.replace(self, backward=False).flops()
        if self.window > 0 and not self.varlen:
            return 4.0 * self.B * self.H * self.d * self.visible_pairs()
        if self.varlen:
            return float(sum(4.0 * self.H * L * L * self.d * 0.5 if self.causal else 4.0 * self.H * L * L * self.d
                             for L in self.lengths))
        f = 4.0 * self.B * self.H * self.Sq * self.Skv * self.d
        return f * 0.5 if self.causal else f

    def rows(self) -> int:
        return self.H * self.total_tokens if self.varlen else self.B * self.H * self.Sq

    def bytes(self, num_splits: int = 0) -> float:
        eb = self.elem_bytes
        q_o = 2 * int(np.prod(self.q_shape())) * eb
        kv = 2 * int(np.prod(self.kv_shape())) * eb
        if self.paged:  # the pages the sequences use, not the whole pool
            kv = 2 * self.B * self.Hkv * self.Skv * self.d * eb
        lse = 4 * self.rows()
        partial = 0
        if num_splits and not self.varlen and self.Sq == 1:
            partial = 2 * self.B * self.H * num_splits * (self.d + 1) * 4
        return float(q_o + kv + lse + partial)

    def make_inputs(self):
        """Seeded host inputs: dict with q, k, v (uint16 bf16 bits or fp32)
        and cu_seqlens (int32) for varlen."""
        base = 1000 * self.wid
        q = synth.normal_tensor(base + synth.TENSOR_Q, self.q_shape(), self.dtype)
        k = synth.normal_tensor(base + synth.TENSOR_K, self.kv_shape(), self.dtype)
        v = synth.normal_tensor(base + synth.TENSOR_V, self.kv_shape(), self.dtype)
        out = {"q": q, "k": k, "v": v, "cu_seqlens": self.cu_seqlens()}
        if self.sinks:
            out["sinks"] = synth.normal_tensor(base + synth.TENSOR_SINKS, (self.H,), "f32") * np.float32(2.0)
        if self.backward:
            out["dout"] = synth.normal_tensor(base + synth.TENSOR_DOUT, self.q_shape(), self.dtype)
        if self.paged:
            out["block_table"] = synth.page_table(base + synth.TENSOR_PAGES, self.B, self.max_pages,
                                                  self.num_pages)
            out["seqlens_k"] = np.full(self.B, self.Skv, np.int32)
        return out


def host_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp32 view of a host input (bf16 bits are widened)."""
    return synth.bf16_bits_to_f32(x) if dtype == "bf16" else np.asarray(x, np.float32)


def to_device(x: np.ndarray, dtype: str, device="cuda"):
    """Host input -> torch tensor on the GPU (bf16 bits keep their bytes)."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device)


VARLEN_LENGTHS = tuple(int(x) for x in synth.varlen_lengths(1000 * 4 + synth.TENSOR_LENGTHS, 8))

WORKLOADS = {
    "single_head_f32": Workload("single_head_f32", 1, B=1, H=1, Hkv=1, Sq=128, Skv=128, d=64,
                                dtype="f32", causal=False),
    "mha_causal_s2048_d64": Workload("mha_causal_s2048_d64", 2, B=4, H=16, Hkv=16, Sq=2048, Skv=2048, d=64,
                                     dtype="bf16", causal=True),
    "mha_s8192_d128": Workload("mha_s8192_d128", 3, B=1, H=32, Hkv=32, Sq=8192, Skv=8192, d=128,
                               dtype="bf16", causal=False),
    "mha_causal_s8192_d128": Workload("mha_causal_s8192_d128", 3, B=1, H=32, Hkv=32, Sq=8192, Skv=8192,
                                      d=128, dtype="bf16", causal=True),
    "varlen_gqa_causal_d128": Workload("varlen_gqa_causal_d128", 4, B=len(VARLEN_LENGTHS), H=32, Hkv=8,
                                       Sq=sum(VARLEN_LENGTHS), Skv=sum(VARLEN_LENGTHS), d=128, dtype="bf16",
                                       causal=True, lengths=VARLEN_LENGTHS),
    "decode_gqa_s16384_d128": Workload("decode_gqa_s16384_d128", 5, B=32, H=32, Hkv=8, Sq=1, Skv=16384, d=128,
                                       dtype="bf16", causal=False, num_splits=16),
    # sliding-window attention with per-head sinks at long context: a window
    # of 4096 keys (the CUDA course's section 12.9.5 example) over 32K tokens,
    # grouped-query heads
    "swa_sink_s32768_d128": Workload("swa_sink_s32768_d128", 7, B=1, H=32, Hkv=8, Sq=32768, Skv=32768, d=128,
                                     dtype="bf16", causal=True, window=4096, sinks=True),
    # the backward pass of the headline shape (dout seeded N(0, 1))
    "bwd_mha_s8192_d128": Workload("bwd_mha_s8192_d128", 8, B=1, H=32, Hkv=32, Sq=8192, Skv=8192, d=128,
                                   dtype="bf16", causal=False, backward=True),
    "bwd_mha_causal_s8192_d128": Workload("bwd_mha_causal_s8192_d128", 9, B=1, H=32, Hkv=32, Sq=8192, Skv=8192,
                                          d=128, dtype="bf16", causal=True, backward=True),
    # the backward of causal attention with a 2048-token window and per-head
    # sinks over 8K tokens (MHA, so that one head's full oracle checks it)
    "bwd_swa_sink_s8192_d128": Workload("bwd_swa_sink_s8192_d128", 11, B=1, H=32, Hkv=32, Sq=8192, Skv=8192,
                                        d=128, dtype="bf16", causal=True, window=2048, sinks=True, backward=True),
    # the backward of the varlen prefill's packing (8 sequences, 22342 tokens)
    "bwd_varlen_gqa_causal_d128": Workload("bwd_varlen_gqa_causal_d128", 10, B=len(VARLEN_LENGTHS), H=32, Hkv=8,
                                           Sq=sum(VARLEN_LENGTHS), Skv=sum(VARLEN_LENGTHS), d=128, dtype="bf16",
                                           causal=True, lengths=VARLEN_LENGTHS, backward=True),
    # the same decode over a paged cache: 16-token pages (the CUDA course's
    # typical block size) scattered by a seeded permutation
    "decode_paged_gqa_s16384_d128": Workload("decode_paged_gqa_s16384_d128", 6, B=32, H=32, Hkv=8, Sq=1,
                                             Skv=16384, d=128, dtype="bf16", causal=False, num_splits=16,
                                             page_size=16),
}
