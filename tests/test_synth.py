"""The seeded input generator: published SplitMix64 outputs, rounding,
chunk independence and N(0,1) moments."""

import numpy as np

from exact_attention_09_amd import synth
from pins import golden


def test_splitmix64_reference_outputs():
    want = [int(h, 16) for h in golden()["splitmix64_seed0"]["outputs_hex"]]
    got = [int(x) for x in synth.splitmix64(0, 0, 3)]
    assert got == want


def test_splitmix64_offsets():
    a = synth.splitmix64(77, 0, 100)
    b = synth.splitmix64(77, 40, 60)
    assert np.array_equal(a[40:], b)


def test_bf16_rounding():
    # bf16 keeps 7 fraction bits: the spacing just above 1 is 2^-7
    x = np.array([1.0, 1.0 + 2 ** -7, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -12, -2.5],
                 np.float32)
    back = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    # exact; tie to even (down); tie to even (up); above the tie (up); exact
    assert back.tolist() == [1.0, 1.0 + 2 ** -7, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5]


def test_normals_chunk_independent():
    a = synth.normal_tensor(5, (3, 1000), "f32")
    b = synth._normals_f64(5, 1000, 2000).astype(np.float32)
    assert np.array_equal(a.ravel()[1000:], b)


def test_normal_moments():
    x = synth.normal_tensor(1001, (1 << 20,), "f32").astype(np.float64)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1.0) < 5e-3
    bits = synth.normal_tensor(1001, (1 << 20,), "bf16")
    y = synth.bf16_bits_to_f32(bits)
    assert np.abs(y - x).max() <= 2.0 ** -8 * np.abs(x).max()


def test_varlen_lengths_range():
    L = synth.varlen_lengths(4003, 1000)
    assert L.min() >= 256 and L.max() <= 4096
    cu = synth.cu_seqlens_from_lengths(L[:8])
    assert cu[0] == 0 and cu[-1] == L[:8].sum() and cu.dtype == np.int32
