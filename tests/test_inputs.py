"""The seeded input generator: determinism and exact dtype rounding (CPU only)."""
import numpy as np
import pytest

from exact_attention_fa2_amd import inputs


def test_deterministic_and_chunk_independent():
    a = inputs.normal((3, 5, 7), 11, 1, "f32")
    b = inputs.normal((3, 5, 7), 11, 1, "f32")
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(a, inputs.normal((3, 5, 7), 11, 2, "f32"))
    assert not np.array_equal(a, inputs.normal((3, 5, 7), 12, 1, "f32"))
    # a tensor spanning several chunks equals its chunks drawn one by one
    n = inputs.CHUNK * 2 + 1000
    big = inputs.normal((n,), 5, 0, "f32")
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([5, 0, 1])))
    np.testing.assert_array_equal(big[inputs.CHUNK:2 * inputs.CHUNK],
                                  g.standard_normal(inputs.CHUNK, dtype=np.float32))
    assert abs(float(big.mean())) < 5e-3 and abs(float(big.std()) - 1) < 5e-3


def test_f16_storage_is_rne_of_the_f32_draw():
    x32 = inputs.normal((1000,), 3, 0, "f32")
    x16 = inputs.normal((1000,), 3, 0, "f16")
    np.testing.assert_array_equal(x16, x32.astype(np.float16))
    np.testing.assert_array_equal(inputs.to_f64(x16, "f16"), x16.astype(np.float64))


def test_bf16_round_to_nearest_even_against_torch():
    torch = pytest.importorskip("torch")
    x = np.concatenate([inputs.normal((20000,), 4, 0, "f32"),
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8,
                                  1.0 + 2.0 ** -8 + 2.0 ** -20], dtype=np.float32)])
    bits = inputs.f32_to_bf16_bits(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, want)
    back = inputs.bf16_bits_to_f32(bits)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    # ties go to even
    assert inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(np.float32([1.0 + 2.0 ** -8])))[0] == 1.0
