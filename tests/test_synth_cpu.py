"""The seeded input generator's 8-bit encoders (CPU): FP8 E4M3 encoding agrees with torch's round-to-nearest-even
cast on every tested value (ties, subnormals, saturation at 448), and int8 rounds half to even and clips at 127."""
import numpy as np
import torch

from synth import f32_to_e4m3_bits, f32_to_int8_bits


def test_e4m3_encoder_matches_torch_cast():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * np.float32(30)
    ties = np.array([1.0625, 1.1875, -1.0625, 2.0 ** -9 * 1.5, 2.0 ** -9 * 2.5, 2.0 ** -10, 464.0, 448.0, 447.0],
                    np.float32)
    x = np.concatenate([x, ties, np.array([0.0, -0.0, 1e6, -1e6, 2.0 ** -20], np.float32)])
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(f32_to_e4m3_bits(x), ref)
    assert not np.any((f32_to_e4m3_bits(x) & 0x7F) == 0x7F)          # never the NaN code


def test_int8_encoder_rounds_half_even_and_clips():
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, 126.6, 127.5, 300, -300, -127.5], np.float32)
    got = f32_to_int8_bits(x).view(np.int8)
    np.testing.assert_array_equal(got, [0, 2, 2, 0, -2, 127, 127, 127, -127, -127])
