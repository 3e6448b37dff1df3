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


def test_mla_q8_inputs_quantise_the_bf16_draws():
    """The 8-bit latent cache holds codes of the same draws as the bf16 cache, divided by per-channel scales: inside
    the code range the dequantised values are within half a code step (FP8: relative 2^-4; int8: absolute scale/2)
    of the draws, and outside it they saturate at the largest code."""
    import dataclasses
    import oracle
    from synth import WORKLOADS, mla_inputs
    w = dataclasses.replace(WORKLOADS["mla_decode_b32"], batch=2, seqlen=64)
    ref = mla_inputs(w, seed=3)
    cv = oracle.bf16_bits_to_f64(ref["c_kv"])
    for kind in ("fp8", "int8"):
        q8 = mla_inputs(w, seed=3, kv=kind)
        assert q8["c_kv"].dtype == np.uint8 and q8["c_scale"].shape == (w.latent,) and q8["pe_scale"].shape == (w.rope,)
        np.testing.assert_array_equal(q8["q_lat"], ref["q_lat"])
        dec = oracle.fp8_e4m3_decode if kind == "fp8" else oracle.int8_decode
        got = dec(q8["c_kv"]) * q8["c_scale"]
        # both come from the same fp32 draw: bf16 rounding (2^-9 relative) plus the code's half step
        tol = np.abs(cv) * (2.0 ** -4 + 2.0 ** -8) + 2.0 ** -9 * 8 * q8["c_scale"] if kind == "fp8" else \
            0.5 * q8["c_scale"] + np.abs(cv) * 2.0 ** -8
        top = (448.0 if kind == "fp8" else 127.0) * q8["c_scale"]
        inside = np.abs(cv) < 0.99 * top
        assert np.all((np.abs(got - cv) <= tol)[inside])
        np.testing.assert_allclose(np.abs(got[np.abs(cv) > 1.01 * top]), np.broadcast_to(top, cv.shape)[np.abs(cv) > 1.01 * top])
