"""Pins of the oracle's fp16 storage conversions against numpy's IEEE-754 binary16 routines.

The oracle decodes every fp16 input exactly and rounds every fp16 output to nearest-even; numpy's
float16 casts are an independent, correctly rounded implementation of the same format.
"""
import numpy as np


def test_decode_all_bit_patterns(oracle):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zero survives
    assert np.signbit(ours[0x8000]) and not np.signbit(ours[0])


def _special_doubles():
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e9, -1e9,
            2.0 ** -14, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26, 3 * 2.0 ** -25,
            np.inf, -np.inf, 6.1e-5, 6.0e-8]
    # exact halfway points between neighbouring fp16 values, normal and subnormal
    h = np.arange(0, 0x7bff, 97, dtype=np.uint16).view(np.float16).astype(np.float64)
    h2 = (np.arange(1, 0x7c00, 97, dtype=np.uint16)).view(np.float16).astype(np.float64)
    return np.concatenate([np.array(vals), (h + h2) / 2, -(h + h2) / 2])


def test_encode_f64_matches_numpy(oracle):
    rng = np.random.default_rng(123)
    x = np.concatenate([
        _special_doubles(),
        rng.standard_normal(20000),
        rng.standard_normal(5000) * 1e4,
        rng.standard_normal(5000) * 1e-5,
        rng.standard_normal(2000) * 1e-7,
    ])
    ours = oracle.f64_to_f16_bits(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_encode_f32_matches_numpy(oracle):
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(4000) * 3e-5).astype(np.float32),
                        _special_doubles().astype(np.float32)])
    ours = oracle.f32_to_f16_bits(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_encode_nan(oracle):
    b = oracle.f64_to_f16_bits(np.array([np.nan]))[0]
    assert (b & 0x7c00) == 0x7c00 and (b & 0x3ff) != 0
