"""Pins for the oracle's number codecs: IEEE/OCP bit-pattern facts, and whole-table agreement
with independent library decoders (numpy float16, torch bfloat16 / float8_e4m3fn)."""
import math

import numpy as np
import pytest
import torch

import oracle


@pytest.mark.parametrize("dtype,bits,value", [
    ("bf16", 0x3F80, 1.0), ("bf16", 0xC000, -2.0), ("bf16", 0x7F80, math.inf),
    ("bf16", 0x0001, 2.0 ** -133), ("bf16", 0x0080, 2.0 ** -126), ("bf16", 0x7F7F, 3.3895313892515355e38),
    ("f16", 0x3C00, 1.0), ("f16", 0x0001, 2.0 ** -24), ("f16", 0x7BFF, 65504.0), ("f16", 0xFC00, -math.inf),
    ("f16", 0x3555, 0.333251953125),
    ("e4m3", 0x38, 1.0), ("e4m3", 0x7E, 448.0), ("e4m3", 0xFE, -448.0), ("e4m3", 0x01, 2.0 ** -9),
    ("e4m3", 0x08, 2.0 ** -6), ("e4m3", 0x07, 7 * 2.0 ** -9), ("e4m3", 0x3C, 1.5),
    ("f32", 0x3F800000, 1.0), ("f32", 0x00000001, 2.0 ** -149),
])
def test_decode_known_patterns(dtype, bits, value):
    got = oracle.decode(dtype, np.array([bits]))[0]
    assert got == value


@pytest.mark.parametrize("dtype,bits", [("e4m3", 0x7F), ("e4m3", 0xFF), ("f16", 0x7E00), ("bf16", 0x7FC0)])
def test_decode_nan(dtype, bits):
    assert math.isnan(oracle.decode(dtype, np.array([bits]))[0])


def test_decode_all_f16_matches_numpy():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ours = oracle.decode("f16", bits)
    ref = bits.view(np.float16).astype(np.float64)
    np.testing.assert_array_equal(ours, ref)


def test_decode_all_bf16_matches_torch():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ours = oracle.decode("bf16", bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_decode_all_e4m3_matches_torch():
    bits = np.arange(256, dtype=np.uint8)
    ours = oracle.decode("e4m3", bits)
    ref = torch.from_numpy(bits).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_encode_f16_matches_numpy_on_random_doubles():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 5, 20000),
                        rng.uniform(-70000, 70000, 2000)])
    ours = oracle.encode_rne("f16", x)
    with np.errstate(over="ignore"):    # beyond 65504: infinity on both sides
        ref = x.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_encode_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(50000) * 10.0 ** rng.integers(-30, 30, 50000)).astype(np.float32)
    ours = oracle.encode_rne("bf16", x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_encode_e4m3_matches_torch_in_range():
    rng = np.random.default_rng(9)
    x = (rng.uniform(-448, 448, 50000) * 2.0 ** rng.integers(-12, 1, 50000)).astype(np.float32)
    ours = oracle.encode_rne("e4m3", x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)


@pytest.mark.parametrize("dtype,value,bits", [
    # exact ties go to the even neighbour
    ("bf16", 1.0 + 2.0 ** -8, 0x3F80),          # between 1 and 1+2^-7: stays at 1 (even)
    ("bf16", 1.0 + 3 * 2.0 ** -8, 0x3F82),      # between 1+2^-7 (odd) and 1+2^-6 (even)
    ("f16", 1.0 + 2.0 ** -11, 0x3C00),
    ("f16", 1.0 + 3 * 2.0 ** -11, 0x3C02),
    ("e4m3", 1.0 + 2.0 ** -4, 0x38),
    ("e4m3", 1.0 + 3 * 2.0 ** -4, 0x3A),
    ("e4m3", 1000.0, 0x7E),                      # saturates to 448
    ("f16", 65520.0, 0x7C00),                    # IEEE overflow to infinity
    ("bf16", -0.0, 0x8000),
])
def test_encode_ties_and_limits(dtype, value, bits):
    assert int(oracle.encode_rne(dtype, np.array([value]))[0]) == bits


def test_roundtrip_is_identity_on_every_finite_pattern():
    for dtype, n in (("f16", 1 << 16), ("bf16", 1 << 16), ("e4m3", 256)):
        bits = np.arange(n, dtype=oracle._STORAGE[dtype])
        vals = oracle.decode(dtype, bits)
        keep = np.isfinite(vals) & ~((vals == 0) & np.signbit(vals))
        back = oracle.encode_rne(dtype, vals[keep])
        np.testing.assert_array_equal(back, bits[keep])
