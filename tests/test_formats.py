"""Storage formats of the synthetic inputs, pinned to their public definitions.

bf16: the upper half of an IEEE-754 binary32 word.  FP8 E4M3: the OCP 8-bit
floating-point format (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
exponent 0 is subnormal with quantum 2^-9; S.1111.111 is NaN; no
infinities, so 0x7E = 448 is the largest finite value).  The concept page's
1M-token scenario stores the indexer keys in FP8; these helpers only convert
formats and hold no arithmetic of the method.
"""
import math

import numpy as np
import pytest

from sparse_attention_12_amd import workloads as wl


@pytest.mark.parametrize("bits,value", [
    (0x00, 0.0), (0x38, 1.0), (0x40, 2.0), (0x44, 3.0), (0x48, 4.0), (0x39, 1.125),
    (0x3F, 1.875), (0x7E, 448.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0xB8, -1.0), (0xC4, -3.0), (0xFE, -448.0), (0x30, 0.5), (0x58, 16.0),
])
def test_e4m3_decode_values(bits, value):
    v = wl.e4m3_bits_to_f32(np.array([bits], np.uint8))[0]
    assert v == value and math.copysign(1.0, v) == math.copysign(1.0, value)


def test_e4m3_nan_and_signed_zero():
    v = wl.e4m3_bits_to_f32(np.array([0x7F, 0xFF, 0x80], np.uint8))
    assert np.isnan(v[0]) and np.isnan(v[1])
    assert v[2] == 0.0 and np.signbit(v[2])


def test_e4m3_decode_is_monotone_and_round_trips():
    pos = wl.e4m3_bits_to_f32(np.arange(0x00, 0x7F, dtype=np.uint8)).astype(np.float64)
    assert np.all(np.diff(pos) > 0)
    # each binade above the subnormals holds 8 evenly spaced values
    for e in range(1, 16):
        seg = pos[8 * e: min(8 * e + 8, 0x7F)]
        assert np.allclose(np.diff(seg), 2.0 ** (e - 7 - 3))
    b = np.arange(256, dtype=np.uint8)
    v = wl.e4m3_bits_to_f32(b)
    back = wl.f32_to_e4m3_bits(v)
    keep = ~np.isnan(v)
    assert np.array_equal(back[keep], b[keep])


def test_e4m3_encode_rounding():
    x = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -11, 449.0, 1e6, -1e6,
                  464.0, 0.3, np.nan], np.float32)
    got = wl.f32_to_e4m3_bits(x)
    # ties go to the even mantissa; above 448 saturates; NaN stays NaN
    assert list(got[:8]) == [0x38, 0x3A, 0x00, 0x01, 0x7E, 0x7E, 0xFE, 0x7E]
    # 0.3 lies between 0.28125 (0x29) and 0.3125 (0x2A); 0.3125 is nearer
    assert got[8] == 0x2A
    assert got[9] == 0x7F


def test_e4m3_encode_is_nearest():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-10, 9, 20000))).astype(np.float32)
    x = x[np.abs(x) <= 448]
    got = wl.e4m3_bits_to_f32(wl.f32_to_e4m3_bits(x)).astype(np.float64)
    grid = wl.e4m3_bits_to_f32(np.arange(256, dtype=np.uint8)).astype(np.float64)
    grid = np.unique(grid[~np.isnan(grid)])
    best = np.abs(grid[None, :] - x.astype(np.float64)[:, None]).min(axis=1)
    assert np.array_equal(np.abs(got - x), best)


def test_small_integers_exact_in_e4m3_and_bf16():
    v = np.arange(-16, 17)
    assert np.array_equal(wl.e4m3_bits_to_f32(wl._small_int_bits(v, "fp8")), v.astype(np.float32))
    assert np.array_equal(wl.bf16_bits_to_f32(wl._small_int_bits(v, "bf16")), v.astype(np.float32))


@pytest.mark.parametrize("bits,value", [(0x3F80, 1.0), (0xC000, -2.0), (0x4040, 3.0),
                                        (0x0001, 2.0 ** -133), (0x7F7F, 3.3895313892515355e38)])
def test_bf16_decode_values(bits, value):
    assert wl.bf16_bits_to_f32(np.array([bits], np.uint16))[0] == np.float32(value)


def test_bf16_encode_ties_to_even():
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20], np.float32)
    assert list(wl.f32_to_bf16_bits(x)) == [0x3F80, 0x3F82, 0x3F81]


def test_fp8_index_workload_draws_the_same_values():
    a = wl.make_decode([300, 2100], "bf16", 2, seed=9)
    b = wl.make_decode([300, 2100], "bf16", 2, seed=9, index_dtype="fp8")
    assert b.qI.dtype == np.uint8 and b.kI.dtype == np.uint8 and b.index_dtype == "fp8"
    assert a.index_dtype == "bf16"
    assert np.array_equal(a.widen(a.qI), b.widen(b.qI))
    assert np.array_equal(a.widen(a.kI), b.widen(b.kI))
    for x, y in zip(a.kv, b.kv):
        assert np.array_equal(x, y)
    p = wl.make_prefill(500, 300, 40, "bf16", seed=3, index_dtype="fp8")
    assert p.kI.dtype == np.uint8 and np.abs(p.widen(p.kI)).max() == 3
