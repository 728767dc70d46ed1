"""Pins for the oracle's binary16 decode, Q8_0 / Q4_0 dequantization and page sizes.

Expected values below are worked by hand from the block definitions (ggml
Q8_0: value = d * q; Q4_0: value = d * (nibble - 8), low nibble = element j,
high nibble = element j + 16), or are sizes printed on page 3.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import dequant_q4_0, dequant_q8_0, f16_to_f64, page_bytes
from kvs_synth import quantize_q4_0, quantize_q8_0

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_f16_every_encoding_matches_numpy_binary16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


@pytest.mark.parametrize("bits,value", [
    (0x3C00, 1.0), (0xBC00, -1.0), (0x3800, 0.5), (0x0001, 2.0 ** -24),
    (0x03FF, 1023 * 2.0 ** -24), (0x0400, 2.0 ** -14), (0x7BFF, 65504.0),
    (0x3555, 0.333251953125), (0xC000, -2.0), (0x7C00, math.inf), (0xFC00, -math.inf),
])
def test_f16_hand_values(bits, value):
    assert f16_to_f64(np.array([bits], np.uint16))[0] == value


def q8_block(scale_bits, codes):
    b = np.zeros(34, np.uint8)
    b[0], b[1] = scale_bits & 0xFF, scale_bits >> 8
    b[2:2 + len(codes)] = np.array(codes, np.int64).astype(np.int8).view(np.uint8)
    return b


def test_q8_0_hand_blocks():
    codes = [0, 1, -1, 127, -128, 2, -2, 64]
    # d = 1: values are the codes
    v = dequant_q8_0(q8_block(0x3C00, codes))
    assert list(v[:8]) == [0.0, 1.0, -1.0, 127.0, -128.0, 2.0, -2.0, 64.0]
    assert np.all(v[8:] == 0.0)
    # d = -1 flips every sign
    assert list(dequant_q8_0(q8_block(0xBC00, codes))[:8]) == [0.0, -1.0, 1.0, -127.0, 128.0, -2.0, 2.0, -64.0]
    # d = 65504 (largest finite): 127 * 65504 = 8319008, -128 * 65504 = -8384512
    v = dequant_q8_0(q8_block(0x7BFF, codes))
    assert v[3] == 8319008.0 and v[4] == -8384512.0
    # d = 2^-24 (smallest subnormal): 127 * 2^-24
    v = dequant_q8_0(q8_block(0x0001, codes))
    assert v[3] == 127 * 2.0 ** -24 and v[4] == -128 * 2.0 ** -24
    # d = 0.333251953125: 3 * d = 0.999755859375
    assert dequant_q8_0(q8_block(0x3555, [3]))[0] == 0.999755859375
    # d = 0: every value is zero
    assert np.all(dequant_q8_0(q8_block(0x0000, codes)) == 0.0)
    # scale is little-endian: bytes (0x00, 0x3C) is 1.0, (0x3C, 0x00) is 0x003C = 60 * 2^-24
    swapped = q8_block(0x003C, [1])
    assert dequant_q8_0(swapped)[0] == 60 * 2.0 ** -24


def q4_block(scale_bits, nibbles):
    """nibbles: 32 values 0..15 for elements 0..31."""
    b = np.zeros(18, np.uint8)
    b[0], b[1] = scale_bits & 0xFF, scale_bits >> 8
    n = np.array(nibbles, np.uint8)
    b[2:] = n[:16] | (n[16:] << 4)
    return b


def test_q4_0_hand_blocks():
    # Byte 0 = 0xF0: element 0 = 0 - 8 = -8, element 16 = 15 - 8 = 7.
    b = np.zeros(18, np.uint8)
    b[0], b[1] = 0x00, 0x3C          # d = 1
    b[2] = 0xF0
    b[3] = 0x08                      # element 1 = 0, element 17 = -8
    b[4] = 0x9A                      # element 2 = 10 - 8 = 2, element 18 = 9 - 8 = 1
    v = dequant_q4_0(b)
    assert v[0] == -8.0 and v[16] == 7.0
    assert v[1] == 0.0 and v[17] == -8.0
    assert v[2] == 2.0 and v[18] == 1.0
    # untouched bytes are 0x00: both nibbles 0 -> -8
    assert v[3] == -8.0 and v[19] == -8.0
    # d = -2: nibble 0 -> 16, nibble 15 -> -14
    b[0], b[1] = 0x00, 0xC0
    v = dequant_q4_0(b)
    assert v[0] == 16.0 and v[16] == -14.0
    # d = 2^-24, nibble 15 -> 7 * 2^-24
    v = dequant_q4_0(q4_block(0x0001, [15] * 32))
    assert np.all(v == 7 * 2.0 ** -24)


def test_round_trip_q8_0():
    """Encode(decode(B)) == B for blocks whose largest code is +-127 and whose
    scale is a positive normal binary16."""
    rng = np.random.default_rng(7)
    blocks = np.zeros((500, 34), np.uint8)
    for k in range(500):
        codes = rng.integers(-127, 128, 32)
        codes[rng.integers(0, 32)] = 127 if rng.random() < 0.5 else -127
        scale = np.float16(rng.uniform(1e-3, 10.0))
        blocks[k] = q8_block(int(np.array(scale).view(np.uint16)), codes)
    x = dequant_q8_0(blocks).astype(np.float32)
    assert np.array_equal(quantize_q8_0(x), blocks)


def test_round_trip_q4_0():
    """Encode(decode(B)) == B for blocks that hold a nibble 0 (the -8 code)
    and a non-zero scale of either sign."""
    rng = np.random.default_rng(8)
    blocks = np.zeros((500, 18), np.uint8)
    for k in range(500):
        nib = rng.integers(0, 16, 32)
        nib[rng.integers(0, 32)] = 0
        scale = np.float16(rng.uniform(1e-3, 10.0) * (1 if rng.random() < 0.5 else -1))
        blocks[k] = q4_block(int(np.array(scale).view(np.uint16)), nib)
    x = dequant_q4_0(blocks).astype(np.float32)
    assert np.array_equal(quantize_q4_0(x), blocks)


def test_page_sizes_printed_on_page3():
    with open(os.path.join(GOLDEN, "page3_sizes.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        # 1024 values per token split as 8 kv heads x 128 (any split gives the same bytes)
        pb = page_bytes(8, c["kv_values_per_token"] // 8, 256, c["type_k"], c["type_v"])
        mib = (c["n_ctx"] // 256) * c["layers"] * pb / 2 ** 20
        if "printed_decimals" in c:
            assert round(mib, c["printed_decimals"]) == c["printed_mib"], c
        else:
            assert mib == c["printed_mib"], c


def test_q8_0_q4_0_page_bytes():
    # 4 kv heads x 128: K row 4 x 4 x 34 = 544 B, V row 4 x 4 x 18 = 288 B
    assert page_bytes(4, 128) == 256 * (544 + 288) == 212992
    assert page_bytes(1, 128) == 53248


def test_numpy_binary16_encoding_rounds_to_nearest_even():
    """The staged-operand probe compares the kernels' f16 operands with
    numpy's float64 -> float16 conversion of the exact value; pin that
    conversion to round-to-nearest-even on every pair of neighbouring finite
    binary16 values (subnormals included): each value maps to itself, a point
    just inside either half of the gap maps to the nearer neighbour, and the
    exact midpoint maps to the neighbour with an even significand."""
    from oracle import f16_to_f64
    bits = np.arange(0, 0x7C00, dtype=np.uint16)          # +0 .. 65504
    vals = f16_to_f64(bits)
    lo, hi = vals[:-1], vals[1:]
    assert np.array_equal(vals.astype(np.float16).view(np.uint16), bits)
    mid = (lo + hi) / 2                                      # exact in float64
    gap = hi - lo
    near_lo = (mid - gap / 8).astype(np.float16).view(np.uint16)
    near_hi = (mid + gap / 8).astype(np.float16).view(np.uint16)
    assert np.array_equal(near_lo, bits[:-1]) and np.array_equal(near_hi, bits[1:])
    at_mid = mid.astype(np.float16).view(np.uint16)
    want = np.where(bits[:-1] % 2 == 0, bits[:-1], bits[1:])
    assert np.array_equal(at_mid, want)
    # negatives mirror, and the largest value's upper half-gap rounds to it
    assert np.array_equal((-vals).astype(np.float16).view(np.uint16), bits | 0x8000)
    assert np.float16(65504.0 + 15.0).view(np.uint16) == 0x7BFF
