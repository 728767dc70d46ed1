"""Pins for the oracle's quantizers and its KV append.

The rule is the ggml reference quantizer for each block type, in float32 with
the scale stored as the nearest binary16:
  Q8_0: d = max|x| / 127, code = round-half-away(x / d), within [-127, 127];
  Q4_0: d = (first element of largest magnitude) / -8,
        nibble = min(15, trunc(x / d + 8.5)).
Expected bytes below are worked by hand from that rule; the round trips and
error bounds follow from it (a block whose values are exact multiples of a
binary16 scale quantizes back to itself).
"""

import math

import numpy as np
import pytest

from oracle import (append_rows, dequant_q4_0, dequant_q8_0, gather_kv, page_bytes,
                    quantize_q4_0_block, quantize_q8_0_block)


def f16_bytes(v):
    b = int(np.array([v], np.float16).view(np.uint16)[0])
    return [b & 0xFF, b >> 8]


# ---- hand-worked blocks ---------------------------------------------------

def test_q8_0_half_way_codes_round_away_from_zero():
    # amax = 127 -> d = 1, 1 / d = 1: the codes are the values rounded half away
    x = np.zeros(32, np.float32)
    x[:9] = [127.0, 63.5, -63.5, 0.5, -0.5, 1.5, -2.5, 0.49999997, -126.5]
    blk = quantize_q8_0_block(x)
    assert blk[:2].tolist() == f16_bytes(1.0)
    codes = blk[2:].view(np.int8)[:9].tolist()
    # round half to even would give 64, -64, 0, 0, 2, -2, 0, -126
    assert codes == [127, 64, -64, 1, -1, 2, -3, 0, -127]


def test_q8_0_scale_is_amax_over_127_rounded_to_binary16():
    x = np.zeros(32, np.float32)
    x[7] = -1.0                       # amax 1 -> d = 1/127 = 0.007874016 -> binary16 0x2008
    x[3] = 0.25                       # 0.25 * 127 = 31.75 -> 32
    blk = quantize_q8_0_block(x)
    assert int(blk[0]) | (int(blk[1]) << 8) == 0x2008
    codes = blk[2:].view(np.int8)
    assert codes[7] == -127 and codes[3] == 32 and np.count_nonzero(codes) == 2


def test_q4_0_negative_extreme_gives_positive_scale():
    x = np.zeros(32, np.float32)
    x[:6] = [-8.0, 7.0, 0.5, -0.5, 3.4999, 6.6]
    x[20] = -7.9                      # not the extreme: |-8| is larger
    blk = quantize_q4_0_block(x)
    assert blk[:2].tolist() == f16_bytes(1.0)     # d = -8 / -8 = 1
    nib = np.concatenate([blk[2:] & 15, blk[2:] >> 4])
    # x + 8.5 truncated, at most 15; zeros give 8
    assert nib[:6].tolist() == [0, 15, 9, 8, 11, 15]
    assert nib[20] == 0 and nib[6] == 8 and nib[31] == 8


def test_q4_0_positive_extreme_gives_negative_scale():
    x = np.zeros(32, np.float32)
    x[0], x[1], x[2] = 8.0, -7.0, 2.0
    blk = quantize_q4_0_block(x)
    assert blk[:2].tolist() == f16_bytes(-1.0)    # d = 8 / -8 = -1
    nib = np.concatenate([blk[2:] & 15, blk[2:] >> 4])
    assert nib[:3].tolist() == [0, 15, 6]        # -x + 8.5 truncated


def test_q4_0_ties_on_magnitude_take_the_first_element():
    x = np.zeros(32, np.float32)
    x[2], x[9] = -4.0, 4.0
    assert quantize_q4_0_block(x)[:2].tolist() == f16_bytes(0.5)    # -4 / -8
    x[2], x[9] = 4.0, -4.0
    assert quantize_q4_0_block(x)[:2].tolist() == f16_bytes(-0.5)   # 4 / -8


def test_zero_blocks():
    z = np.zeros(32, np.float32)
    b8 = quantize_q8_0_block(z)
    assert b8.tolist() == [0] * 34
    b4 = quantize_q4_0_block(z)
    # the extreme stays +0, so d = +0 / -8 = -0 (binary16 0x8000); nibbles 8
    assert b4[:2].tolist() == [0x00, 0x80] and b4[2:].tolist() == [0x88] * 16


# ---- round trips and error bounds ----------------------------------------

def test_q8_0_round_trip_of_blocks_with_an_extreme_code():
    rng = np.random.default_rng(1)
    for _ in range(300):
        e = int(rng.integers(-10, 12))
        d = np.float16(np.ldexp(1.0 + rng.integers(0, 1024) / 1024.0, e))
        codes = rng.integers(-127, 128, 32).astype(np.int8)
        codes[rng.integers(0, 32)] = 127 if rng.random() < 0.5 else -127
        blk = np.zeros(34, np.uint8)
        blk[:2] = np.array([d], np.float16).view(np.uint8)
        blk[2:] = codes.view(np.uint8)
        x = dequant_q8_0(blk).astype(np.float32)       # exact: 11-bit scale x 8-bit code
        assert np.array_equal(quantize_q8_0_block(x), blk)


def test_q4_0_round_trip_of_blocks_with_a_zero_nibble():
    rng = np.random.default_rng(2)
    for _ in range(300):
        e = int(rng.integers(-10, 12))
        d = np.float16(np.ldexp(1.0 + rng.integers(0, 1024) / 1024.0, e)) * (1 if rng.random() < 0.5 else -1)
        nib = rng.integers(1, 16, 32)
        nib[rng.integers(0, 32)] = 0                     # value -8 d: the unique largest magnitude
        blk = np.zeros(18, np.uint8)
        blk[:2] = np.array([d], np.float16).view(np.uint8)
        blk[2:] = (nib[:16] | (nib[16:] << 4)).astype(np.uint8)
        x = dequant_q4_0(blk).astype(np.float32)
        assert np.array_equal(quantize_q4_0_block(x), blk)


def test_error_bounds_on_random_blocks():
    rng = np.random.default_rng(3)
    for _ in range(200):
        x = (rng.standard_normal(32) * np.exp(rng.uniform(-4, 4))).astype(np.float32)
        b8 = quantize_q8_0_block(x)
        d8 = float(np.max(np.abs(x))) / 127.0
        err8 = np.max(np.abs(dequant_q8_0(b8) - x))
        # half a step, plus the binary16 rounding of the scale times the largest code
        assert err8 <= d8 / 2 + 127 * d8 * 2.0 ** -11 + 1e-12
        b4 = quantize_q4_0_block(x)
        d4 = float(np.max(np.abs(x))) / 8.0
        err4 = np.max(np.abs(dequant_q4_0(b4) - x))
        # a full step for the top nibble clamp (x / d + 8.5 can reach 16.5),
        # half a step elsewhere, plus the scale rounding
        assert err4 <= d4 + 8 * d4 * 2.0 ** -11 + 1e-12


# ---- append placement -----------------------------------------------------

def test_append_rows_lands_where_gather_reads_and_nowhere_else():
    H, D, T = 2, 128, 256
    n_pages = 3
    rng = np.random.default_rng(4)
    recs = rng.integers(0, 256, (n_pages, page_bytes(H, D, T)), dtype=np.uint8)
    # keep the untouched rows finite so that gather can read them
    pos0, n = 250, 12                                   # crosses from page 0 into page 1
    k = rng.standard_normal((n, H, D)).astype(np.float32)
    v = rng.standard_normal((n, H, D)).astype(np.float16)
    out = append_rows(recs, k, v, pos0=pos0, n_kv_heads=H, head_dim=D)
    # appended tokens read back as the dequantized blocks of their values
    K, V = gather_kv(out, H, D, pos0, n)
    for i in range(n):
        for g in range(H):
            for b in range(D // 32):
                kb = quantize_q8_0_block(k[i, g, 32 * b:32 * b + 32])
                vb = quantize_q4_0_block(v[i, g, 32 * b:32 * b + 32].astype(np.float32))
                assert np.array_equal(K[i, g, 32 * b:32 * b + 32], dequant_q8_0(kb))
                assert np.array_equal(V[i, g, 32 * b:32 * b + 32], dequant_q4_0(vb))
    # every byte outside those rows is the input's
    changed = np.argwhere(out != recs)
    kbytes = H * T * (D // 32) * 34
    for p, off in changed:
        if off < kbytes:
            row = (off % (T * (D // 32) * 34)) // ((D // 32) * 34)
        else:
            row = ((off - kbytes) % (T * (D // 32) * 18)) // ((D // 32) * 18)
        tok = p * T + row
        assert pos0 <= tok < pos0 + n, (p, off, tok)
    assert page_bytes(H, D, T) == recs.shape[1]
    assert np.array_equal(out[2], recs[2])              # page 2 untouched


def test_append_rows_q8_0_v_lands_where_gather_reads_and_nowhere_else():
    H, D, T = 2, 64, 256
    n_pages = 3
    rng = np.random.default_rng(5)
    pb = page_bytes(H, D, T, "q8_0", "q8_0")
    assert pb == T * H * (D // 32) * (34 + 34)
    recs = rng.integers(0, 256, (n_pages, pb), dtype=np.uint8)
    pos0, n = 509, 6                                    # crosses from page 1 into page 2
    k = rng.standard_normal((n, H, D)).astype(np.float32)
    v = (8.0 * rng.standard_normal((n, H, D))).astype(np.float32)
    out = append_rows(recs, k, v, pos0=pos0, n_kv_heads=H, head_dim=D, type_v="q8_0")
    K, V = gather_kv(out, H, D, pos0, n, type_v="q8_0")
    for i in range(n):
        for g in range(H):
            for b in range(D // 32):
                kb = quantize_q8_0_block(k[i, g, 32 * b:32 * b + 32])
                vb = quantize_q8_0_block(v[i, g, 32 * b:32 * b + 32])
                assert np.array_equal(K[i, g, 32 * b:32 * b + 32], dequant_q8_0(kb))
                assert np.array_equal(V[i, g, 32 * b:32 * b + 32], dequant_q8_0(vb))
    blk = (D // 32) * 34                                # bytes of one token row of one head, K or V
    kbytes = H * T * blk
    for p, off in np.argwhere(out != recs):
        row = ((off if off < kbytes else off - kbytes) % (T * blk)) // blk
        tok = p * T + row
        assert pos0 <= tok < pos0 + n, (p, off, tok)
    assert np.array_equal(out[0], recs[0])              # page 0 untouched
