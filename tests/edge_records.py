"""Hand-built page records at the edges of the Q8_0 / Q4_0 block formats.

Block contents are chosen directly as bytes (no quantizer): binary16 scales
from a regime's set, Q8_0 codes over the whole int8 range (-128 included,
with some blocks all -128 or all 127) and Q4_0 nibbles over 0..15 (with some
blocks all 0 or all 15, in both the low and the high nibble). V blocks are
Q4_0, or Q8_0 (codes drawn like K's) for the q8_0-q8_0 pair. The bytes are
packed into page records by the shared packer, so that the oracle and the
library read exactly the same records.
"""

import numpy as np

from kvs_synth import KVGeometry, pack_page_records

QK = 32

# binary16 encodings
F16_ONE, F16_MINUS_ONE = 0x3C00, 0xBC00
F16_MIN_SUB, F16_MINUS_MIN_SUB = 0x0001, 0x8001   # +-2^-24
F16_MAX = 0x7BFF                                  # 65504
F16_ZERO = 0x0000

# Scale regimes: each maps a generator and a shape to uint16 scale bits.
#   big:    +-65504 and other scales above 8188 (V operands need the shift)
#   mid:    +-256, +-511.75, +-512, +-1024: either side of the 511.75 bound
#           above which Q8_0 V operands need the shift
#   tiny:   subnormal scales, 2^-24 .. 1023 * 2^-24, both signs
#   mixed:  +-1, +-2^-14, 0, +-0.5, -2^-3: within a factor 2^14 of the largest
#   edges:  the set {+-1, +-2^-24, 65504, 0} at random (K only: V's spread
#           would leave the documented accuracy range)
def _scales(regime, g, shape):
    if regime == "big":
        mag = g.choice(np.array([F16_MAX, 0x7A00, 0x7000, 0x7400], np.uint16), size=shape)
        return mag | (g.integers(0, 2, size=shape, dtype=np.uint16) << 15)
    if regime == "mid":
        mag = g.choice(np.array([0x5C00, 0x5FFF, 0x6000, 0x6400], np.uint16), size=shape)
        return mag | (g.integers(0, 2, size=shape, dtype=np.uint16) << 15)
    if regime == "tiny":
        mag = g.integers(1, 1024, size=shape).astype(np.uint16)
        mag[g.random(shape) < 0.3] = F16_MIN_SUB
        return mag | (g.integers(0, 2, size=shape, dtype=np.uint16) << 15)
    if regime == "mixed":
        return g.choice(np.array([F16_ONE, F16_MINUS_ONE, 0x0400, 0x8400, F16_ZERO, 0x3800, 0xB800, 0xB000],
                                 np.uint16), size=shape)
    if regime == "edges":
        return g.choice(np.array([F16_ONE, F16_MINUS_ONE, F16_MIN_SUB, F16_MINUS_MIN_SUB, F16_MAX, F16_ZERO],
                                 np.uint16), size=shape)
    raise ValueError(regime)


def edge_blocks(seed, n_tok, n_kv_heads, head_dim, k_regime, v_regime, type_v="q4_0"):
    """Token-major Q8_0 K blocks uint8 [n_tok, Hkv, nb, 34] and V blocks
    uint8 [n_tok, Hkv, nb, 18] (Q4_0) or [..., 34] (Q8_0)."""
    g = np.random.default_rng(seed)
    nb = head_dim // QK
    shape = (n_tok, n_kv_heads, nb)
    kd = _scales(k_regime, g, shape)
    vd = _scales(v_regime, g, shape)
    codes = g.integers(-128, 128, size=shape + (QK,), dtype=np.int16)
    codes[g.random(shape + (QK,)) < 0.05] = -128
    sel = g.random(shape)
    codes[sel < 0.02] = -128
    codes[(sel >= 0.02) & (sel < 0.04)] = 127
    nib = g.integers(0, 16, size=shape + (QK,), dtype=np.uint8)
    sel = g.random(shape)
    nib[sel < 0.02] = 0
    nib[(sel >= 0.02) & (sel < 0.04)] = 15
    # blocks whose low nibbles are all 0 and high all 15, and the reverse
    nib[(sel >= 0.04) & (sel < 0.06), :16] = 0
    nib[(sel >= 0.04) & (sel < 0.06), 16:] = 15
    nib[(sel >= 0.06) & (sel < 0.08), :16] = 15
    nib[(sel >= 0.06) & (sel < 0.08), 16:] = 0
    kq = np.empty(shape + (34,), np.uint8)
    kq[..., 0] = kd & 0xFF
    kq[..., 1] = kd >> 8
    kq[..., 2:] = codes.astype(np.int8).view(np.uint8)
    if type_v == "q8_0":
        vcodes = g.integers(-128, 128, size=shape + (QK,), dtype=np.int16)
        sel = g.random(shape)
        vcodes[sel < 0.03] = -128
        vcodes[(sel >= 0.03) & (sel < 0.06)] = 127
        vcodes[g.random(shape + (QK,)) < 0.05] = -128
        vq = np.empty(shape + (34,), np.uint8)
        vq[..., 0] = vd & 0xFF
        vq[..., 1] = vd >> 8
        vq[..., 2:] = vcodes.astype(np.int8).view(np.uint8)
        return kq, vq
    vq = np.empty(shape + (18,), np.uint8)
    vq[..., 0] = vd & 0xFF
    vq[..., 1] = vd >> 8
    vq[..., 2:] = nib[..., :16] | (nib[..., 16:] << 4)
    return kq, vq


def edge_layer_records(seed, n_kv, n_kv_heads, k_regime, v_regime, head_dim=128, type_v="q4_0"):
    """Page records uint8 [n_pages, page_bytes] of one layer, rows past n_kv
    poisoned (0xFF: NaN scales)."""
    geom = KVGeometry(n_kv_heads, head_dim, type_v=type_v)
    n_pages = -(-n_kv // 256)
    kq, vq = edge_blocks(seed, n_kv, n_kv_heads, head_dim, k_regime, v_regime, type_v)
    return pack_page_records(kq, vq, geom, n_pages)
