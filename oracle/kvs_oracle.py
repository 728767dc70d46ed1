"""Float64 reference for dequantization, page gathers and attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): the library never
imports this module.

Definitions followed, all written out directly:
  * Q8_0 block (34 B): a binary16 scale d, then 32 signed bytes q; element i
    is d * q[i]. Q4_0 block (18 B): a binary16 scale d, then 16 bytes; byte j
    holds element j in its low nibble and element j + 16 in its high nibble;
    element i is d * (nibble - 8). These are the ggml types the pages run
    their cache in (page 1, "What it is useful for"; page 2, "TLDR": the
    q8_0-q4_0 pair). V may also be Q8_0 (page 3, "1. Correctness - PPL
    parity": the q8_0-q8_0 pair); K is Q8_0 in both pairs.
  * A page is 256 consecutive token rows of one layer (page 2, "Dynamic draft
    eject": the keep threshold counts 256-token pages). Token t lives in page
    t // 256, row t % 256. Within a page record, the K tiles of every kv head
    come first (head-major, then token row, then block), then the V tiles in
    the same order.
  * Attention: query i at position q_pos0 + i, head h, reads kv head
    h // (Hq / Hkv). Its allowed keys are t < n_kv, and t <= q_pos0 + i when
    causal. s_t = scale * sum_c q[i,h,c] K[t,g,c]; m = max s_t;
    p_t = exp(s_t - m); l = sum p_t; out = sum p_t V[t,g,:] / l;
    lse = m + ln l. A row with no allowed key gives out = 0, lse = -inf.
    Streaming moves bytes only, so the result does not depend on which pages
    are resident (page 3, "KLD": the same math, reordered).
"""

import math

import numpy as np

QK = 32
Q8_0_BYTES = 34
Q4_0_BYTES = 18
F16_BYTES = 2

_BLOCK = {  # (bytes per block, values per block)
    "q8_0": (Q8_0_BYTES, QK),
    "q4_0": (Q4_0_BYTES, QK),
    "f16": (F16_BYTES, 1),
}


def f16_to_f64(bits) -> np.ndarray:
    """Exact value of IEEE 754 binary16 encodings (uint16), as float64.

    sign = bit 15, exponent = bits 10..14 (bias 15), fraction = bits 0..9.
    Exponent 0 is subnormal (2^-14 * f/1024); exponent 31 is inf or NaN.
    """
    bits = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where((bits >> 15) & 1, -1.0, 1.0)
    e = (bits >> 10) & 0x1F
    f = (bits & 0x3FF).astype(np.float64)
    normal = np.ldexp(1.0 + f / 1024.0, (e - 15).astype(np.int32))
    sub = np.ldexp(f / 1024.0, -14)
    mag = np.where(e == 0, sub, normal)
    mag = np.where(e == 31, np.where(f == 0, np.inf, np.nan), mag)
    return sign * mag


def _scale(blocks: np.ndarray) -> np.ndarray:
    b = blocks.astype(np.uint16)
    return f16_to_f64(b[..., 0] | (b[..., 1] << 8))


def dequant_q8_0(blocks) -> np.ndarray:
    """uint8 [..., 34] -> float64 [..., 32]."""
    blocks = np.asarray(blocks, dtype=np.uint8)
    assert blocks.shape[-1] == Q8_0_BYTES
    d = _scale(blocks)
    q = np.ascontiguousarray(blocks[..., 2:]).view(np.int8).astype(np.float64)
    return d[..., None] * q


def dequant_q4_0(blocks) -> np.ndarray:
    """uint8 [..., 18] -> float64 [..., 32]."""
    blocks = np.asarray(blocks, dtype=np.uint8)
    assert blocks.shape[-1] == Q4_0_BYTES
    d = _scale(blocks)
    qs = blocks[..., 2:]
    nib = np.concatenate([qs & 0x0F, qs >> 4], axis=-1).astype(np.float64)
    return d[..., None] * (nib - 8.0)


def page_bytes(n_kv_heads: int, head_dim: int, page_tokens: int = 256,
               type_k: str = "q8_0", type_v: str = "q4_0") -> int:
    """Bytes of one page record (one layer, page_tokens rows of K and V)."""
    def row(t):
        nbytes, nvals = _BLOCK[t]
        assert head_dim % nvals == 0
        return n_kv_heads * (head_dim // nvals) * nbytes
    return page_tokens * (row(type_k) + row(type_v))


_DEQUANT_V = {"q4_0": dequant_q4_0, "q8_0": dequant_q8_0}


def gather_kv(records: np.ndarray, n_kv_heads: int, head_dim: int, tok0: int, n_tok: int,
              page_tokens: int = 256, type_v: str = "q4_0"):
    """Dequantized K and V (float64 [n_tok, Hkv, head_dim]) for tokens
    tok0 .. tok0 + n_tok - 1, read from host page records uint8 [n_pages, page_bytes].
    K blocks are Q8_0; V blocks are `type_v` ("q4_0" or "q8_0")."""
    T, H = page_tokens, n_kv_heads
    nb = head_dim // QK
    vbytes = _BLOCK[type_v][0]
    records = np.asarray(records, dtype=np.uint8)
    assert records.shape[1] == page_bytes(H, head_dim, T, "q8_0", type_v)
    if n_tok == 0:
        z = np.zeros((0, H, head_dim))
        return z, z.copy()
    p0, p1 = tok0 // T, (tok0 + n_tok - 1) // T + 1
    assert p1 <= records.shape[0]
    rec = records[p0:p1]
    kbytes = H * T * nb * Q8_0_BYTES
    kb = rec[:, :kbytes].reshape(p1 - p0, H, T, nb, Q8_0_BYTES)
    vb = rec[:, kbytes:kbytes + H * T * nb * vbytes].reshape(p1 - p0, H, T, nb, vbytes)
    # [pages, H, T, nb, 32] -> [pages, T, H, nb*32] -> tokens
    k = dequant_q8_0(kb).transpose(0, 2, 1, 3, 4).reshape((p1 - p0) * T, H, head_dim)
    v = _DEQUANT_V[type_v](vb).transpose(0, 2, 1, 3, 4).reshape((p1 - p0) * T, H, head_dim)
    lo = tok0 - p0 * T
    return k[lo:lo + n_tok], v[lo:lo + n_tok]


def attend(q, K, V, *, n_kv: int, scale: float, causal: bool, q_pos0: int,
           heads=None):
    """Softmax attention in float64.

    q: [n_q, Hq, d] (float32 or float16, converted exactly); K, V: float64
    [>= n_kv, Hkv, d] holding tokens 0 .. n_kv-1. heads: optional list of
    query heads to compute (others are left as NaN). Returns
    (out float64 [n_q, Hq, d], lse float64 [n_q, Hq]).
    """
    q = np.asarray(q).astype(np.float64)
    n_q, Hq, d = q.shape
    Hkv = K.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    out = np.full((n_q, Hq, d), np.nan)
    lse = np.full((n_q, Hq), np.nan)
    hs_all = range(Hq) if heads is None else heads
    for i in range(n_q):
        lim = min(n_kv, q_pos0 + i + 1) if causal else n_kv
        for h in hs_all:
            if lim <= 0:
                out[i, h] = 0.0
                lse[i, h] = -math.inf
                continue
            g = h // G
            s = float(scale) * (K[:lim, g, :] @ q[i, h, :])
            m = s.max()
            p = np.exp(s - m)
            l = p.sum()
            out[i, h] = (p @ V[:lim, g, :]) / l
            lse[i, h] = m + math.log(l)
    return out, lse


def attend_layer(records, q, *, n_kv: int, n_kv_heads: int, head_dim: int, scale: float,
                 causal: bool, q_pos0: int, heads=None, page_tokens: int = 256,
                 type_v: str = "q4_0"):
    """Gather the whole layer from its host records, then attend."""
    K, V = gather_kv(records, n_kv_heads, head_dim, 0, n_kv, page_tokens, type_v)
    return attend(q, K, V, n_kv=n_kv, scale=scale, causal=causal, q_pos0=q_pos0, heads=heads)


# ---------------------------------------------------------------------------
# KV append: quantizing a step's new K and V rows into the page records.
#
# The rule is the ggml reference quantizer for each block type (the pages
# name the types only; their blocks come from llama.cpp's quantizers), in
# float32 with the scale stored as the nearest binary16:
#   Q8_0: amax = max |x_i|; d = amax / 127; id = 1 / d (0 when d = 0);
#         q_i = round-half-away-from-zero(x_i * id), kept within [-127, 127].
#   Q4_0: m = the element of largest magnitude (the first one on ties; +0 for
#         an all-zero block); d = m / -8; id = 1 / d (0 when d = 0);
#         nibble_i = min(15, trunc(x_i * id + 8.5)).
# Each step below is one float32 operation, rounded to nearest even, written
# out one element at a time so that it can be read against the rule.
# Inputs must be finite, with a block's max |x| either 0 or at least 2^-100
# (so that 1 / d stays finite).
# ---------------------------------------------------------------------------

def _f16_bits(d32) -> int:
    return int(np.array([d32], dtype=np.float32).astype(np.float16).view(np.uint16)[0])


def quantize_q8_0_block(x) -> np.ndarray:
    """32 float32 values -> one Q8_0 block (uint8 [34])."""
    x = np.asarray(x, dtype=np.float32)
    assert x.shape == (QK,)
    amax = np.float32(0.0)
    for v in x:
        a = np.float32(abs(v))
        if a > amax:
            amax = a
    d = np.float32(amax / np.float32(127.0))
    inv = np.float32(np.float32(1.0) / d) if d != 0 else np.float32(0.0)
    out = np.zeros(Q8_0_BYTES, dtype=np.uint8)
    bits = _f16_bits(d)
    out[0], out[1] = bits & 0xFF, bits >> 8
    for i, v in enumerate(x):
        y = float(np.float32(v * inv))            # a float32 value, exact as a Python float
        r = math.floor(abs(y) + 0.5)              # exact: |y| + 0.5 is exact in float64
        q = int(math.copysign(r, y)) if r else 0
        q = max(-127, min(127, q))
        out[2 + i] = q & 0xFF
    return out


def quantize_q4_0_block(x) -> np.ndarray:
    """32 float32 values -> one Q4_0 block (uint8 [18])."""
    x = np.asarray(x, dtype=np.float32)
    assert x.shape == (QK,)
    amax, m = np.float32(0.0), np.float32(0.0)
    for v in x:
        a = np.float32(abs(v))
        if a > amax:
            amax, m = a, v
    d = np.float32(m / np.float32(-8.0))
    inv = np.float32(np.float32(1.0) / d) if d != 0 else np.float32(0.0)
    nib = []
    for v in x:
        y = np.float32(np.float32(v * inv) + np.float32(8.5))
        nib.append(min(15, int(math.trunc(float(y)))))
    out = np.zeros(Q4_0_BYTES, dtype=np.uint8)
    bits = _f16_bits(d)
    out[0], out[1] = bits & 0xFF, bits >> 8
    for j in range(16):
        out[2 + j] = nib[j] | (nib[j + 16] << 4)
    return out


def append_rows(records, k_new, v_new, *, pos0: int, n_kv_heads: int, head_dim: int,
                page_tokens: int = 256, type_v: str = "q4_0") -> np.ndarray:
    """Copy of the page records (uint8 [n_pages, page_bytes]) with tokens
    pos0 .. pos0 + n - 1 replaced by the quantized rows of k_new / v_new
    ([n, Hkv, head_dim]; float16 inputs are widened to float32 exactly), K
    as Q8_0 and V as `type_v`. Token t goes to page t // page_tokens, row
    t % page_tokens; every other byte is kept."""
    recs = np.array(records, dtype=np.uint8, copy=True)
    k_new = np.asarray(k_new).astype(np.float32)
    v_new = np.asarray(v_new).astype(np.float32)
    n, H, T = k_new.shape[0], n_kv_heads, page_tokens
    nb = head_dim // QK
    assert k_new.shape == (n, H, head_dim) and v_new.shape == (n, H, head_dim)
    assert recs.shape[1] == page_bytes(H, head_dim, T, "q8_0", type_v)
    vbytes = _BLOCK[type_v][0]
    quant_v = quantize_q8_0_block if type_v == "q8_0" else quantize_q4_0_block
    k_tile, v_tile = T * nb * Q8_0_BYTES, T * nb * vbytes
    for i in range(n):
        t = pos0 + i
        page, r = t // T, t % T
        assert page < recs.shape[0]
        for g in range(H):
            for b in range(nb):
                ko = g * k_tile + (r * nb + b) * Q8_0_BYTES
                recs[page, ko:ko + Q8_0_BYTES] = quantize_q8_0_block(k_new[i, g, b * QK:(b + 1) * QK])
                vo = H * k_tile + g * v_tile + (r * nb + b) * vbytes
                recs[page, vo:vo + vbytes] = quant_v(v_new[i, g, b * QK:(b + 1) * QK])
    return recs
