"""Random draws, block encoding and page packing for synthetic KV pages.

Page record format (one record per layer and 256-token page), the format the
library documents in its public header:

    [ K tiles: for kv head g, for token row t, for block b: Q8_0 block (34 B) ]
    [ V tiles: for kv head g, for token row t, for block b: Q4_0 block (18 B)
      or, for the q8_0-q8_0 pair, a Q8_0 block (34 B) ]

A Q8_0 block is a little-endian binary16 scale followed by 32 two's-complement
bytes; a Q4_0 block is a binary16 scale followed by 16 bytes whose low nibble
holds element j and whose high nibble holds element j + 16. These are the
ggml block types named on page 1 ("What it is useful for": Q8_0 K / Q4_0 V).

The quantizers below only manufacture test inputs. They follow the usual ggml
reference rules (Q8_0: scale = max|x| / 127, codes rounded half away from zero;
Q4_0: scale = (signed element of largest magnitude) / -8, codes
min(15, trunc(x / d + 8.5))), computed in float32 with the scale stored as the
nearest binary16. Any deterministic rule would do: parity is checked from the
bytes onward.
"""

from dataclasses import dataclass
import math

import numpy as np

SEED_TAG = 0x6B7673  # ASCII "kvs"
STREAM_K, STREAM_V, STREAM_Q, STREAM_RESIDENCY = 0, 1, 2, 3
QK = 32
Q8_0_BLOCK = 34
Q4_0_BLOCK = 18
POISON_BYTE = 0xFF   # a binary16 scale of 0xFFFF is a NaN


@dataclass(frozen=True)
class KVGeometry:
    n_kv_heads: int
    head_dim: int
    page_tokens: int = 256
    type_v: str = "q4_0"     # "q4_0" or "q8_0" (K is always Q8_0)

    @property
    def v_block(self) -> int:           # bytes of one V block
        return Q8_0_BLOCK if self.type_v == "q8_0" else Q4_0_BLOCK

    @property
    def nb(self) -> int:
        return self.head_dim // QK

    @property
    def k_tile_bytes(self) -> int:      # one kv head's K for one page
        return self.page_tokens * self.nb * Q8_0_BLOCK

    @property
    def v_tile_bytes(self) -> int:      # one kv head's V for one page
        return self.page_tokens * self.nb * self.v_block

    @property
    def k_region_bytes(self) -> int:
        return self.n_kv_heads * self.k_tile_bytes

    @property
    def page_bytes(self) -> int:
        return self.n_kv_heads * (self.k_tile_bytes + self.v_tile_bytes)


def rng_for(cid: int, layer: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_TAG, cid, layer, stream])))


def quantize_q8_0(x: np.ndarray) -> np.ndarray:
    """float32 [..., 32] -> uint8 [..., 34] Q8_0 blocks."""
    x = np.asarray(x, dtype=np.float32)
    assert x.shape[-1] == QK
    amax = np.max(np.abs(x), axis=-1)
    d = (amax / np.float32(127.0)).astype(np.float32)
    inv = np.zeros_like(d)
    nz = d != 0
    inv[nz] = np.float32(1.0) / d[nz]
    v = (x * inv[..., None]).astype(np.float32)
    v64 = v.astype(np.float64)          # exact: round half away from zero without f32 re-rounding
    q = np.trunc(v64 + np.copysign(0.5, v64))
    q = np.clip(q, -127, 127).astype(np.int8)
    out = np.empty(x.shape[:-1] + (Q8_0_BLOCK,), dtype=np.uint8)
    out[..., 0:2] = d.astype(np.float16).view(np.uint16)[..., None].view(np.uint8).reshape(d.shape + (2,))
    out[..., 2:] = q.view(np.uint8)
    return out


def quantize_q4_0(x: np.ndarray) -> np.ndarray:
    """float32 [..., 32] -> uint8 [..., 18] Q4_0 blocks."""
    x = np.asarray(x, dtype=np.float32)
    assert x.shape[-1] == QK
    idx = np.argmax(np.abs(x), axis=-1)
    m = np.take_along_axis(x, idx[..., None], axis=-1)[..., 0]
    d = (m / np.float32(-8.0)).astype(np.float32)
    inv = np.zeros_like(d)
    nz = d != 0
    inv[nz] = np.float32(1.0) / d[nz]
    v = (x * inv[..., None]).astype(np.float32) + np.float32(8.5)
    q = np.minimum(np.trunc(v), 15).astype(np.uint8)
    out = np.empty(x.shape[:-1] + (Q4_0_BLOCK,), dtype=np.uint8)
    out[..., 0:2] = d.astype(np.float16).view(np.uint16)[..., None].view(np.uint8).reshape(d.shape + (2,))
    out[..., 2:] = q[..., :16] | (q[..., 16:] << 4)
    return out


def pack_page_records(kq: np.ndarray, vq: np.ndarray, geom: KVGeometry, n_pages: int,
                      out: np.ndarray | None = None, first_page: int = 0,
                      tail: str = "poison") -> np.ndarray:
    """Pack token-major blocks into page records.

    kq: uint8 [n_tok, Hkv, nb, 34]; vq: uint8 [n_tok, Hkv, nb, geom.v_block],
    tokens starting at page `first_page`. Rows past n_tok in the last page are filled
    with 0xFF ("poison": NaN scales) or zeros.
    """
    T, H, nb = geom.page_tokens, geom.n_kv_heads, geom.nb
    n_tok = kq.shape[0]
    VB = geom.v_block
    assert kq.shape == (n_tok, H, nb, Q8_0_BLOCK) and vq.shape == (n_tok, H, nb, VB)
    assert n_tok <= n_pages * T
    if out is None:
        out = np.empty((first_page + n_pages, geom.page_bytes), dtype=np.uint8)
    fill = POISON_BYTE if tail == "poison" else 0
    pad = n_pages * T - n_tok
    if pad:
        kq = np.concatenate([kq, np.full((pad, H, nb, Q8_0_BLOCK), fill, np.uint8)])
        vq = np.concatenate([vq, np.full((pad, H, nb, VB), fill, np.uint8)])
    # [pages, T, H, nb, B] -> [pages, H, T, nb, B]
    k = kq.reshape(n_pages, T, H, nb, Q8_0_BLOCK).transpose(0, 2, 1, 3, 4).reshape(n_pages, -1)
    v = vq.reshape(n_pages, T, H, nb, VB).transpose(0, 2, 1, 3, 4).reshape(n_pages, -1)
    dst = out[first_page:first_page + n_pages]
    dst[:, :geom.k_region_bytes] = k
    dst[:, geom.k_region_bytes:] = v
    return out


def layer_records(cid: int, layer: int, n_kv: int, geom: KVGeometry, tail: str = "poison",
                  out: np.ndarray | None = None, slab_pages: int = 64) -> np.ndarray:
    """Page records for one layer: K and V drawn from N(0,1) token-major
    [n_kv, Hkv, head_dim] (one stream each), quantized per 32-run."""
    T, H, d = geom.page_tokens, geom.n_kv_heads, geom.head_dim
    n_pages = -(-n_kv // T)
    if out is None:
        out = np.empty((n_pages, geom.page_bytes), dtype=np.uint8)
    assert out.shape == (n_pages, geom.page_bytes) and out.dtype == np.uint8
    rk, rv = rng_for(cid, layer, STREAM_K), rng_for(cid, layer, STREAM_V)
    for p0 in range(0, n_pages, slab_pages):
        np_ = min(slab_pages, n_pages - p0)
        t0, t1 = p0 * T, min(n_kv, (p0 + np_) * T)
        kx = rk.standard_normal((t1 - t0, H, d), dtype=np.float32)
        vx = rv.standard_normal((t1 - t0, H, d), dtype=np.float32)
        kq = quantize_q8_0(kx.reshape(t1 - t0, H, d // QK, QK))
        vq = (quantize_q8_0 if geom.type_v == "q8_0" else quantize_q4_0)(vx.reshape(t1 - t0, H, d // QK, QK))
        pack_page_records(kq, vq, geom, np_, out=out, first_page=p0, tail=tail)
    return out


def poison_tail(records: np.ndarray, n_kv: int, geom: KVGeometry) -> None:
    """Overwrite rows at or past n_kv with 0xFF in place (NaN scales)."""
    T = geom.page_tokens
    n_pages = records.shape[0]
    for t in range(n_kv, n_pages * T):
        p, r = divmod(t, T)
        for g in range(geom.n_kv_heads):
            k0 = g * geom.k_tile_bytes + r * geom.nb * Q8_0_BLOCK
            records[p, k0:k0 + geom.nb * Q8_0_BLOCK] = POISON_BYTE
            v0 = geom.k_region_bytes + g * geom.v_tile_bytes + r * geom.nb * geom.v_block
            records[p, v0:v0 + geom.nb * geom.v_block] = POISON_BYTE


def make_q(cid: int, layer: int, n_q: int, n_q_heads: int, head_dim: int, dtype: str) -> np.ndarray:
    """Queries: float32 N(0,1)/sqrt(head_dim) ("f32"), or N(0,1) rounded to float16 ("f16")."""
    r = rng_for(cid, layer, STREAM_Q)
    x = r.standard_normal((n_q, n_q_heads, head_dim), dtype=np.float32)
    if dtype == "f32":
        return (x / np.float32(math.sqrt(head_dim))).astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    raise ValueError(dtype)


def residency_mask(cid: int, layer: int, n_pages: int, n_resident: int,
                   own_page: bool = False) -> np.ndarray:
    """uint8 [n_pages], 1 = resident. The most recent ceil(R/2) pages plus
    floor(R/2) older pages drawn without replacement (seeded per layer). With
    own_page, the last page (a prefill ubatch's own rows) is always resident
    and R counts the prefix only."""
    mask = np.zeros(n_pages, dtype=np.uint8)
    n_prefix = n_pages - (1 if own_page else 0)
    if own_page and n_pages:
        mask[-1] = 1
    R = max(0, min(n_resident, n_prefix))
    recent = -(-R // 2)
    mask[n_prefix - recent:n_prefix] = 1
    older = R - recent
    if older:
        pick = rng_for(cid, layer, STREAM_RESIDENCY).choice(n_prefix - recent, size=older, replace=False)
        mask[pick] = 1
    return mask
