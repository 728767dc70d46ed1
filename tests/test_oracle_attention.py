"""Pins for the oracle's page gather and attention.

The gather is pinned by hand-placed sentinel blocks. Attention is pinned by a
50-digit mpmath brute force on tiny inputs (decoding the raw bytes with its
own loops) and by closed forms: a single key, a zero scale (plain means and
lse = ln n), a dominant key, GQA head constants, causal prefix means, ragged
tails with NaN-poisoned rows, log-sum-exp split invariance and key
permutation invariance.
"""

import math

import mpmath
import numpy as np
import pytest

from oracle import attend, attend_layer, gather_kv, page_bytes
from kvs_synth import KVGeometry, layer_records, make_q, quantize_q4_0, quantize_q8_0, pack_page_records


def sentinel_records(n_pages, H, d, T):
    """Records whose every block encodes its own (page, head, row, block)."""
    nb = d // 32
    rec = np.zeros((n_pages, page_bytes(H, d, T)), np.uint8)
    kbytes = H * T * nb * 34
    for p in range(n_pages):
        for g in range(H):
            for r in range(T):
                for b in range(nb):
                    o = ((g * T + r) * nb + b) * 34
                    rec[p, o:o + 2] = (0x00, 0x3C)                  # d = 1
                    codes = np.arange(32, dtype=np.int64) - 16
                    codes[0], codes[1], codes[2], codes[3] = p, g, r - 128, b
                    rec[p, o + 2:o + 34] = codes.astype(np.int8).view(np.uint8)
                    o = kbytes + ((g * T + r) * nb + b) * 18
                    rec[p, o:o + 2] = (0x00, 0x3C)
                    nib = np.full(32, 8, np.uint8)
                    nib[0], nib[1], nib[2], nib[3], nib[4], nib[5] = g, b, r & 15, r >> 4, p & 15, p >> 4
                    rec[p, o + 2:o + 18] = nib[:16] | (nib[16:] << 4)
    return rec


def test_gather_sentinels():
    H, d, T = 3, 64, 16
    rec = sentinel_records(4, H, d, T)
    for tok0, n_tok in [(0, 64), (5, 30), (17, 1), (63, 1), (31, 2)]:
        K, V = gather_kv(rec, H, d, tok0, n_tok, page_tokens=T)
        assert K.shape == (n_tok, H, d) and V.shape == (n_tok, H, d)
        for i in range(n_tok):
            t = tok0 + i
            p, r = divmod(t, T)
            for g in range(H):
                for b in range(d // 32):
                    k = K[i, g, 32 * b:32 * b + 32]
                    assert (k[0], k[1], k[2], k[3]) == (p, g, r - 128, b)
                    assert np.array_equal(k[4:], np.arange(4, 32) - 16)
                    v = V[i, g, 32 * b:32 * b + 32] + 8
                    assert (v[0], v[1], v[2], v[3], v[4], v[5]) == (g, b, r & 15, r >> 4, p & 15, p >> 4)
                    assert np.all(v[6:] == 8)


def sentinel_records_q8v(n_pages, H, d, T):
    """q8_0-q8_0 records: K blocks as in sentinel_records, V blocks Q8_0 with
    d = -2 and codes (b, g, r - 128, p, r & 7, then 60 - j)."""
    nb = d // 32
    rec = np.zeros((n_pages, page_bytes(H, d, T, "q8_0", "q8_0")), np.uint8)
    kbytes = H * T * nb * 34
    for p in range(n_pages):
        for g in range(H):
            for r in range(T):
                for b in range(nb):
                    o = ((g * T + r) * nb + b) * 34
                    rec[p, o:o + 2] = (0x00, 0x3C)
                    codes = np.arange(32, dtype=np.int64) - 16
                    codes[0], codes[1], codes[2], codes[3] = p, g, r - 128, b
                    rec[p, o + 2:o + 34] = codes.astype(np.int8).view(np.uint8)
                    o = kbytes + ((g * T + r) * nb + b) * 34
                    rec[p, o:o + 2] = (0x00, 0xC0)                  # d = -2
                    codes = 60 - np.arange(32, dtype=np.int64)
                    codes[0], codes[1], codes[2], codes[3], codes[4] = b, g, r - 128, p, r & 7
                    rec[p, o + 2:o + 34] = codes.astype(np.int8).view(np.uint8)
    return rec


def test_gather_sentinels_q8_0_v():
    H, d, T = 3, 64, 16
    rec = sentinel_records_q8v(4, H, d, T)
    for tok0, n_tok in [(0, 64), (5, 30), (17, 1), (63, 1)]:
        K, V = gather_kv(rec, H, d, tok0, n_tok, page_tokens=T, type_v="q8_0")
        assert K.shape == (n_tok, H, d) and V.shape == (n_tok, H, d)
        for i in range(n_tok):
            p, r = divmod(tok0 + i, T)
            for g in range(H):
                for b in range(d // 32):
                    k = K[i, g, 32 * b:32 * b + 32]
                    assert (k[0], k[1], k[2], k[3]) == (p, g, r - 128, b)
                    v = V[i, g, 32 * b:32 * b + 32] / -2.0
                    assert (v[0], v[1], v[2], v[3], v[4]) == (b, g, r - 128, p, r & 7)
                    assert np.array_equal(v[5:], 60 - np.arange(5, 32))
    # the same bytes read with the other V type give a different layout: the
    # record size alone already tells them apart
    with pytest.raises(AssertionError):
        gather_kv(rec, H, d, 0, 1, page_tokens=T, type_v="q4_0")


def small_case(cid, H, Hq, d, n_kv, T, n_q=1, q_dtype="f32", layer=0, type_v="q4_0"):
    geom = KVGeometry(H, d, T, type_v)
    rec = layer_records(cid, layer, n_kv, geom, tail="poison")
    q = make_q(cid, layer, n_q, Hq, d, q_dtype)
    return rec, q


def brute_force(rec, q, n_kv, H, d, T, scale, causal, q_pos0, type_v="q4_0"):
    """50-digit attention straight from the record bytes, with explicit loops."""
    mpmath.mp.dps = 50
    nb = d // 32
    kbytes = H * T * nb * 34

    def f16(lo, hi):
        return mpmath.mpf(float(np.array([lo | (hi << 8)], np.uint16).view(np.float16)[0]))

    def kval(t, g, c):
        p, r = divmod(t, T)
        o = ((g * T + r) * nb + c // 32) * 34
        blk = rec[p, o:o + 34]
        qv = int(blk[2 + c % 32])
        qv = qv - 256 if qv >= 128 else qv
        return f16(int(blk[0]), int(blk[1])) * qv

    def vval(t, g, c):
        p, r = divmod(t, T)
        if type_v == "q8_0":
            o = kbytes + ((g * T + r) * nb + c // 32) * 34
            blk = rec[p, o:o + 34]
            qv = int(blk[2 + c % 32])
            qv = qv - 256 if qv >= 128 else qv
            return f16(int(blk[0]), int(blk[1])) * qv
        o = kbytes + ((g * T + r) * nb + c // 32) * 18
        blk = rec[p, o:o + 18]
        j = c % 32
        nib = int(blk[2 + j]) & 15 if j < 16 else int(blk[2 + j - 16]) >> 4
        return f16(int(blk[0]), int(blk[1])) * (nib - 8)

    n_q, Hq, _ = q.shape
    G = Hq // H
    out = np.zeros((n_q, Hq, d))
    lse = np.zeros((n_q, Hq))
    Kc = {(t, g): [kval(t, g, c) for c in range(d)] for t in range(n_kv) for g in range(H)}
    Vc = {(t, g): [vval(t, g, c) for c in range(d)] for t in range(n_kv) for g in range(H)}
    for i in range(n_q):
        lim = min(n_kv, q_pos0 + i + 1) if causal else n_kv
        for h in range(Hq):
            g = h // G
            qv = [mpmath.mpf(float(x)) for x in q[i, h]]
            s = [mpmath.mpf(scale) * mpmath.fsum(qv[c] * Kc[(t, g)][c] for c in range(d)) for t in range(lim)]
            w = [mpmath.exp(x) for x in s]
            l = mpmath.fsum(w)
            for c in range(d):
                out[i, h, c] = float(mpmath.fsum(w[t] * Vc[(t, g)][c] for t in range(lim)) / l)
            lse[i, h] = float(mpmath.log(l))
    return out, lse


@pytest.mark.parametrize("n_kv,causal,n_q,q_dtype,type_v", [(37, False, 1, "f32", "q4_0"), (40, True, 3, "f16", "q4_0"),
                                                             (37, False, 1, "f32", "q8_0"), (40, True, 3, "f16", "q8_0")])
def test_brute_force_tiny(n_kv, causal, n_q, q_dtype, type_v):
    H, Hq, d, T = 2, 6, 32, 16
    rec, q = small_case(11, H, Hq, d, n_kv, T, n_q=n_q, q_dtype=q_dtype, type_v=type_v)
    scale = 1.0 if q_dtype == "f32" else 1.0 / math.sqrt(d)
    q_pos0 = n_kv - n_q
    out, lse = attend_layer(rec, q, n_kv=n_kv, n_kv_heads=H, head_dim=d, scale=scale,
                            causal=causal, q_pos0=q_pos0, page_tokens=T, type_v=type_v)
    bo, bl = brute_force(rec, q, n_kv, H, d, T, scale, causal, q_pos0, type_v)
    assert np.max(np.abs(out - bo)) <= 1e-12 * max(1.0, np.max(np.abs(bo)))
    assert np.max(np.abs(lse - bl)) <= 1e-12 * max(1.0, np.max(np.abs(bl)))


def test_single_key_returns_its_value():
    H, Hq, d, T = 2, 4, 64, 16
    rec, q = small_case(12, H, Hq, d, 1, T)
    K, V = gather_kv(rec, H, d, 0, 1, T)
    out, lse = attend(q, K, V, n_kv=1, scale=1.0, causal=False, q_pos0=0)
    for h in range(Hq):
        assert np.array_equal(out[0, h], V[0, h // 2])
        s = float(np.dot(q[0, h].astype(np.float64), K[0, h // 2]))
        assert abs(lse[0, h] - s) <= 1e-12 * max(1.0, abs(s))


def test_zero_scale_gives_mean_and_log_n():
    H, Hq, d, T = 2, 4, 64, 16
    n_kv = 45
    rec, q = small_case(13, H, Hq, d, n_kv, T)
    K, V = gather_kv(rec, H, d, 0, n_kv, T)
    out, lse = attend(q, K, V, n_kv=n_kv, scale=0.0, causal=False, q_pos0=0)
    for h in range(Hq):
        mean = np.array([math.fsum(V[:, h // 2, c]) / n_kv for c in range(d)])
        assert np.max(np.abs(out[0, h] - mean)) <= 1e-14
        assert abs(lse[0, h] - math.log(n_kv)) <= 1e-14


def test_causal_prefix_means_pin_the_boundary():
    H, Hq, d, T = 1, 2, 32, 16
    n_kv, n_q = 50, 4
    rec, q = small_case(14, H, Hq, d, n_kv, T, n_q=n_q)
    K, V = gather_kv(rec, H, d, 0, n_kv, T)
    q_pos0 = 20
    out, lse = attend(q, K, V, n_kv=n_kv, scale=0.0, causal=True, q_pos0=q_pos0)
    for i in range(n_q):
        n = q_pos0 + i + 1          # keys 0 .. q_pos0 + i inclusive
        mean = V[:n, 0].sum(axis=0) / n
        assert np.max(np.abs(out[i, 0] - mean)) <= 1e-14
        assert abs(lse[i, 0] - math.log(n)) <= 1e-14


def test_dominant_key_wins_with_the_right_sign():
    H, Hq, d, T = 1, 1, 64, 16
    n_kv = 30
    rec, _ = small_case(15, H, Hq, d, n_kv, T)
    K, V = gather_kv(rec, H, d, 0, n_kv, T)
    j = 17
    q = (K[j, 0] / np.linalg.norm(K[j, 0]) * 0.2).astype(np.float32)[None, None, :]
    out, _ = attend(q, K, V, n_kv=n_kv, scale=400.0, causal=False, q_pos0=0)
    assert np.max(np.abs(out[0, 0] - V[j, 0])) <= 1e-6


def test_gqa_head_mapping_is_contiguous():
    """kv head g has V == g + 1 everywhere, so query head h returns h // G + 1."""
    H, G, d, T = 4, 3, 32, 16
    n_kv = 20
    geom = KVGeometry(H, d, T)
    rng = np.random.default_rng(3)
    kq = quantize_q8_0(rng.standard_normal((n_kv, H, 1, 32)).astype(np.float32))
    vq = np.zeros((n_kv, H, 1, 18), np.uint8)
    vq[..., 0:2] = (0x00, 0x3C)
    for g in range(H):
        nib = 8 + g + 1
        vq[:, g, 0, 2:] = nib | (nib << 4)
    rec = pack_page_records(kq, vq, geom, 2)
    q = make_q(16, 0, 1, H * G, d, "f32")
    out, _ = attend_layer(rec, q, n_kv=n_kv, n_kv_heads=H, head_dim=d, scale=1.0, causal=False,
                          q_pos0=0, page_tokens=T)
    for h in range(H * G):
        assert np.max(np.abs(out[0, h] - (h // G + 1))) <= 1e-13


def test_ragged_tail_with_poisoned_rows_is_ignored():
    H, Hq, d, T = 2, 2, 32, 16
    n_kv = 37                       # 3 pages, 11 poisoned rows in the last
    rec, q = small_case(17, H, Hq, d, n_kv, T)
    assert rec.shape[0] == 3
    out, lse = attend_layer(rec, q, n_kv=n_kv, n_kv_heads=H, head_dim=d, scale=0.0, causal=False,
                            q_pos0=0, page_tokens=T)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    K, V = gather_kv(rec, H, d, 0, n_kv, T)
    for h in range(Hq):
        assert np.max(np.abs(out[0, h] - V[:, h].mean(axis=0))) <= 1e-14
    # the poisoned rows really are NaN if read
    Kall, _ = gather_kv(rec, H, d, 0, 48, T)
    assert np.all(np.isnan(Kall[n_kv:]))


def test_empty_cache_gives_zero_and_minus_inf():
    q = np.ones((1, 2, 32), np.float32)
    z = np.zeros((0, 1, 32))
    out, lse = attend(q, z, z, n_kv=0, scale=1.0, causal=False, q_pos0=0)
    assert np.all(out == 0.0) and np.all(lse == -math.inf)


def test_lse_split_invariance():
    """Attending to disjoint key ranges and merging with log-sum-exp weights
    reproduces one pass over all keys."""
    H, Hq, d, T = 2, 6, 64, 16
    n_kv = 90
    rec, q = small_case(18, H, Hq, d, n_kv, T, n_q=2)
    K, V = gather_kv(rec, H, d, 0, n_kv, T)
    full, full_lse = attend(q, K, V, n_kv=n_kv, scale=1.0, causal=False, q_pos0=0)
    cuts = [0, 7, 16, 40, 41, 90]
    parts = [attend(q, K[a:b], V[a:b], n_kv=b - a, scale=1.0, causal=False, q_pos0=0)
             for a, b in zip(cuts[:-1], cuts[1:])]
    lses = np.stack([p[1] for p in parts])                 # [parts, n_q, Hq]
    M = lses.max(axis=0)
    w = np.exp(lses - M)                                    # relative mass of each part
    merged = sum(w[j][..., None] * parts[j][0] for j in range(len(parts))) / w.sum(axis=0)[..., None]
    assert np.max(np.abs(merged - full)) <= 1e-12
    assert np.max(np.abs(M + np.log(w.sum(axis=0)) - full_lse)) <= 1e-12


def test_key_permutation_invariance():
    H, Hq, d, T = 1, 3, 32, 16
    n_kv = 33
    rec, q = small_case(19, H, Hq, d, n_kv, T)
    K, V = gather_kv(rec, H, d, 0, n_kv, T)
    perm = np.random.default_rng(0).permutation(n_kv)
    a, la = attend(q, K, V, n_kv=n_kv, scale=1.0, causal=False, q_pos0=0)
    b, lb = attend(q, K[perm], V[perm], n_kv=n_kv, scale=1.0, causal=False, q_pos0=0)
    assert np.max(np.abs(a - b)) <= 1e-14 and np.max(np.abs(la - lb)) <= 1e-13


def test_verify_rows_equal_decode_over_their_prefix():
    H, Hq, d, T = 2, 4, 32, 16
    n_kv, n_q = 60, 4
    rec, q = small_case(20, H, Hq, d, n_kv, T, n_q=n_q)
    K, V = gather_kv(rec, H, d, 0, n_kv, T)
    ver, vl = attend(q, K, V, n_kv=n_kv, scale=1.0, causal=True, q_pos0=n_kv - n_q)
    for i in range(n_q):
        n = n_kv - n_q + i + 1
        dec, dl = attend(q[i:i + 1], K, V, n_kv=n, scale=1.0, causal=False, q_pos0=0)
        assert np.array_equal(ver[i], dec[0]) and np.array_equal(vl[i], dl[0])


def test_identical_queries_in_a_group_give_identical_rows():
    H, Hq, d, T = 2, 6, 32, 16
    n_kv = 40
    rec, q = small_case(21, H, Hq, d, n_kv, T)
    q[0, 1] = q[0, 0]
    q[0, 2] = q[0, 0]
    out, _ = attend_layer(rec, q, n_kv=n_kv, n_kv_heads=H, head_dim=d, scale=1.0, causal=False,
                          q_pos0=0, page_tokens=T)
    assert np.array_equal(out[0, 1], out[0, 0]) and np.array_equal(out[0, 2], out[0, 0])
