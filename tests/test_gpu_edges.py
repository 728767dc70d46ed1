"""Block-format edge cases on the GPU, through the C ABI, against the oracle.

Records are built byte by byte (tests/edge_records.py): Q8_0 codes over the
whole int8 range (-128 included), binary16 scales at the edges (+-65504,
subnormals down to 2^-24, zero, both signs), Q4_0 nibbles 0 and 15 in both
positions, and, for the q8_0-q8_0 pair, Q8_0 V codes over the whole int8
range with V scales either side of 511.75. Checked here:
  * kvs_debug_gather is bit-exact with the oracle's float64 dequantization;
  * attention at decode width (the decode kernel), verify width (the
    matrix-core kernel converting in the kernel) and prefill width (staged
    operands), f32 and f16 queries, is within 2e-3 of the oracle (normwise
    per row; lse within 2e-3 absolute), resident and streamed;
  * the staged matrix-core operands (kvs_debug_stage) equal the exact values
    for K (the codes and scale bits) and the round-to-nearest-even binary16 of
    the exact V element (divided by 8 where a Q4_0 block's scales exceed 8188,
    by 128 where a Q8_0 block's exceed 511.75);
  * an 8-nat score spread at verify and prefill widths stays within 2e-3.
"""

import math

import numpy as np
import pytest
import torch

import host_streamed_paged_amd as kvs
from edge_records import edge_layer_records
from kvs_case import mask_all, mask_random, normwise_error, say
from oracle import attend, f16_to_f64, gather_kv

pytestmark = pytest.mark.gpu

TOL = 2e-3
HKV, HQ = 2, 12
N_KV = 4 * 256 + 77          # 5 pages, ragged tail


class EdgeCase:
    """A pool over hand-built records (one or more layers)."""

    def __init__(self, records, *, max_q, resident_fn, ring=4, chunk=2, group=1, flags=0, type_v="q4_0"):
        self.records = records
        self.type_v = type_v
        self.L = len(records)
        self.n_pages = records[0].shape[0]
        self.host = [torch.from_numpy(r).pin_memory() for r in records]
        self.masks = [np.asarray(resident_fn(l, self.n_pages), np.uint8) for l in range(self.L)]
        self.cfg = kvs.Config(n_layers=self.L, n_kv_heads=HKV, n_q_heads=HQ, max_pages=self.n_pages,
                              max_q_tokens=max_q, ring_pages=ring, chunk_pages=chunk, group_pages=group, flags=flags,
                              type_v=kvs.TYPE_Q8_0 if type_v == "q8_0" else kvs.TYPE_Q4_0)
        self.arena = kvs.Pool.arena_for(self.cfg, int(sum(int(m.sum()) for m in self.masks)))
        self.pool = kvs.Pool(self.cfg, self.arena)
        for l in range(self.L):
            self.pool.host_pages_set(l, self.host[l])
            self.pool.page_table_set(l, self.masks[l])

    def close(self):
        self.pool.close()


def regime_records(k_regime, v_regime, n_layers=2, seed=0, type_v="q4_0"):
    return [edge_layer_records(1000 * seed + 17 * l + 3, N_KV, HKV, k_regime, v_regime, type_v=type_v)
            for l in range(n_layers)]


# (V type, K regime, V regime): scales at the edges of binary16 for K in
# every combination with V regimes inside the documented accuracy range
REGIMES = [("q4_0", "edges", "mixed"), ("q4_0", "big", "big"), ("q4_0", "tiny", "tiny"), ("q4_0", "mixed", "big"),
           ("q4_0", "big", "tiny"), ("q4_0", "tiny", "mixed"),
           ("q8_0", "edges", "mid"), ("q8_0", "big", "big"), ("q8_0", "tiny", "tiny"), ("q8_0", "mixed", "mixed")]
REGIME_IDS = [f"{t}-K{k}-V{v}" for t, k, v in REGIMES]


def key_std(records, l, type_v="q4_0"):
    """Standard deviation of the exact key elements of a layer (sizes the
    softmax scale so scores spread over a few nats)."""
    K, _ = gather_kv(records[l], HKV, 128, 0, N_KV, type_v=type_v)
    s = float(np.sqrt(np.mean(K * K)))
    return s if s > 0 else 1.0


@pytest.mark.parametrize("type_v,k_regime,v_regime", REGIMES, ids=REGIME_IDS)
def test_edge_gather_bit_exact(type_v, k_regime, v_regime):
    recs = regime_records(k_regime, v_regime, type_v=type_v)
    say(f"edge gather {type_v} K={k_regime} V={v_regime}")
    c = EdgeCase(recs, max_q=1, resident_fn=mask_random(0.5, seed=4), type_v=type_v)
    try:
        for l in range(c.L):
            k = torch.empty((N_KV, HKV, 128), dtype=torch.float32, device="cuda")
            v = torch.empty_like(k)
            c.pool.debug_gather(l, 0, N_KV, k, v)
            torch.cuda.synchronize()
            rk, rv = gather_kv(recs[l], HKV, 128, 0, N_KV, type_v=type_v)
            kk, vv = k.cpu().numpy(), v.cpu().numpy()
            # float32 holds every element exactly: compare the bits (signed zeros included)
            assert np.array_equal(kk.view(np.uint32), rk.astype(np.float32).view(np.uint32)), l
            assert np.array_equal(vv.view(np.uint32), rv.astype(np.float32).view(np.uint32)), l
    finally:
        c.close()


# widths: (query tokens, query dtype, causal) -> decode (6 rows per kv head),
# verify (24 rows, matrix cores converting in the kernel), prefill (72 rows,
# staged operands)
WIDTHS = [(1, "f32", False), (4, "f32", True), (12, "f16", True), (12, "f32", True)]


@pytest.mark.parametrize("type_v,k_regime,v_regime", REGIMES, ids=REGIME_IDS)
@pytest.mark.parametrize("n_q,qdt,causal", WIDTHS, ids=["decode", "verify", "prefill-f16", "prefill-f32"])
def test_edge_attention_within_tolerance(type_v, k_regime, v_regime, n_q, qdt, causal):
    recs = regime_records(k_regime, v_regime, seed=1, type_v=type_v)
    g = np.random.default_rng(99)
    worst = 0.0
    for resident in (mask_all, mask_random(0.4, seed=6)):
        say(f"edge attention {type_v} K={k_regime} V={v_regime} n_q={n_q} {qdt} causal={causal} "
            f"residency={getattr(resident, '__name__', 'fn')}")
        c = EdgeCase(recs, max_q=n_q, resident_fn=resident, group=2, type_v=type_v)
        try:
            for l in range(c.L):
                q = g.standard_normal((n_q, HQ, 128)).astype(np.float32)
                q = q.astype(np.float16) if qdt == "f16" else q
                # scores spread over about 2 nats whatever the key magnitudes
                scale = 2.0 / (key_std(recs, l, type_v) * math.sqrt(128))
                q_pos0 = N_KV - n_q
                qd = torch.from_numpy(q).cuda()
                out = torch.empty((n_q, HQ, 128), dtype=torch.float32, device="cuda")
                lse = torch.empty((n_q, HQ), dtype=torch.float32, device="cuda")
                c.pool.attend(l, qd, N_KV, q_pos0, scale, causal, out, lse)
                torch.cuda.synchronize()
                K, V = gather_kv(recs[l], HKV, 128, 0, N_KV, type_v=type_v)
                ref, ref_lse = attend(q, K, V, n_kv=N_KV, scale=scale, causal=causal, q_pos0=q_pos0)
                o = out.cpu().numpy()
                assert np.all(np.isfinite(o)), l
                err = normwise_error(o, ref)
                lerr = float(np.max(np.abs(lse.cpu().numpy() - ref_lse)))
                say(f"layer {l}: normwise {err:.3e} lse {lerr:.3e}")
                assert err <= TOL, (l, err)
                assert lerr <= TOL, (l, lerr)
                worst = max(worst, err)
        finally:
            c.close()
    say(f"worst normwise {worst:.3e}")


@pytest.mark.parametrize("type_v", ["q4_0", "q8_0"])
@pytest.mark.parametrize("n_q,qdt,scale", [(4, "f32", 8.0), (12, "f16", 8.0 / math.sqrt(128)),
                                           (12, "f32", 8.0), (40, "f16", 8.0 / math.sqrt(128))],
                         ids=["verify-f32", "prefill-f16", "prefill-f32", "prefill-f16-40tok"])
def test_eight_nat_score_spread(n_q, qdt, scale, type_v):
    """Scores with a standard deviation of about 8 nats (f32 queries
    N(0,1)/sqrt(128) at scale 8, f16 queries N(0,1) at 8/sqrt(128), over keys
    of unit size): the matrix-core path keeps scores in float32, so the
    output stays within 2e-3."""
    from kvs_case import Case
    say(f"8-nat spread {type_v} n_q={n_q} {qdt} scale={scale:.4f}")
    c = Case(cid=93, n_layers=2, n_kv_heads=HKV, n_q_heads=HQ, n_kv=N_KV,
             cfg_kw=dict(max_q_tokens=n_q, ring_pages=4, chunk_pages=2, group_pages=2),
             resident_fn=mask_random(0.5, seed=2), type_v=type_v)
    try:
        qs = [c.queries(l, n_q, qdt) for l in range(c.L)]
        outs, lses = c.attend_all(qs, q_pos0=N_KV - n_q, scale=scale, causal=True)
        for l in range(c.L):
            ref, ref_lse = c.oracle(l, qs[l], q_pos0=N_KV - n_q, scale=scale, causal=True)
            err = normwise_error(outs[l], ref)
            lerr = float(np.max(np.abs(lses[l] - ref_lse)))
            say(f"layer {l}: normwise {err:.3e} lse {lerr:.3e}")
            assert err <= TOL, (l, err)
            assert lerr <= TOL, (l, lerr)
    finally:
        c.close()


def _staged_index():
    """Token and channel of each staged K and V operand element, in the
    order the tile stores them (the layout documented in kvs.h)."""
    T, b, lane, e = np.meshgrid(np.arange(16), np.arange(4), np.arange(64), np.arange(8), indexing="ij")
    k_tok, k_dim = 16 * T + lane % 16, 32 * b + 8 * (lane // 16) + e
    c, ct, lane, s = np.meshgrid(np.arange(8), np.arange(8), np.arange(64), np.arange(8), indexing="ij")
    j = lane // 16
    v_tok = 32 * c + np.where(s < 4, 4 * j + s, 12 + 4 * j + s)
    v_ch = 16 * ct + lane % 16
    return k_tok.ravel(), k_dim.ravel(), v_tok.ravel(), v_ch.ravel()


_IDX = _staged_index()


def decode_staged_tile(tile):
    """Staged tile bytes of one (page, kv head) -> (K codes as float [256, 128],
    K scales float32 [256, 4], V operands as float16 [256, 128], V shifts
    int32 [4 sub-blocks, 4 blocks]) in token-major order."""
    t = np.frombuffer(tile.tobytes(), dtype=np.uint8)
    k_tok, k_dim, v_tok, v_ch = _IDX
    kcodes = np.full((256, 128), np.nan, np.float32)
    kcodes[k_tok, k_dim] = t[:65536].view(np.float16).astype(np.float32)
    vv = np.full((256, 128), np.nan, np.float16)
    vv[v_tok, v_ch] = t[65536:131072].view(np.float16)
    kscale = t[131072:135168].view(np.float32).reshape(256, 4)
    shifts = t[135168:135232].view(np.int32).reshape(4, 4).copy()
    return kcodes, kscale, vv, shifts


STAGED = [("q4_0", "edges", "big"), ("q4_0", "tiny", "tiny"), ("q4_0", "mixed", "mixed"),
          ("q8_0", "edges", "mid"), ("q8_0", "big", "big"), ("q8_0", "tiny", "mixed")]


@pytest.mark.parametrize("type_v,k_regime,v_regime", STAGED, ids=[f"{t}-K{k}-V{v}" for t, k, v in STAGED])
@pytest.mark.parametrize("zero_copy", [False, True], ids=["ring", "zero-copy"])
def test_staged_operands_bit_exact(type_v, k_regime, v_regime, zero_copy):
    """kvs_debug_stage converts every page with the staging code of the
    prefill path; streamed pages pass through the ring (or are read in place).
    K operands are the codes exactly, the scales their exact float32 values;
    each V operand is the round-to-nearest-even binary16 of d * (u - 8) /
    2^shift (Q4_0) or d * code / 2^shift (Q8_0) computed exactly from the
    oracle's float64 dequantization; the shift of a 64-token sub-block and
    block is 3 exactly when a cached row of it has a Q4_0 V scale magnitude
    above 8188, 7 exactly when a Q8_0 one exceeds 511.75."""
    recs = regime_records(k_regime, v_regime, n_layers=1, seed=5, type_v=type_v)
    say(f"staged operands {type_v} K={k_regime} V={v_regime} zero_copy={zero_copy}")
    c = EdgeCase(recs, max_q=1, resident_fn=mask_random(0.5, seed=8),
                 flags=kvs.FLAG_ZERO_COPY if zero_copy else 0, type_v=type_v)
    try:
        n_pages = c.n_pages
        dst = torch.empty(n_pages * HKV * kvs.STAGED_TILE_BYTES, dtype=torch.uint8, device="cuda")
        c.pool.debug_stage(0, N_KV, dst)
        torch.cuda.synchronize()
        tiles = dst.cpu().numpy().reshape(n_pages, HKV, kvs.STAGED_TILE_BYTES)
        K, V = gather_kv(recs[0], HKV, 128, 0, n_pages * 256, type_v=type_v)
        vblk = 34 if type_v == "q8_0" else 18
        big_bits, big_shift = (0x5FFF, 7) if type_v == "q8_0" else (0x6FFF, 3)
        rec = recs[0]
        for p in range(n_pages):
            valid = min(256, N_KV - 256 * p)
            for g in range(HKV):
                kcodes, kscale, vv, shifts = decode_staged_tile(tiles[p, g])
                kb = rec[p, g * 256 * 136:(g + 1) * 256 * 136].reshape(256, 4, 34)
                codes = kb[:, :, 2:].view(np.int8).reshape(256, 128).astype(np.float32)
                sbits = kb[:, :, 0].astype(np.uint16) | (kb[:, :, 1].astype(np.uint16) << 8)
                sval = f16_to_f64(sbits).astype(np.float32)   # exact
                assert np.array_equal(kcodes[:valid], codes[:valid]), (p, g)
                assert np.array_equal(kscale[:valid].view(np.uint32), sval[:valid].view(np.uint32)), (p, g)
                vo = HKV * 256 * 136 + g * 256 * 4 * vblk
                vb = rec[p, vo:vo + 256 * 4 * vblk].reshape(256, 4, vblk)
                vbits = (vb[:, :, 0].astype(np.uint16) | (vb[:, :, 1].astype(np.uint16) << 8)) & 0x7FFF
                cached = np.arange(256) < valid
                want_shift = np.zeros((4, 4), np.int64)
                for sb in range(4):
                    rows = vbits[64 * sb:64 * sb + 64][cached[64 * sb:64 * sb + 64]]
                    if len(rows):
                        want_shift[sb] = np.where(rows.max(axis=0) > big_bits, big_shift, 0)
                assert np.array_equal(shifts, want_shift), (p, g, shifts, want_shift)
                div = np.repeat(np.repeat(2.0 ** want_shift, 64, axis=0), 32, axis=1)   # [token, channel]
                exact = V[256 * p:256 * p + 256, g, :] / div
                want = exact[:valid].astype(np.float16)
                assert np.array_equal(vv[:valid].view(np.uint16) & 0x7FFF, want.view(np.uint16) & 0x7FFF) and \
                    np.array_equal(np.signbit(vv[:valid]) | (want == 0), np.signbit(want) | (want == 0)), (p, g)
                assert np.all(vv[valid:] == 0), (p, g)   # uncached rows are zeroed
    finally:
        c.close()
