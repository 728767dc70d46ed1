"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Sizes span several page tiles, split-K groups and ring chunks, with a ragged
last page whose unused rows are NaN-poisoned. Bars: dequantization and page
gathers bit-exact; attention within 2e-3 normwise relative error per output
row (max_c |o - r| / max_c |r|, maximized over query token x head), lse within
2e-3 absolute; outputs bit-identical across residency, ring and chunk sizes.
"""

import math

import numpy as np
import pytest
import torch

import host_streamed_paged_amd as kvs
from kvs_case import Case, mask_all, mask_none, mask_random, normwise_error, say
from oracle import gather_kv

pytestmark = pytest.mark.gpu

TOL = 2e-3
N_KV = 5 * 256 + 77          # 6 pages, ragged tail of 77 rows


def small_case(resident_fn, *, cid=31, n_layers=3, n_kv=N_KV, Hkv=2, Hq=12, max_q=1, ring=4, chunk=2,
               group=1, flags=0, slots=None):
    say(f"case cid={cid} layers={n_layers} n_kv={n_kv} Hkv={Hkv} Hq={Hq} ring={ring} chunk={chunk} "
        f"group={group} flags={flags} residency={getattr(resident_fn, '__name__', 'fn')}")
    return Case(cid=cid, n_layers=n_layers, n_kv_heads=Hkv, n_q_heads=Hq, n_kv=n_kv, slots=slots,
                cfg_kw=dict(max_q_tokens=max_q, ring_pages=ring, chunk_pages=chunk,
                            group_pages=group, flags=flags),
                resident_fn=resident_fn)


@pytest.mark.parametrize("resident", [mask_all, mask_none, mask_random(0.5)], ids=["all", "none", "half"])
def test_gather_bit_exact(resident):
    c = small_case(resident)
    try:
        for l in range(c.L):
            for tok0, n_tok in [(0, c.n_pages * 256), (100, 700), (255, 2), (N_KV - 1, 1)]:
                say(f"kvs_debug_gather layer={l} tok0={tok0} n_tok={n_tok}")
                k = torch.empty((n_tok, c.Hkv, 128), dtype=torch.float32, device="cuda")
                v = torch.empty_like(k)
                c.pool.debug_gather(l, tok0, n_tok, k, v)
                torch.cuda.synchronize()
                rk, rv = gather_kv(c.records[l], c.Hkv, 128, tok0, n_tok)
                valid = max(0, min(n_tok, N_KV - tok0))
                assert np.array_equal(k.cpu().numpy()[:valid], rk[:valid].astype(np.float32))
                assert np.array_equal(v.cpu().numpy()[:valid], rv[:valid].astype(np.float32))
                if valid < n_tok:   # poisoned rows decode to NaN on both sides
                    assert np.all(np.isnan(k.cpu().numpy()[valid:]))
    finally:
        c.close()


def test_read_page_matches_host_records():
    c = small_case(mask_random(0.5))
    try:
        for l in range(c.L):
            for p in range(c.n_pages):
                if c.masks[l][p]:
                    assert np.array_equal(c.pool.debug_read_page(l, p), c.records[l][p])
                else:
                    with pytest.raises(kvs.KvsError) as e:
                        c.pool.debug_read_page(l, p)
                    assert e.value.code == kvs.ERR_NOT_RESIDENT
    finally:
        c.close()


def check(c, outs, lses, qs, *, q_pos0, scale, causal):
    worst = 0.0
    for l in range(c.L):
        ref, ref_lse = c.oracle(l, qs[l], q_pos0=q_pos0, scale=scale, causal=causal)
        err = normwise_error(outs[l], ref)
        lerr = float(np.max(np.abs(lses[l] - ref_lse)))
        say(f"layer {l}: normwise {err:.3e} lse {lerr:.3e}")
        assert err <= TOL, (l, err)
        assert lerr <= TOL, (l, lerr)
        worst = max(worst, err)
    return worst


@pytest.mark.parametrize("resident", [mask_all, mask_none, mask_random(0.5)], ids=["all", "none", "half"])
def test_decode_parity(resident):
    c = small_case(resident)
    try:
        qs = [c.queries(l, 1, "f32") for l in range(c.L)]
        outs, lses = c.attend_all(qs, q_pos0=N_KV - 1, scale=1.0, causal=False)
        check(c, outs, lses, qs, q_pos0=N_KV - 1, scale=1.0, causal=False)
    finally:
        c.close()


def test_verify_parity():
    c = small_case(mask_random(0.4, seed=2), max_q=4, group=2)
    try:
        qs = [c.queries(l, 4, "f32") for l in range(c.L)]
        outs, lses = c.attend_all(qs, q_pos0=N_KV - 4, scale=1.0, causal=True)
        check(c, outs, lses, qs, q_pos0=N_KV - 4, scale=1.0, causal=True)
    finally:
        c.close()


def test_prefill_parity():
    n_q = 300
    c = small_case(mask_random(0.3, seed=3), n_layers=2, max_q=n_q, group=2, ring=4, chunk=2)
    try:
        qs = [c.queries(l, n_q, "f16") for l in range(c.L)]
        scale = 1.0 / math.sqrt(128)
        outs, lses = c.attend_all(qs, q_pos0=N_KV - n_q, scale=scale, causal=True)
        check(c, outs, lses, qs, q_pos0=N_KV - n_q, scale=scale, causal=True)
    finally:
        c.close()


# Score spread: f32 queries are N(0,1)/sqrt(128), f16 queries N(0,1); the
# scales keep the standard deviation of the scores near 1 to 2 (natural log
# units), the range of the workloads. The matrix-core path rounds q * scale and
# d * k to f16, so its score error grows with the spread (about 2^-12 |s|).
@pytest.mark.parametrize("n_q,causal,qdt,scale", [(2, True, "f32", 1.0), (3, False, "f16", 0.15),
                                                 (6, True, "f16", 1 / math.sqrt(128)), (8, False, "f32", 2.0),
                                                 (11, True, "f32", 1.0)],
                         ids=["rows12", "rows18-noncausal", "rows36", "rows48-noncausal", "rows66"])
def test_multi_row_parity(n_q, causal, qdt, scale):
    """Query blocks between decode and prefill widths (16- and 32-row tiles of
    the matrix-core kernel, ragged row tiles included; the full-size tests
    cover the 64-row tiles)."""
    c = small_case(mask_random(0.5, seed=7), n_layers=2, max_q=n_q, group=2)
    try:
        qs = [c.queries(l, n_q, qdt) for l in range(c.L)]
        q_pos0 = N_KV - n_q
        outs, lses = c.attend_all(qs, q_pos0=q_pos0, scale=scale, causal=causal)
        check(c, outs, lses, qs, q_pos0=q_pos0, scale=scale, causal=causal)
    finally:
        c.close()


def test_prefill_and_matrix_core_paths_agree():
    """A block wider than 64 rows per kv head runs the prefill kernel; a
    narrower one the matrix-core kernel. The first 10 query tokens of an
    11-token block (66 rows, prefill) and a 10-token block (60 rows) both match
    the oracle, and
    each other to the same tolerance (their softmax runs over sub-blocks of
    different sizes, so the bits may differ)."""
    c = small_case(mask_random(0.5, seed=11), n_layers=2, max_q=11, group=2)
    try:
        qs11 = [c.queries(l, 11, "f32") for l in range(c.L)]
        qs10 = [q[:10].copy() for q in qs11]
        q_pos0 = N_KV - 11
        o11, l11 = c.attend_all(qs11, q_pos0=q_pos0, scale=1.0, causal=True)
        o10, l10 = c.attend_all(qs10, q_pos0=q_pos0, scale=1.0, causal=True)
        check(c, o11, l11, qs11, q_pos0=q_pos0, scale=1.0, causal=True)
        check(c, o10, l10, qs10, q_pos0=q_pos0, scale=1.0, causal=True)
        for l in range(c.L):
            assert normwise_error(o11[l][:10], o10[l].astype(np.float64)) <= TOL, l
            assert float(np.max(np.abs(l11[l][:10] - l10[l]))) <= TOL, l
    finally:
        c.close()


@pytest.mark.parametrize("qdt", ["f16", "f32"])
def test_prefill_bit_identical_across_residency_and_ring(qdt):
    """Large query blocks (64-row tiles, last one ragged) give the same bits
    whichever pages are resident and however the ring chunks the rest, for
    f16 queries and for f32 queries (two f16 limbs: the prefill kernel's
    variant that waits for every memory operation before its barriers)."""
    n_q = 40
    base = None
    for v in [dict(resident=mask_all, ring=4, chunk=2, group=3),
              dict(resident=mask_none, ring=2, chunk=1, group=3, flags=kvs.FLAG_POISON_RING),
              dict(resident=mask_random(0.4, seed=9), ring=8, chunk=4, group=3),
              dict(resident=mask_none, ring=18, chunk=3, group=3, flags=kvs.FLAG_POISON_RING)]:
        c = small_case(v["resident"], n_layers=2, max_q=n_q, ring=v["ring"], chunk=v["chunk"],
                       group=v["group"], flags=v.get("flags", 0))
        try:
            qs = [c.queries(l, n_q, qdt) for l in range(c.L)]
            outs, lses = c.attend_all(qs, q_pos0=N_KV - n_q, scale=0.12 if qdt == "f16" else 0.12 * math.sqrt(128),
                                      causal=True)
            if base is None:
                check(c, outs, lses, qs, q_pos0=N_KV - n_q, scale=0.12 if qdt == "f16" else 0.12 * math.sqrt(128),
                      causal=True)
                base = (outs, lses)
            else:
                for l in range(c.L):
                    assert np.array_equal(outs[l], base[0][l]), (v, l)
                    assert np.array_equal(lses[l], base[1][l]), (v, l)
        finally:
            c.close()


def test_outputs_bit_identical_across_residency_ring_and_chunks():
    variants = [
        dict(resident=mask_all, ring=4, chunk=2),
        dict(resident=mask_none, ring=1, chunk=1),
        dict(resident=mask_none, ring=6, chunk=3),
        dict(resident=mask_random(0.5), ring=4, chunk=4),
        dict(resident=mask_random(0.3, seed=5), ring=2, chunk=1, flags=kvs.FLAG_POISON_RING),
        # four or more chunk slots: two or three compute lanes (a divisor of
        # the slot count, which is at least twice the lanes) when no group
        # spans two chunks
        dict(resident=mask_none, ring=4, chunk=1),
        dict(resident=mask_random(0.5, seed=6), ring=8, chunk=2, flags=kvs.FLAG_POISON_RING),
        dict(resident=mask_none, ring=6, chunk=1, flags=kvs.FLAG_POISON_RING),
        dict(resident=mask_random(0.3, seed=8), ring=12, chunk=2),
        dict(resident=mask_random(0.2, seed=12), ring=16, chunk=2),
    ]
    for group in (1, 3):
        base = None
        for v in variants:
            c = small_case(v["resident"], max_q=4, ring=v["ring"], chunk=v["chunk"],
                           group=group, flags=v.get("flags", 0))
            try:
                qs = [c.queries(l, 4, "f32") for l in range(c.L)]
                outs, lses = c.attend_all(qs, q_pos0=N_KV - 4, scale=1.0, causal=True)
                if base is None:
                    check(c, outs, lses, qs, q_pos0=N_KV - 4, scale=1.0, causal=True)
                    base = (outs, lses)
                else:
                    for l in range(c.L):
                        assert np.array_equal(outs[l], base[0][l]), (v, group, l)
                        assert np.array_equal(lses[l], base[1][l]), (v, group, l)
            finally:
                c.close()


def test_verify_over_many_segments_slices_them_across_workers():
    """A verify block over many single-page groups: the matrix-core launch
    (8 kv heads x one 32-row tile, 160 segments; more than twice the 512
    workers that 256 compute units hold) gives each worker a slice of the
    segments, some two and some three. All resident, checked against the
    oracle; all streamed through the ring, whose chunk launches take one
    worker per segment, the same bits."""
    n_q, n_kv = 4, 160 * 256 - 45
    base = None
    for v in [dict(resident=mask_all, ring=8, chunk=2),
              dict(resident=mask_none, ring=8, chunk=2, flags=kvs.FLAG_POISON_RING)]:
        c = small_case(v["resident"], cid=41, n_layers=2, n_kv=n_kv, Hkv=8, Hq=48, max_q=n_q, ring=v["ring"],
                       chunk=v["chunk"], group=1, flags=v.get("flags", 0))
        try:
            qs = [c.queries(l, n_q, "f32") for l in range(c.L)]
            outs, lses = c.attend_all(qs, q_pos0=n_kv - n_q, scale=1.0, causal=True)
            if base is None:
                check(c, outs, lses, qs, q_pos0=n_kv - n_q, scale=1.0, causal=True)
                base = (outs, lses)
            else:
                for l in range(c.L):
                    assert np.array_equal(outs[l], base[0][l]), (v, l)
                    assert np.array_equal(lses[l], base[1][l]), (v, l)
        finally:
            c.close()


@pytest.mark.parametrize("n_q", [1, 4], ids=["decode", "verify"])
def test_empty_cache_returns_zero_and_minus_inf(n_q):
    c = small_case(mask_all, n_layers=1, max_q=n_q)
    try:
        pool = c.pool
        pool.page_table_set(0, np.zeros(0, np.uint8))
        q = torch.randn(n_q, c.Hq, 128, device="cuda")
        out = torch.full_like(q, 7.0)
        lse = torch.zeros(n_q, c.Hq, device="cuda")
        pool.attend(0, q, 0, 0, 1.0, False, out, lse)
        torch.cuda.synchronize()
        assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    finally:
        c.close()


def test_errors_leave_state_usable():
    c = small_case(mask_random(0.5), max_q=2)
    try:
        q = torch.from_numpy(c.queries(0, 3, "f32")).cuda()
        out = torch.empty_like(q)
        with pytest.raises(kvs.KvsError) as e:
            c.pool.attend(0, q, N_KV, N_KV - 3, 1.0, True, out)
        assert e.value.code == kvs.ERR_BATCH_TOO_WIDE
        with pytest.raises(kvs.KvsError) as e:
            c.pool.attend(0, q[:1], N_KV - 300, 0, 1.0, False, out[:1])
        assert e.value.code == kvs.ERR_INVALID_ARG
        # prefetch layer 1, then try layer 0: the ring is lent to layer 1
        c.pool.stream_enqueue(1)
        with pytest.raises(kvs.KvsError) as e:
            c.pool.attend(0, q[:1], N_KV, 0, 1.0, False, out[:1])
        assert e.value.code == kvs.ERR_STATE
        c.pool.attend(1, q[:1], N_KV, 0, 1.0, False, out[:1])
        # too many resident pages for the slots
        assert c.pool.status().slot_count == sum(int(m.sum()) for m in c.masks)
        with pytest.raises(kvs.KvsError) as e:
            c.pool.page_table_set(0, np.ones(c.n_pages, np.uint8))
        assert e.value.code == kvs.ERR_NO_SLOTS
        # after all the errors, a normal pass still matches the oracle
        qs = [c.queries(l, 1, "f32") for l in range(c.L)]
        outs, lses = c.attend_all(qs, q_pos0=N_KV - 1, scale=1.0, causal=False)
        check(c, outs, lses, qs, q_pos0=N_KV - 1, scale=1.0, causal=False)
        st = c.pool.status()
        assert st.pages_streamed > 0 and st.bytes_h2d == st.pages_streamed * kvs.page_bytes(c.cfg)
    finally:
        c.close()


def test_tiny_decode_workload():
    from kvs_synth import WORKLOADS
    wl = WORKLOADS["tiny_decode"]
    c = Case(cid=wl.cid, n_layers=1, n_kv_heads=1, n_q_heads=1, n_kv=wl.n_kv, resident_fn=mask_all,
             cfg_kw=dict(max_q_tokens=1, ring_pages=4, chunk_pages=2, group_pages=1))
    try:
        qs = [c.queries(0, 1, wl.q_dtype)]
        outs, lses = c.attend_all(qs, q_pos0=wl.q_pos0, scale=wl.scale, causal=wl.causal)
        check(c, outs, lses, qs, q_pos0=wl.q_pos0, scale=wl.scale, causal=wl.causal)
    finally:
        c.close()


def test_graph_replay_matches_eager():
    """A resident-only step captured in a HIP graph and replayed several
    times, with eager work and synchronizations between replays, gives the
    eager result bit for bit each time; streamed layers refuse capture."""
    c = small_case(mask_all, n_layers=3)
    try:
        dq = [torch.from_numpy(c.queries(l, 1, "f32")).cuda() for l in range(c.L)]
        eager = [torch.empty_like(q) for q in dq]
        for l in range(c.L):
            c.pool.attend(l, dq[l], N_KV, N_KV - 1, 1.0, False, eager[l])
        torch.cuda.synchronize()
        outs = [torch.empty_like(q) for q in dq]
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for l in range(c.L):
                c.pool.attend(l, dq[l], N_KV, N_KV - 1, 1.0, False, outs[l], stream=s)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for l in range(c.L):
                c.pool.attend(l, dq[l], N_KV, N_KV - 1, 1.0, False, outs[l], stream=s)
        scratch = torch.empty_like(dq[0])
        for rep in range(4):
            for o in outs:
                o.fill_(float("nan"))
            c.pool.attend(rep % c.L, dq[0], N_KV, N_KV - 1, 1.0, False, scratch)   # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for l in range(c.L):
                assert torch.equal(outs[l], eager[l]), (rep, l)
        del g
    finally:
        c.close()
    c = small_case(mask_none, n_layers=1)
    try:
        q = torch.from_numpy(c.queries(0, 1, "f32")).cuda()
        out = torch.empty_like(q)
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with pytest.raises(kvs.KvsError) as e:
            with torch.cuda.graph(g, stream=s):
                c.pool.attend(0, q, N_KV, N_KV - 1, 1.0, False, out, stream=s)
        assert e.value.code == kvs.ERR_UNSUPPORTED
    finally:
        c.close()


# (n_kv_heads, n_q_heads, query tokens, causal): every query-row count R of the
# decode kernel (R = query tokens x query heads per kv head, 1..6), with
# causal blocks of 2 tokens among them
DECODE_ROWS = [(2, 2, 1, False), (2, 4, 1, False), (2, 6, 1, False), (2, 4, 2, True), (1, 5, 1, False),
               (2, 6, 2, True)]


@pytest.mark.parametrize("Hkv,Hq,n_q,causal", DECODE_ROWS,
                         ids=["R1", "R2", "R3", "R4-causal", "R5", "R6-causal"])
@pytest.mark.parametrize("group", [1, 3], ids=["group1", "group3"])
def test_decode_rows_groups_and_residency(Hkv, Hq, n_q, causal, group):
    """The decode kernel for each row count, with one-page groups and with
    3-page groups (runs of several pages: the next page's loads are issued
    while the current one computes; groups split across ring chunks resume a
    stored group state). All pages resident (one launch), then half of them
    streamed through a ring on three compute lanes: both within 2e-3 of the
    oracle, and the same bits."""
    base = None
    for resident, ring, chunk in [(mask_all, 4, 2), (mask_random(0.5, seed=17), 12, 2)]:
        c = small_case(resident, n_layers=2, Hkv=Hkv, Hq=Hq, max_q=n_q, ring=ring, chunk=chunk,
                       group=group)
        try:
            qs = [c.queries(l, n_q, "f32") for l in range(c.L)]
            q_pos0 = N_KV - n_q
            outs, lses = c.attend_all(qs, q_pos0=q_pos0, scale=1.0, causal=causal)
            check(c, outs, lses, qs, q_pos0=q_pos0, scale=1.0, causal=causal)
            if base is None:
                base = (outs, lses)
            else:
                for l in range(c.L):
                    assert np.array_equal(outs[l], base[0][l]), l
                    assert np.array_equal(lses[l], base[1][l]), l
        finally:
            c.close()
