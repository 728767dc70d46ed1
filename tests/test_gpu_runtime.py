"""The host runtime on the GPU, through the C ABI: raw page records as the
kernels see them (ring included), ordering of calls issued on different
streams, a layer that grows page by page with newest-page residency, and a
draft layer in a pinned region of the pool.

Bars: exported records equal the host records byte for byte; attention is
within 2e-3 of the oracle (normwise per row, lse absolute) and bit-identical
to the same work issued on one stream or with every page resident; appended
rows are bit-exact with the oracle's quantizer.
"""

import numpy as np
import pytest
import torch

import host_streamed_paged_amd as kvs
from kvs_case import Case, mask_all, mask_none, mask_random, normwise_error, say
from kvs_synth import KVGeometry, layer_records
from oracle import append_rows, attend_layer

pytestmark = pytest.mark.gpu

TOL = 2e-3
N_KV = 5 * 256 + 77


def small(resident_fn, *, ring=4, chunk=2, group=1, flags=0, n_layers=2, Hkv=2, Hq=12, max_q=4, cid=61):
    say(f"runtime case ring={ring} chunk={chunk} group={group} flags={flags} "
        f"residency={getattr(resident_fn, '__name__', 'fn')}")
    return Case(cid=cid, n_layers=n_layers, n_kv_heads=Hkv, n_q_heads=Hq, n_kv=N_KV,
                cfg_kw=dict(max_q_tokens=max_q, ring_pages=ring, chunk_pages=chunk, group_pages=group, flags=flags),
                resident_fn=resident_fn)


@pytest.mark.parametrize("v", [dict(resident=mask_none, ring=1, chunk=1),
                               dict(resident=mask_random(0.5, seed=3), ring=4, chunk=2),
                               dict(resident=mask_none, ring=8, chunk=2, group=1),
                               dict(resident=mask_random(0.3, seed=4), ring=6, chunk=3, group=2),
                               dict(resident=mask_none, ring=4, chunk=1, group=3),
                               dict(resident=mask_random(0.5, seed=5), ring=4, chunk=2, flags=kvs.FLAG_ZERO_COPY),
                               dict(resident=mask_all, ring=4, chunk=2)],
                         ids=["ring1", "half-ring4", "none-lanes", "ring6-chunk3", "split-groups", "zero-copy", "all"])
def test_exported_records_equal_host_records(v):
    """Every page as the attention kernels read it, streamed pages taken from
    the ring chunk they were copied into during the pass (several compute
    lanes, split groups, a one-page ring), equals its pinned host record."""
    c = small(v["resident"], ring=v["ring"], chunk=v["chunk"], group=v.get("group", 1), flags=v.get("flags", 0))
    try:
        pb = kvs.page_bytes(c.cfg)
        for l in range(c.L):
            dst = torch.full((c.n_pages, pb), 0x5A, dtype=torch.uint8, device="cuda")
            c.pool.stream_enqueue(l)
            c.pool.debug_export_pages(l, dst)
            torch.cuda.synchronize()
            got = dst.cpu().numpy()
            for p in range(c.n_pages):
                assert np.array_equal(got[p], c.records[l][p]), (l, p, bool(c.masks[l][p]))
        st = c.pool.status()
        n_streamed = sum(int((1 - m).sum()) for m in c.masks)
        if not v.get("flags"):
            assert st.pages_streamed >= n_streamed
    finally:
        c.close()


def test_calls_on_different_streams_are_ordered():
    """Layers attended alternately on two streams with no host wait between
    them (each call reuses the pool's split-K workspace and ring), a gather
    and an export on a third: outputs equal the single-stream run bit for bit
    and match the oracle."""
    c = small(mask_random(0.5, seed=9), n_layers=4, ring=4, chunk=1, max_q=4)
    try:
        qs = [c.queries(l, 4, "f32") for l in range(c.L)]
        base, base_lse = c.attend_all(qs, q_pos0=N_KV - 4, scale=1.0, causal=True)
        for l in range(c.L):
            ref, ref_lse = c.oracle(l, qs[l], q_pos0=N_KV - 4, scale=1.0, causal=True)
            assert normwise_error(base[l], ref) <= TOL
        s = [torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()]
        dq = [torch.from_numpy(q).cuda() for q in qs]
        torch.cuda.synchronize()
        for rep in range(3):
            outs = [torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda") for q in dq]
            lses = [torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda") for q in dq]
            k = torch.empty((N_KV, c.Hkv, 128), dtype=torch.float32, device="cuda")
            v = torch.empty_like(k)
            pb = kvs.page_bytes(c.cfg)
            ex = torch.empty((c.n_pages, pb), dtype=torch.uint8, device="cuda")
            torch.cuda.synchronize()
            for l in range(c.L):
                c.pool.attend(l, dq[l], N_KV, N_KV - 4, 1.0, True, outs[l], lses[l], stream=s[l % 2])
                if l == 1:
                    c.pool.debug_gather(2, 0, N_KV, k, v, stream=s[2])
                    c.pool.debug_export_pages(3, ex, stream=s[2])
            torch.cuda.synchronize()
            for l in range(c.L):
                assert np.array_equal(outs[l].cpu().numpy(), base[l]), (rep, l)
                assert np.array_equal(lses[l].cpu().numpy(), base_lse[l]), (rep, l)
            assert np.array_equal(ex.cpu().numpy(), c.records[3]), rep
    finally:
        c.close()


def test_growing_layer_newest_page_window():
    """A decode layer grows by appended rows (kvs_append, f32, 100 at a
    time); at each new page the table is set again with the newest-page
    window (kvs_residency_promote_newest, 2 resident pages) so the oldest
    resident page is streamed. Only newly resident pages are uploaded; host
    records equal the oracle's appended records byte for byte; attention after
    each step matches the oracle and an all-resident pool bit for bit."""
    H, HQ, W = 2, 12, 2
    geom = KVGeometry(H, 128)
    max_pages = 8
    n0 = 2 * 256 + 40
    recs = layer_records(77, 0, max_pages * 256, geom)       # capacity; rows past n0 are rewritten
    rows_total = 5 * 256
    g = np.random.default_rng(5)
    new_k = (g.standard_normal((rows_total, H, 128)) * 1.3).astype(np.float32)
    new_v = g.standard_normal((rows_total, H, 128)).astype(np.float32)
    host_w = torch.from_numpy(recs.copy()).pin_memory()       # windowed pool's records
    host_a = torch.from_numpy(recs.copy()).pin_memory()       # all-resident pool's records
    cfg = kvs.Config(n_layers=1, n_kv_heads=H, n_q_heads=HQ, max_pages=max_pages, max_q_tokens=1, ring_pages=2,
                     chunk_pages=1, group_pages=1)
    pw = kvs.Pool(cfg, kvs.Pool.arena_for(cfg, W))
    pa = kvs.Pool(cfg, kvs.Pool.arena_for(cfg, max_pages))
    oracle_recs = recs.copy()
    try:
        pw.host_pages_set(0, host_w)
        pa.host_pages_set(0, host_a)
        n_kv = n0
        n_pages = -(-n_kv // 256)
        mask = kvs.residency_promote_newest(np.zeros(0, np.uint8), n_pages, W)
        pw.page_table_set(0, mask)
        pa.page_table_set(0, np.ones(n_pages, np.uint8))
        pb = kvs.page_bytes(cfg)
        assert pw.status().resident_upload_bytes == W * pb
        done = 0
        step = 0
        while done < rows_total:
            n = min(100, rows_total - done)
            new_pages = -(-(n_kv + n) // 256)
            if new_pages > n_pages:
                up0 = pw.status().resident_upload_bytes
                mask = kvs.residency_promote_newest(mask, new_pages, W)
                pw.page_table_set(0, mask)
                pa.page_table_set(0, np.ones(new_pages, np.uint8))
                # one new page became resident: one page uploaded
                assert pw.status().resident_upload_bytes - up0 == (new_pages - n_pages) * pb
                assert int(mask.sum()) == W and mask[-1] == 1
                n_pages = new_pages
            kd = torch.from_numpy(new_k[done:done + n]).cuda()
            vd = torch.from_numpy(new_v[done:done + n]).cuda()
            pw.append(0, kd, vd, n_kv)
            pa.append(0, kd, vd, n_kv)
            oracle_recs = append_rows(oracle_recs, new_k[done:done + n], new_v[done:done + n], pos0=n_kv,
                                      n_kv_heads=H, head_dim=128)
            n_kv += n
            done += n
            q = g.standard_normal((1, HQ, 128)).astype(np.float32) / np.float32(np.sqrt(128))
            qd = torch.from_numpy(q).cuda()
            ow = torch.empty((1, HQ, 128), dtype=torch.float32, device="cuda")
            oa = torch.empty_like(ow)
            lw = torch.empty((1, HQ), dtype=torch.float32, device="cuda")
            la = torch.empty_like(lw)
            pw.attend(0, qd, n_kv, n_kv - 1, 1.0, False, ow, lw)
            pa.attend(0, qd, n_kv, n_kv - 1, 1.0, False, oa, la)
            torch.cuda.synchronize()
            say(f"step {step}: n_kv {n_kv}, pages {n_pages}, resident {np.flatnonzero(mask).tolist()}")
            assert np.array_equal(ow.cpu().numpy(), oa.cpu().numpy()), step
            assert np.array_equal(lw.cpu().numpy(), la.cpu().numpy()), step
            # the authoritative records hold the oracle's bytes, in both pools
            assert np.array_equal(host_w.numpy(), oracle_recs), step
            assert np.array_equal(host_a.numpy(), oracle_recs), step
            ref, ref_lse = attend_layer(oracle_recs, q, n_kv=n_kv, n_kv_heads=H, head_dim=128, scale=1.0,
                                        causal=False, q_pos0=n_kv - 1)
            err = normwise_error(ow.cpu().numpy(), ref)
            assert err <= TOL, (step, err)
            assert float(np.max(np.abs(lw.cpu().numpy() - ref_lse))) <= TOL
            step += 1
    finally:
        pw.close()
        pa.close()


def test_pinned_draft_layer_shares_the_pool():
    """Two target layers and a draft layer (one more logical layer of the same
    pool). The draft layer's window of 3 pages lives in a pinned region
    carved from the top of the slot range: other layers cannot take those
    slots, the draft cannot take others; attention on every layer matches the
    oracle; resetting the region returns its slots once the draft holds none."""
    c = Case(cid=83, n_layers=3, n_kv_heads=2, n_q_heads=12, n_kv=N_KV,
             cfg_kw=dict(max_q_tokens=1, ring_pages=4, chunk_pages=2, group_pages=1),
             resident_fn=lambda l, n: np.zeros(n, np.uint8), slots=10)
    try:
        pool = c.pool
        n = c.n_pages
        st = pool.status()
        assert st.slot_count == 10 and st.slots_used == 0
        pool.pin_layer(2, 3)
        assert pool.status().pinned_slots == 3
        # the two target layers may hold 7 general slots between them
        pool.page_table_set(0, np.array([1, 1, 1, 1, 0, 0], np.uint8)[:n])
        with pytest.raises(kvs.KvsError) as e:
            pool.page_table_set(1, np.array([1, 1, 1, 1, 0, 0], np.uint8)[:n])
        assert e.value.code == kvs.ERR_NO_SLOTS
        pool.page_table_set(1, np.array([0, 0, 1, 0, 1, 1], np.uint8)[:n])
        # the draft window: newest pages, at most 3 resident, in its region
        window = kvs.residency_promote_newest(np.zeros(0, np.uint8), n, 3)
        assert window.tolist() == [0, 0, 0, 1, 1, 1][:n]
        pool.page_table_set(2, window)
        with pytest.raises(kvs.KvsError) as e:
            pool.page_table_set(2, np.ones(n, np.uint8))
        assert e.value.code == kvs.ERR_NO_SLOTS
        assert pool.status().slots_used == 10
        qs = [c.queries(l, 1, "f32") for l in range(3)]
        outs, lses = c.attend_all(qs, q_pos0=N_KV - 1, scale=1.0, causal=False)
        for l in range(3):
            ref, ref_lse = c.oracle(l, qs[l], q_pos0=N_KV - 1, scale=1.0, causal=False)
            assert normwise_error(outs[l], ref) <= TOL, l
            assert float(np.max(np.abs(lses[l] - ref_lse))) <= TOL, l
        # a second region cannot take slots held by resident pages; reset
        # needs the draft to hold none
        with pytest.raises(kvs.KvsError) as e:
            pool.pin_layer(0, 1)
        assert e.value.code == kvs.ERR_STATE
        with pytest.raises(kvs.KvsError) as e:
            pool.reset_pinned()
        assert e.value.code == kvs.ERR_STATE
        pool.page_table_set(2, np.zeros(n, np.uint8))
        pool.reset_pinned()
        assert pool.status().pinned_slots == 0
        # the region's slots are general again: layer 1 can now hold 6 pages
        pool.page_table_set(1, np.ones(n, np.uint8))
        outs2, _ = c.attend_all(qs, q_pos0=N_KV - 1, scale=1.0, causal=False)
        assert np.array_equal(outs2[1], outs[1]) and np.array_equal(outs2[0], outs[0])
    finally:
        c.close()
