"""KV append on the GPU (kvs_append, through the C ABI) against the oracle.

Both V block types (Q4_0 and Q8_0) are covered. Bars: the appended bytes are
bit-exact with the oracle's quantizer, in the
authoritative host records and in every resident device slot, and no other
byte changes; attention over the appended cache is within 2e-3 (normwise per
row, lse absolute) of the oracle on the updated records, and bit-identical
whether the page that received the rows is resident or streamed.
"""

import numpy as np
import pytest
import torch

import host_streamed_paged_amd as kvs
from kvs_case import Case, mask_all, mask_none, mask_random, normwise_error, say
from oracle import append_rows, attend_layer

pytestmark = pytest.mark.gpu

TOL = 2e-3
H, HQ = 4, 24
N_KV = 5 * 256 + 77          # 6 pages, the last one ragged


def new_rows(seed, n, dtype):
    g = np.random.default_rng(seed)
    k = (g.standard_normal((n, H, 128)) * 1.7).astype(np.float32)
    v = g.standard_normal((n, H, 128)).astype(np.float32)
    # a few blocks with a zero row, an exact tie and a large spread
    k[0, 0, :32] = 0.0
    v[0, 1, 32:64] = 0.0
    v[-1, 2, 5], v[-1, 2, 9] = 3.0, -3.0
    k[-1, 3, 64:96] *= np.float32(1e-3)
    if dtype == "f16":
        return k.astype(np.float16), v.astype(np.float16)
    return k, v


def make_case(resident_fn, cid=57, type_v="q4_0"):
    say(f"append case cid={cid} n_kv={N_KV} {type_v} residency={getattr(resident_fn, '__name__', 'fn')}")
    return Case(cid=cid, n_layers=2, n_kv_heads=H, n_q_heads=HQ, n_kv=N_KV,
                cfg_kw=dict(max_q_tokens=4, ring_pages=4, chunk_pages=2, group_pages=1),
                resident_fn=resident_fn, type_v=type_v)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("type_v", ["q4_0", "q8_0"])
@pytest.mark.parametrize("resident", [mask_all, mask_none, mask_random(0.5, seed=3)], ids=["all", "none", "half"])
def test_append_writes_quantized_rows_bit_exact(resident, type_v):
    c = make_case(resident, type_v=type_v)
    try:
        # (layer, input dtype, pos0, rows): the tail of the last page; rows
        # across a page boundary, over existing ones; a single decode row; a
        # whole page (8192 blocks)
        for l, dt, pos0, n in [(0, "f32", N_KV - 40, 40), (1, "f16", 2 * 256 - 10, 30), (0, "f32", 3 * 256 + 5, 1),
                               (1, "f32", 3 * 256, 256)]:
            say(f"append layer {l} {dt} tokens [{pos0}, {pos0 + n})")
            k, v = new_rows(10 + pos0, n, dt)
            before = c.host[l].numpy().copy()
            c.pool.append(l, dev(k), dev(v), pos0)
            torch.cuda.synchronize()
            expect = append_rows(before, k, v, pos0=pos0, n_kv_heads=H, head_dim=128, type_v=type_v)
            got = c.host[l].numpy()
            assert np.array_equal(got, expect), (l, pos0)
            for p in range(c.n_pages):
                if c.masks[l][p]:
                    assert np.array_equal(c.pool.debug_read_page(l, p), expect[p]), (l, p)
    finally:
        c.close()


@pytest.mark.parametrize("type_v", ["q4_0", "q8_0"])
def test_attention_after_append_matches_oracle_and_ignores_residency(type_v):
    """Decode: one new row at the last position, then attention over it.
    Verify: four new rows (the draft), then a causal 4-token block. The page
    that takes the rows is resident in one pool and streamed in the other."""
    base = None
    for tail_resident in (True, False):
        def mask(l, n):
            m = np.array(mask_random(0.5, seed=4)(l, n), np.uint8)
            m[n - 1] = 1 if tail_resident else 0
            return m
        c = make_case(mask, cid=58, type_v=type_v)
        try:
            records = [r.copy() for r in c.records]
            outs = []
            for l in range(c.L):
                n_new, dt = (1, "f32") if l == 0 else (4, "f16")
                pos0 = N_KV - n_new
                k, v = new_rows(20 + l, n_new, dt)
                c.pool.append(l, dev(k), dev(v), pos0)
                records[l] = append_rows(records[l], k, v, pos0=pos0, n_kv_heads=H, head_dim=128, type_v=type_v)
                q = c.queries(l, n_new, "f32")
                out = torch.empty((n_new, HQ, 128), dtype=torch.float32, device="cuda")
                lse = torch.empty((n_new, HQ), dtype=torch.float32, device="cuda")
                c.pool.attend(l, dev(q), N_KV, pos0, 1.0, True, out, lse)
                torch.cuda.synchronize()
                o, s = out.cpu().numpy(), lse.cpu().numpy()
                ref, ref_lse = attend_layer(records[l], q, n_kv=N_KV, n_kv_heads=H, head_dim=128, scale=1.0,
                                            causal=True, q_pos0=pos0, type_v=type_v)
                err = normwise_error(o, ref)
                lerr = float(np.max(np.abs(s - ref_lse)))
                say(f"tail resident={tail_resident} layer {l}: normwise {err:.3e} lse {lerr:.3e}")
                assert err <= TOL and lerr <= TOL
                assert np.array_equal(c.host[l].numpy(), records[l])
                outs.append((o, s))
            if base is None:
                base = outs
            else:
                for (o, s), (bo, bs) in zip(outs, base):
                    assert np.array_equal(o, bo) and np.array_equal(s, bs)
        finally:
            c.close()


def test_append_errors_leave_the_records_unchanged():
    c = make_case(mask_random(0.5, seed=5), cid=59)
    try:
        k, v = new_rows(1, 4, "f32")
        kd, vd = dev(k), dev(v)
        before = [h.numpy().copy() for h in c.host]
        for pos0 in (c.n_pages * 256 - 3, -1):                      # past the layer's pages; negative
            with pytest.raises(kvs.KvsError) as e:
                c.pool.append(0, kd, vd, pos0)
            assert e.value.code == kvs.ERR_INVALID_ARG
        buf = torch.zeros(4 * H * 128 + 1, device="cuda")
        with pytest.raises(kvs.KvsError) as e:                      # 4-byte aligned only
            c.pool.append(0, buf[1:].view(4, H, 128), vd, 0)
        assert e.value.code == kvs.ERR_INVALID_ARG
        # a pending prefetch may be reading a streamed page's record
        streamed = [p for p in range(c.n_pages) if not c.masks[0][p]]
        resident = [p for p in range(c.n_pages) if c.masks[0][p]]
        c.pool.stream_enqueue(0)
        with pytest.raises(kvs.KvsError) as e:
            c.pool.append(0, kd, vd, streamed[0] * 256)
        assert e.value.code == kvs.ERR_STATE
        torch.cuda.synchronize()
        for h, b in zip(c.host, before):
            assert np.array_equal(h.numpy(), b)
        # a resident page may still take rows while the prefetch is pending
        c.pool.append(0, kd, vd, resident[0] * 256)
        q = dev(c.queries(0, 1, "f32"))
        out = torch.empty((1, HQ, 128), dtype=torch.float32, device="cuda")
        c.pool.attend(0, q, N_KV, N_KV - 1, 1.0, True, out)        # consumes the prefetch
        c.pool.append(0, kd[:0], vd[:0], 0)                          # no rows: a no-op
        torch.cuda.synchronize()
        expect = append_rows(before[0], k, v, pos0=resident[0] * 256, n_kv_heads=H, head_dim=128)
        assert np.array_equal(c.host[0].numpy(), expect)
        assert np.array_equal(c.host[1].numpy(), before[1])
    finally:
        c.close()


def test_append_on_another_stream_orders_before_a_multi_lane_attention():
    """Rows appended on a side stream into a streamed page, then attention on
    the default stream with no host synchronization in between: a 4-slot ring
    in 2-page chunks runs two compute lanes, whose ring copies must wait for
    the append. Checked against the oracle on the updated records, over
    several rounds."""
    def mask(l, n):
        m = np.zeros(n, np.uint8)
        m[0] = 1
        return m
    c = Case(cid=60, n_layers=1, n_kv_heads=H, n_q_heads=HQ, n_kv=N_KV,
             cfg_kw=dict(max_q_tokens=4, ring_pages=8, chunk_pages=2, group_pages=1),
             resident_fn=mask)
    try:
        info, _, _ = kvs.plan_layer(c.cfg, c.masks[0])
        assert info.n_chunks >= 2 and info.whole_groups == 1
        side = torch.cuda.Stream()
        records = c.records[0].copy()
        q = dev(c.queries(0, 1, "f32"))
        for rnd in range(3):
            pos0 = N_KV - 1 - 300 * rnd                   # pages 5, 4, 3: all streamed
            k, v = new_rows(30 + rnd, 1, "f32")
            # the new key is aligned with the query of its group's first head,
            # so that the new row dominates those rows' attention: a missed
            # append would move the output far past the bar
            qn = c.queries(0, 1, "f32")
            for g in range(H):
                k[0, g] = 10.0 * qn[0, g * (HQ // H)]
            kd, vd = dev(k), dev(v)
            torch.cuda.synchronize()
            with torch.cuda.stream(side):
                c.pool.append(0, kd, vd, pos0, stream=side)
            records = append_rows(records, k, v, pos0=pos0, n_kv_heads=H, head_dim=128)
            out = torch.empty((1, HQ, 128), dtype=torch.float32, device="cuda")
            c.pool.attend(0, q, N_KV, N_KV - 1, 1.0, True, out)
            torch.cuda.synchronize()
            ref, _ = attend_layer(records, c.queries(0, 1, "f32"), n_kv=N_KV, n_kv_heads=H, head_dim=128,
                                  scale=1.0, causal=True, q_pos0=N_KV - 1)
            err = normwise_error(out.cpu().numpy(), ref)
            say(f"side-stream append round {rnd}: normwise {err:.3e}")
            assert err <= TOL
    finally:
        c.close()
