"""Zero-copy A/B (KVS_FLAG_ZERO_COPY): streamed pages read in place from their
pinned host records by the attention kernels, with no ring.

Bars: the same kernels fold the same pages in the same order, so outputs are
bit-identical to the ring path (decode, verify, and a prefill-width block of
more than 64 rows per kv head, with whole groups and with groups split across
chunks); gathers are
bit-exact with the oracle; a streamed zero-copy layer can be captured in a HIP
graph and replayed.
"""

import numpy as np
import pytest
import torch

import host_streamed_paged_amd as kvs
from kvs_case import Case, mask_none, mask_random, normwise_error, say
from oracle import gather_kv

pytestmark = pytest.mark.gpu

TOL = 2e-3
N_KV = 5 * 256 + 77


def case(resident_fn, flags, *, n_q=4, ring=4, chunk=2, group=1, cid=71, n_layers=2):
    say(f"zero-copy case flags={flags} n_q={n_q} ring={ring} chunk={chunk} group={group}")
    return Case(cid=cid, n_layers=n_layers, n_kv_heads=2, n_q_heads=12, n_kv=N_KV,
                cfg_kw=dict(max_q_tokens=n_q, ring_pages=ring, chunk_pages=chunk,
                            group_pages=group, flags=flags),
                resident_fn=resident_fn)


@pytest.mark.parametrize("n_q,qdt,scale,group,chunk", [
    (1, "f32", 1.0, 1, 2),        # decode
    (4, "f32", 1.0, 2, 2),        # verify (matrix cores, 24 rows)
    (11, "f16", 0.12, 3, 1),      # 66 rows: prefill kernel; groups of 3 split across 1-page chunks
])
def test_zero_copy_equals_the_ring_bit_for_bit(n_q, qdt, scale, group, chunk):
    resident = mask_random(0.4, seed=8)
    res = []
    for flags in (0, kvs.FLAG_ZERO_COPY):
        c = case(resident, flags, n_q=n_q, ring=2 * chunk, chunk=chunk, group=group)
        try:
            qs = [c.queries(l, n_q, qdt) for l in range(c.L)]
            outs, lses = c.attend_all(qs, q_pos0=N_KV - n_q, scale=scale, causal=True)
            if flags:
                for l in range(c.L):
                    ref, ref_lse = c.oracle(l, qs[l], q_pos0=N_KV - n_q, scale=scale, causal=True)
                    err = normwise_error(outs[l], ref)
                    say(f"zero-copy layer {l}: normwise {err:.3e}")
                    assert err <= TOL
                    assert float(np.max(np.abs(lses[l] - ref_lse))) <= TOL
                st = c.pool.status()
                assert st.bytes_h2d == 0, "the ring moved bytes in zero-copy mode"
            res.append((outs, lses))
        finally:
            c.close()
    for l in range(len(res[0][0])):
        assert np.array_equal(res[0][0][l], res[1][0][l]), l
        assert np.array_equal(res[0][1][l], res[1][1][l]), l


def test_zero_copy_gather_bit_exact():
    c = case(mask_random(0.5, seed=9), kvs.FLAG_ZERO_COPY, n_layers=1)
    try:
        for tok0, n_tok in [(0, N_KV), (300, 500)]:
            k = torch.empty((n_tok, 2, 128), dtype=torch.float32, device="cuda")
            v = torch.empty_like(k)
            c.pool.debug_gather(0, tok0, n_tok, k, v)
            torch.cuda.synchronize()
            rk, rv = gather_kv(c.records[0], 2, 128, tok0, n_tok)
            assert np.array_equal(k.cpu().numpy(), rk.astype(np.float32))
            assert np.array_equal(v.cpu().numpy(), rv.astype(np.float32))
    finally:
        c.close()


def test_zero_copy_streamed_layer_replays_in_a_graph():
    """With nothing streamed through the ring, a layer of streamed pages can be
    captured; each replay (eager work and synchronizations in between) gives the
    eager result bit for bit."""
    c = case(mask_none, kvs.FLAG_ZERO_COPY, n_q=1, n_layers=2, cid=72)
    try:
        dq = [torch.from_numpy(c.queries(l, 1, "f32")).cuda() for l in range(c.L)]
        eager = [torch.empty_like(q) for q in dq]
        for l in range(c.L):
            c.pool.attend(l, dq[l], N_KV, N_KV - 1, 1.0, True, eager[l])
        torch.cuda.synchronize()
        outs = [torch.empty_like(q) for q in dq]
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for l in range(c.L):
                c.pool.attend(l, dq[l], N_KV, N_KV - 1, 1.0, True, outs[l], stream=s)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for l in range(c.L):
                c.pool.attend(l, dq[l], N_KV, N_KV - 1, 1.0, True, outs[l], stream=s)
        scratch = torch.empty_like(dq[0])
        for rep in range(3):
            for o in outs:
                o.fill_(float("nan"))
            c.pool.attend(rep % c.L, dq[0], N_KV, N_KV - 1, 1.0, True, scratch)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for l in range(c.L):
                assert torch.equal(outs[l], eager[l]), (rep, l)
        del g
    finally:
        c.close()


def test_zero_copy_long_prefill_layer_equals_the_ring():
    """A 70-page layer at prefill width (66 rows per kv head): the zero-copy
    launch gives the ring's bits."""
    n_kv, n_q = 70 * 256 - 31, 11                     # 70 pages, ragged tail; 66 rows
    res = []
    for flags in (0, kvs.FLAG_ZERO_COPY):
        say(f"long prefill layer flags={flags} n_kv={n_kv}")
        c = Case(cid=73, n_layers=1, n_kv_heads=2, n_q_heads=12, n_kv=n_kv,
                 cfg_kw=dict(max_q_tokens=n_q, ring_pages=8, chunk_pages=4, group_pages=1,
                             flags=flags),
                 resident_fn=mask_random(0.3, seed=10))
        try:
            qs = [c.queries(0, n_q, "f16")]
            outs, lses = c.attend_all(qs, q_pos0=n_kv - n_q, scale=0.12, causal=True)
            if flags:
                ref, ref_lse = c.oracle(0, qs[0], q_pos0=n_kv - n_q, scale=0.12, causal=True)
                err = normwise_error(outs[0], ref)
                say(f"zero-copy long prefill layer: normwise {err:.3e}")
                assert err <= TOL and float(np.max(np.abs(lses[0] - ref_lse))) <= TOL
            res.append((outs[0], lses[0]))
        finally:
            c.close()
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
