"""Kernel timing through the C ABI (kvs_profile_enable / kvs_profile_read).

The start/stop event pair of each timed launch rides on that kernel's own
dispatch. These tests check the counts per kind (attention 0, combine 1),
that every timed launch took a positive time no longer than the whole pass,
and that profiling changes no output bit.
"""

import numpy as np
import pytest
import torch

from kvs_case import mask_all, mask_random, say
from test_gpu_parity import small_case

pytestmark = pytest.mark.gpu


def _run(c, qs, **kw):
    return c.attend_all(qs, **kw)


def test_profile_counts_and_times_decode():
    c = small_case(mask_all, n_layers=2, Hkv=2, Hq=12)
    try:
        qs = [c.queries(l, 1, "f32") for l in range(c.L)]
        kw = dict(q_pos0=c.n_kv - 1, scale=1.0, causal=False, prefetch=False)
        ref, _ = _run(c, qs, **kw)
        for kind in (0, 1):
            c.pool.profile_read(kind, reset=True)
        c.pool.profile_enable(True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        out, _ = _run(c, qs, **kw)
        e1.record()
        torch.cuda.synchronize()
        c.pool.profile_enable(False)
        wall_ms = e0.elapsed_time(e1)
        n_att, ms_att = c.pool.profile_read(0)
        n_cmb, ms_cmb = c.pool.profile_read(1)
        say(f"decode profile: {n_att} attention launches {ms_att:.4f} ms, {n_cmb} combines {ms_cmb:.4f} ms, "
            f"pass {wall_ms:.4f} ms")
        assert n_att == c.L and n_cmb == c.L   # all resident: one attention launch per layer
        with pytest.raises(Exception):
            c.pool.profile_read(2)   # no third kind
        assert 0.0 < ms_att <= wall_ms and 0.0 < ms_cmb <= wall_ms
        for l in range(c.L):
            assert np.array_equal(out[l], ref[l])
        # a read with reset clears the counts
        assert c.pool.profile_read(0) == (0, 0.0)
    finally:
        c.close()


def test_profile_streamed_lanes_and_prefill():
    # streamed pages through the ring on several lanes, and a block wide
    # enough for the prefill kernel (more than 64 rows per kv head)
    c = small_case(mask_random(0.3, seed=21), n_layers=2, Hkv=2, Hq=12, max_q=16, ring=12, chunk=2)
    try:
        n_q = 16   # 16 queries x 6 heads = 96 rows per kv head: the prefill kernel
        qs = [c.queries(l, n_q, "f16") for l in range(c.L)]
        kw = dict(q_pos0=c.n_kv - n_q, scale=0.088, causal=True, prefetch=True)
        ref, _ = _run(c, qs, **kw)
        for kind in (0, 1):
            c.pool.profile_read(kind, reset=True)
        c.pool.profile_enable(True)
        out, _ = _run(c, qs, **kw)
        c.pool.profile_enable(False)
        n_att, ms_att = c.pool.profile_read(0)
        n_cmb, ms_cmb = c.pool.profile_read(1)
        say(f"streamed profile: {n_att} attention {ms_att:.4f} ms, {n_cmb} combines")
        assert n_cmb == c.L
        assert n_att >= c.L and ms_att > 0.0      # resident launch plus chunk launches on the lanes
        for l in range(c.L):
            assert np.array_equal(out[l], ref[l])
    finally:
        c.close()


def test_profiling_stays_off_graph_capture():
    # launches captured into a graph are not timed (a replay would not refill
    # the event pair); capture and replays work with profiling on
    c = small_case(mask_all, n_layers=1, Hkv=2, Hq=12)
    try:
        q = torch.from_numpy(c.queries(0, 1, "f32")).cuda()
        ref = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        c.pool.attend(0, q, c.n_kv, c.n_kv - 1, 1.0, False, ref, None)
        torch.cuda.synchronize()
        for kind in (0, 1):
            c.pool.profile_read(kind, reset=True)
        c.pool.profile_enable(True)
        out = torch.empty_like(ref)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            c.pool.attend(0, q, c.n_kv, c.n_kv - 1, 1.0, False, out, None, stream=s)   # eager: timed
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            c.pool.attend(0, q, c.n_kv, c.n_kv - 1, 1.0, False, out, None, stream=s)
        for rep in range(3):
            out.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            say(f"graph replay {rep} with profiling on")
            assert torch.equal(out, ref)
        c.pool.profile_enable(False)
        n_att, _ = c.pool.profile_read(0)
        n_cmb, _ = c.pool.profile_read(1)
        assert (n_att, n_cmb) == (1, 1)   # the eager call only
    finally:
        c.close()
