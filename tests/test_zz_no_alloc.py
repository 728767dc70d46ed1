"""kvs_attend_noalloc through the C ABI: the same kernels as kvs_attend with
the split-K partials in the library's fixed scratch array. Its outputs equal
kvs_attend's bit for bit, on two calls in a row where the second has the
smaller input (fewer query tokens, a shorter layer); a call that would need
more than the fixed scratch is refused before any device work."""

import numpy as np
import pytest
import torch

import host_streamed_paged_amd as kvs
from kvs_case import Case, mask_random, normwise_error, say

pytestmark = pytest.mark.gpu

N_KV_LONG = 5 * 256 + 77
N_KV_SHORT = 2 * 256 + 31


def run(pool, fn, layer, q, n_kv, q_pos0, causal):
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    getattr(pool, fn)(layer, q, n_kv, q_pos0, 1.0, causal, out, lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("widths", [(4, 2), (12, 1)], ids=["verify-then-smaller", "prefill-then-decode"])
def test_noalloc_equals_attend_on_consecutive_calls(widths):
    say(f"noalloc widths={widths}")
    c_long = Case(cid=121, n_layers=1, n_kv_heads=2, n_q_heads=12, n_kv=N_KV_LONG,
                  cfg_kw=dict(max_q_tokens=max(widths), ring_pages=4, chunk_pages=2, group_pages=2),
                  resident_fn=mask_random(0.5, seed=3))
    c_short = Case(cid=122, n_layers=1, n_kv_heads=2, n_q_heads=12, n_kv=N_KV_SHORT,
                   cfg_kw=dict(max_q_tokens=max(widths), ring_pages=4, chunk_pages=2, group_pages=1),
                   resident_fn=mask_random(0.5, seed=4))
    try:
        for case, n_kv, n_q in ((c_long, N_KV_LONG, widths[0]), (c_short, N_KV_SHORT, widths[1])):
            q = torch.from_numpy(case.queries(0, n_q, "f16" if n_q > 6 else "f32")).cuda()
            o_ref, l_ref = run(case.pool, "attend", 0, q, n_kv, n_kv - n_q, True)
            o, l = run(case.pool, "attend_noalloc", 0, q, n_kv, n_kv - n_q, True)
            say(f"n_kv={n_kv} n_q={n_q}: noalloc vs attend equal={np.array_equal(o, o_ref)}")
            assert np.array_equal(o, o_ref) and np.array_equal(l, l_ref)
            ref, _ = case.oracle(0, q.cpu().numpy(), q_pos0=n_kv - n_q, scale=1.0, causal=True)
            assert normwise_error(o, ref) <= 2e-3
    finally:
        c_long.close()
        c_short.close()


def test_noalloc_refuses_more_than_its_scratch():
    # 6 one-page groups x 300 query tokens x 12 heads x 520 B > 4 MiB
    c = Case(cid=123, n_layers=1, n_kv_heads=2, n_q_heads=12, n_kv=N_KV_LONG,
             cfg_kw=dict(max_q_tokens=300, ring_pages=4, chunk_pages=2, group_pages=1),
             resident_fn=mask_random(0.5, seed=5))
    try:
        q = torch.zeros((300, 12, 128), dtype=torch.float16, device="cuda")
        out = torch.empty((300, 12, 128), dtype=torch.float32, device="cuda")
        with pytest.raises(kvs.KvsError) as e:
            c.pool.attend_noalloc(0, q, N_KV_LONG, N_KV_LONG - 300, 1.0, True, out)
        assert e.value.code == kvs.ERR_INVALID_ARG and "scratch" in str(e.value)
        # the pool is still usable afterwards
        c.pool.attend_noalloc(0, q[:4], N_KV_LONG, N_KV_LONG - 4, 1.0, True, out[:4])
        torch.cuda.synchronize()
        assert np.all(np.isfinite(out[:4].cpu().numpy()))
    finally:
        c.close()
