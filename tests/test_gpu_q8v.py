"""The q8_0-q8_0 pair (Q8_0 K and Q8_0 V; page 3, "1. Correctness - PPL
parity" runs its cache with -ctk q8_0 -ctv q8_0) on the GPU, through the C
ABI, against the oracle: the same bars as the q8_0-q4_0 pair (gathers
bit-exact; attention within 2e-3 normwise per row and lse within 2e-3 at
decode, verify, intermediate and prefill widths; bits independent of
residency, ring and chunk sizes). Block-format edge cases and appends for
this pair run in the edge and append tests."""

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


def q8_case(resident_fn, *, cid=71, n_layers=2, Hkv=2, Hq=12, max_q=1, ring=4, chunk=2, group=1, flags=0):
    say(f"q8_0-q8_0 case cid={cid} layers={n_layers} n_kv={N_KV} ring={ring} chunk={chunk} group={group} "
        f"flags={flags} residency={getattr(resident_fn, '__name__', 'fn')}")
    return Case(cid=cid, n_layers=n_layers, n_kv_heads=Hkv, n_q_heads=Hq, n_kv=N_KV, type_v="q8_0",
                cfg_kw=dict(max_q_tokens=max_q, ring_pages=ring, chunk_pages=chunk, group_pages=group, flags=flags),
                resident_fn=resident_fn)


def test_pair_is_supported_and_page_size():
    assert kvs.type_pair_supported(kvs.TYPE_Q8_0, kvs.TYPE_Q8_0)
    assert not kvs.type_pair_supported(kvs.TYPE_Q4_0, kvs.TYPE_Q8_0)
    cfg = kvs.Config(n_layers=1, n_kv_heads=4, n_q_heads=24, max_pages=8, type_v=kvs.TYPE_Q8_0)
    assert kvs.page_bytes(cfg) == 4 * 256 * (136 + 136) == 278528


@pytest.mark.parametrize("resident", [mask_all, mask_none, mask_random(0.5)], ids=["all", "none", "half"])
def test_gather_bit_exact(resident):
    c = q8_case(resident)
    try:
        for l in range(c.L):
            for tok0, n_tok in [(0, c.n_pages * 256), (100, 700), (N_KV - 1, 1)]:
                say(f"kvs_debug_gather layer={l} tok0={tok0} n_tok={n_tok}")
                k = torch.empty((n_tok, c.Hkv, 128), dtype=torch.float32, device="cuda")
                v = torch.empty_like(k)
                c.pool.debug_gather(l, tok0, n_tok, k, v)
                torch.cuda.synchronize()
                rk, rv = gather_kv(c.records[l], c.Hkv, 128, tok0, n_tok, type_v="q8_0")
                valid = max(0, min(n_tok, N_KV - tok0))
                assert np.array_equal(k.cpu().numpy()[:valid], rk[:valid].astype(np.float32))
                assert np.array_equal(v.cpu().numpy()[:valid], rv[:valid].astype(np.float32))
    finally:
        c.close()


def check(c, outs, lses, qs, *, q_pos0, scale, causal):
    for l in range(c.L):
        ref, ref_lse = c.oracle(l, qs[l], q_pos0=q_pos0, scale=scale, causal=causal)
        err = normwise_error(outs[l], ref)
        lerr = float(np.max(np.abs(lses[l] - ref_lse)))
        say(f"layer {l}: normwise {err:.3e} lse {lerr:.3e}")
        assert err <= TOL, (l, err)
        assert lerr <= TOL, (l, lerr)


# (query tokens, dtype, causal, scale): decode rows 6 and 3 per kv head (the
# decode kernel), 24 and 36 rows (the matrix-core kernel), 300 tokens (the
# prefill kernel)
WIDTHS = [(1, "f32", False, 1.0, 12), (1, "f32", False, 1.0, 6), (4, "f32", True, 1.0, 12),
          (6, "f16", True, 1 / math.sqrt(128), 12), (300, "f16", True, 1 / math.sqrt(128), 12)]


@pytest.mark.parametrize("n_q,qdt,causal,scale,Hq", WIDTHS, ids=["decode6", "decode3", "verify", "rows36", "prefill"])
@pytest.mark.parametrize("resident", [mask_all, mask_random(0.4, seed=2)], ids=["all", "mixed"])
def test_attention_parity(n_q, qdt, causal, scale, Hq, resident):
    c = q8_case(resident, Hq=Hq, max_q=n_q, group=2)
    try:
        qs = [c.queries(l, n_q, qdt) for l in range(c.L)]
        q_pos0 = N_KV - n_q if causal else N_KV - 1
        outs, lses = c.attend_all(qs, q_pos0=q_pos0, scale=scale, causal=causal)
        check(c, outs, lses, qs, q_pos0=q_pos0, scale=scale, causal=causal)
    finally:
        c.close()


@pytest.mark.parametrize("n_q,qdt", [(1, "f32"), (40, "f16")], ids=["decode", "prefill"])
def test_bit_identical_across_residency_ring_and_chunks(n_q, qdt):
    base = None
    for v in [dict(resident=mask_all, ring=4, chunk=2),
              dict(resident=mask_none, ring=2, chunk=1, flags=kvs.FLAG_POISON_RING),
              dict(resident=mask_random(0.4, seed=9), ring=8, chunk=4),
              dict(resident=mask_none, ring=6, chunk=3, flags=kvs.FLAG_ZERO_COPY)]:
        c = q8_case(v["resident"], max_q=n_q, ring=v["ring"], chunk=v["chunk"], group=3, flags=v.get("flags", 0))
        try:
            qs = [c.queries(l, n_q, qdt) for l in range(c.L)]
            q_pos0 = N_KV - n_q
            outs, lses = c.attend_all(qs, q_pos0=q_pos0, scale=0.12, causal=True)
            if base is None:
                check(c, outs, lses, qs, q_pos0=q_pos0, scale=0.12, causal=True)
                base = (outs, lses)
            else:
                for l in range(c.L):
                    assert np.array_equal(outs[l], base[0][l]), (v, l)
                    assert np.array_equal(lses[l], base[1][l]), (v, l)
        finally:
            c.close()
