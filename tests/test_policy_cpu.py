"""Pool policy (pure host functions, no device): automatic sizing and the
newest-page residency rule.

Pins: the resident tokens and stage sizes page 3 logs for its automatic
sizing (tests/golden/page3_sizes.json), the floor and ceiling it states, and
hand-worked residency updates; properties on random masks.
"""

import json
import math
import os

import numpy as np
from hypothesis import given, settings, strategies as st

import host_streamed_paged_amd as kvs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page3_sizes.json")


def test_resident_tokens_match_the_logged_ones():
    g = json.load(open(GOLDEN))
    for case in g["residency"]["cases"]:
        assert kvs.auto_resident_pages(case["n_ctx"]) * 256 == case["printed_resident_tokens"]


def test_stage_sizes_match_the_logged_ones():
    g = json.load(open(GOLDEN))
    for case in g["auto_stage"]["cases"]:
        mib = kvs.auto_stage_bytes(case["layers"], case["n_ctx"], case["bytes_per_token"]) / 2 ** 20
        assert round(mib, case["printed_decimals"]) == case["printed_mib"], case


def test_floor_ceiling_and_small_contexts():
    assert kvs.auto_resident_pages(0) == 0
    assert kvs.auto_resident_pages(4096) == 8          # 10 % is 410 tokens: the 2048-token floor wins
    assert kvs.auto_resident_pages(20480) == 8         # 2048 tokens exactly
    assert kvs.auto_resident_pages(20481) == 9         # 2049 tokens, rounded up to 9 pages
    assert kvs.auto_resident_pages(1000) == 4          # never more than the context's own pages
    assert kvs.auto_stage_bytes(64, 2 ** 24, 4096) == 8192 * 2 ** 20   # capped at 8192 MiB
    assert kvs.auto_stage_bytes(0, 65536, 2176) == 0


def test_budget_is_the_minimum_plus_the_resident_pages():
    cfg = kvs.Config(n_layers=16, n_kv_heads=4, n_q_heads=24, max_pages=1024, max_q_tokens=1,
                     ring_pages=32, chunk_pages=4, group_pages=1)
    base, pb = kvs.min_budget_bytes(cfg), kvs.page_bytes(cfg)
    assert kvs.auto_budget_bytes(cfg, 0) == base
    b = kvs.auto_budget_bytes(cfg, 262144)
    assert b == base + 16 * 103 * pb
    assert kvs.slots_for_budget(cfg, b) == 16 * 103
    big = kvs.Config(n_layers=64, n_kv_heads=8, n_q_heads=64, max_pages=65536, max_q_tokens=1,
                     ring_pages=32, chunk_pages=4, group_pages=1)
    assert kvs.auto_budget_bytes(big, 2 ** 24) == 8192 * 2 ** 20


def test_promote_newest_hand_worked():
    # 4 resident of 6; three new pages with room for 4: each new page pushes out the oldest
    assert kvs.residency_promote_newest([1, 0, 1, 1, 0, 1], 9, 4).tolist() == [0, 0, 0, 0, 0, 1, 1, 1, 1]
    # room to spare: nothing is evicted
    assert kvs.residency_promote_newest([1, 0, 0], 5, 10).tolist() == [1, 0, 0, 1, 1]
    # no growth: unchanged
    assert kvs.residency_promote_newest([0, 1, 1], 3, 1).tolist() == [0, 1, 1]
    # no room at all: new pages stream
    assert kvs.residency_promote_newest([0, 0], 4, 0).tolist() == [0, 0, 0, 0]
    # from an empty layer
    assert kvs.residency_promote_newest([], 3, 2).tolist() == [0, 1, 1]


@settings(max_examples=300, deadline=None)
@given(n_cur=st.integers(0, 40), grow=st.integers(0, 20), max_res=st.integers(0, 30), seed=st.integers(0, 2 ** 31 - 1))
def test_promote_newest_properties(n_cur, grow, max_res, seed):
    cur = (np.random.default_rng(seed).random(n_cur) < 0.5).astype(np.uint8)
    n_new = n_cur + grow
    out = kvs.residency_promote_newest(cur, n_new, max_res)
    assert out.shape == (n_new,)
    assert np.all(out[:n_cur] <= cur), "a streamed page was promoted"
    if grow == 0:
        assert np.array_equal(out, cur)
        return
    # the newest min(grow, max_res) pages are resident, older new ones are not
    k = min(grow, max_res)
    assert np.all(out[n_new - k:] == 1) and np.all(out[n_cur:n_new - k] == 0)
    total = int(out.sum())
    assert total == max(k, min(int(cur.sum()) + k, max_res)) if max_res > 0 else total == int(cur.sum())
    # what was evicted is the oldest: every page still resident is newer than every evicted one
    evicted = np.where((cur == 1) & (out[:n_cur] == 0))[0]
    kept = np.where(out[:n_cur] == 1)[0]
    if evicted.size and kept.size:
        assert evicted.max() < kept.min()
