"""Launch-plan invariants of the host runtime, through kvs_plan_layer (pure
host code: no device needed).

The plan splits one layer's pages into a resident launch and ring-chunk
launches. The kernels rely on: every page computed exactly once; a group's
pages computed in ascending order; a chunk launch reading only streamed pages
of its own chunk; chunks of at most chunk_pages pages in ascending streamed
order. When group_pages <= chunk_pages the planner keeps each group inside
one launch, which is what lets two chunk launches run concurrently.
"""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import host_streamed_paged_amd as kvs


def cfg_for(n_pages, G, C, ring=None):
    ring = ring if ring is not None else 4 * C
    return kvs.Config(n_layers=1, n_kv_heads=4, n_q_heads=24, max_pages=max(1, n_pages), max_q_tokens=4,
                      ring_pages=ring, chunk_pages=C, group_pages=G)


def check_plan(mask, G, C):
    n = len(mask)
    info, segs, chunks = kvs.plan_layer(cfg_for(n, G, C), mask)
    streamed = [i for i in range(n) if not mask[i]]
    rank = {p: r for r, p in enumerate(streamed)}
    n_groups = -(-n // G)
    assert info.n_groups == n_groups and info.n_streamed == len(streamed)
    assert info.n_segs == len(segs) and info.n_chunks == len(chunks)

    # chunks: ascending, contiguous ranks, at most C pages each, covering every streamed page
    r = 0
    for c, (rank0, npages, seg0, nseg) in enumerate(chunks):
        assert rank0 == r and 1 <= npages <= C
        r += npages
    assert r == len(streamed)

    # segments: resident launch first, then each chunk's
    owner = [None] * n           # launch index that computes each page (-1 resident)
    next_page = [g * G for g in range(n_groups)]
    launches = [(-1, 0, info.n_resident_segs)] + [(c, ch[2], ch[3]) for c, ch in enumerate(chunks)]
    assert launches[1][1] == info.n_resident_segs if len(chunks) else True
    group_launches = {}
    for li, seg0, nseg in launches:
        for group, page0, npg, flags in segs[seg0:seg0 + nseg]:
            assert npg >= 1 and page0 == next_page[group], "group pages out of order"
            assert bool(flags & 1) == (page0 == group * G)
            for p in range(page0, page0 + npg):
                assert p // G == group and owner[p] is None
                owner[p] = li
                if li == -1:
                    assert mask[p], "resident launch reads a streamed page"
                elif not mask[p]:
                    rank0, npages = chunks[li][0], chunks[li][1]
                    assert rank0 <= rank[p] < rank0 + npages, "chunk launch reads another chunk's page"
            next_page[group] = page0 + npg
            group_launches.setdefault(group, set()).add(li)
    assert all(o is not None for o in owner), "page not computed"

    # resident launch = exactly the groups with no streamed page, whole
    fully_res = {g for g in range(n_groups) if all(mask[g * G:min(n, (g + 1) * G)])}
    assert {int(s[0]) for s in segs[:info.n_resident_segs]} == fully_res

    split = any(len(v) > 1 for v in group_launches.values())
    assert info.whole_groups == (0 if split else 1)
    if G <= C:
        assert info.whole_groups == 1
    max_streamed_in_group = max([sum(1 for p in range(g * G, min(n, (g + 1) * G)) if not mask[p])
                                 for g in range(n_groups)] or [0])
    if max_streamed_in_group > C:
        assert info.whole_groups == 0
    return info, segs, chunks


def test_single_page_groups_give_full_chunks():
    rng = np.random.default_rng(0)
    mask = (rng.random(300) < 0.3).astype(np.uint8)
    info, segs, chunks = check_plan(mask, 1, 4)
    n_str = int((mask == 0).sum())
    assert list(chunks[:, 1]) == [4] * (n_str // 4) + ([n_str % 4] if n_str % 4 else [])


def test_groups_are_never_split_when_they_fit_a_chunk():
    rng = np.random.default_rng(1)
    mask = (rng.random(640) < 0.28).astype(np.uint8)
    info, segs, chunks = check_plan(mask, 4, 4)
    assert info.whole_groups == 1
    assert np.all(segs[:, 3] & 1), "every segment starts its group"


def test_large_groups_are_split_across_chunks():
    mask = np.zeros(64, np.uint8)
    info, segs, chunks = check_plan(mask, 16, 4)
    assert info.whole_groups == 0 and info.n_chunks == 16


def test_all_resident_and_empty_layers():
    info, segs, chunks = check_plan(np.ones(37, np.uint8), 3, 2)
    assert info.n_chunks == 0 and info.n_resident_segs == 13
    info, segs, chunks = check_plan(np.zeros(0, np.uint8), 3, 2)
    assert info.n_segs == 0 and info.n_chunks == 0


@settings(max_examples=300, deadline=None)
@given(n=st.integers(1, 90), G=st.integers(1, 12), C=st.sampled_from([1, 2, 3, 4, 8, 16]),
       frac=st.floats(0.0, 1.0), seed=st.integers(0, 2**31 - 1))
def test_plan_invariants_random(n, G, C, frac, seed):
    mask = (np.random.default_rng(seed).random(n) < frac).astype(np.uint8)
    check_plan(mask, G, C)


def test_plan_rejects_bad_arguments():
    cfg = cfg_for(8, 2, 4)
    with pytest.raises(kvs.KvsError) as e:
        kvs.plan_layer(cfg, np.ones(9, np.uint8))   # more pages than max_pages
    assert e.value.code == kvs.ERR_INVALID_ARG
    bad = cfg_for(8, 2, 3, ring=16)                  # chunk does not divide the ring
    with pytest.raises(kvs.KvsError):
        kvs.plan_layer(bad, np.ones(8, np.uint8))
