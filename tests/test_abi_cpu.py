"""The C-ABI library without a GPU: it loads, exports every declared symbol,
and its pure configuration, type-pair and budget functions behave as
documented. No compute call is made."""

import ctypes
import os
import re

import pytest

import host_streamed_paged_amd as kvs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    with open(os.path.join(ROOT, "include", "kvs.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvs_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = kvs.lib()
    names = declared_symbols()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert sorted(kvs.EXPORTS) == names


def base_cfg(**kw):
    c = dict(n_layers=16, n_kv_heads=4, n_q_heads=24, max_pages=1024, max_q_tokens=1, ring_pages=16,
             chunk_pages=4, group_pages=1)
    c.update(kw)
    return kvs.Config(**c)


def test_type_pair_gate():
    assert kvs.type_pair_supported(kvs.TYPE_Q8_0, kvs.TYPE_Q4_0)
    assert kvs.type_pair_supported(kvs.TYPE_Q8_0, kvs.TYPE_Q8_0)
    for tk, tv in [(kvs.TYPE_F16, kvs.TYPE_F16), (kvs.TYPE_Q4_0, kvs.TYPE_Q4_0), (kvs.TYPE_Q4_0, kvs.TYPE_Q8_0),
                   (kvs.TYPE_Q8_0, kvs.TYPE_F16)]:
        assert not kvs.type_pair_supported(tk, tv)
    assert kvs.config_validate(base_cfg(type_k=kvs.TYPE_Q8_0, type_v=kvs.TYPE_Q8_0)) == kvs.OK
    rc = kvs.config_validate(base_cfg(type_k=kvs.TYPE_F16, type_v=kvs.TYPE_F16))
    assert rc == kvs.ERR_UNSUPPORTED
    assert "Q8_0" in kvs.last_error() and "Q4_0" in kvs.last_error()


def test_page_bytes_per_type_pair():
    """The record sizes of both pairs: 256 tokens x Hkv x (136 B of Q8_0 K +
    72 B of Q4_0 V or 136 B of Q8_0 V), as the oracle computes them."""
    from oracle import page_bytes as oracle_page_bytes
    for tv, name in [(kvs.TYPE_Q4_0, "q4_0"), (kvs.TYPE_Q8_0, "q8_0")]:
        for hkv in (1, 4, 8):
            cfg = base_cfg(n_kv_heads=hkv, n_q_heads=6 * hkv, type_v=tv)
            assert kvs.page_bytes(cfg) == oracle_page_bytes(hkv, 128, 256, "q8_0", name)


@pytest.mark.parametrize("kw,code", [
    (dict(), kvs.OK),
    (dict(head_dim=64), kvs.ERR_UNSUPPORTED),
    (dict(page_tokens=128), kvs.ERR_UNSUPPORTED),
    (dict(n_layers=0), kvs.ERR_INVALID_ARG),
    (dict(n_q_heads=25), kvs.ERR_INVALID_ARG),
    (dict(n_q_heads=2), kvs.ERR_INVALID_ARG),
    (dict(max_pages=0), kvs.ERR_INVALID_ARG),
    (dict(max_q_tokens=0), kvs.ERR_INVALID_ARG),
    (dict(ring_pages=16, chunk_pages=5), kvs.ERR_INVALID_ARG),
    (dict(group_pages=0), kvs.ERR_INVALID_ARG),
    (dict(flags=kvs.FLAG_ZERO_COPY), kvs.OK),
    (dict(flags=kvs.FLAG_ZERO_COPY | kvs.FLAG_POISON_RING), kvs.OK),
    (dict(flags=4), kvs.ERR_INVALID_ARG),
])
def test_config_validation(kw, code):
    assert kvs.config_validate(base_cfg(**kw)) == code


def test_page_bytes_and_budget_math():
    c = base_cfg()
    pb = kvs.page_bytes(c)
    assert pb == 212992
    mb = kvs.min_budget_bytes(c)
    ring = 16 * pb
    groups = 1024
    work = groups * 1 * 24 * 130 * 4
    tables = 16 * (1024 * 4 + (2 * groups + 1024 + 1) * 16)
    assert mb >= ring + work + tables
    assert mb <= ring + work + tables + 256 * (2 + 2 * 16)
    assert kvs.slots_for_budget(c, mb - 1) == 0
    assert kvs.slots_for_budget(c, mb) == 0
    assert kvs.slots_for_budget(c, mb + 103 * 16 * pb) == 103 * 16
    # slot indices travel in 24 bits of the device launch plan: the count is capped
    assert kvs.slots_for_budget(c, mb + (1 << 24) * pb) == (1 << 23) - 1
    # the smallest useful pool holds one page of ring
    one = base_cfg(ring_pages=1, chunk_pages=1, max_pages=1, n_layers=1)
    assert kvs.min_budget_bytes(one) >= kvs.page_bytes(one)


def test_workspace_scales_with_verify_width_and_groups():
    a = kvs.min_budget_bytes(base_cfg(max_q_tokens=1))
    b = kvs.min_budget_bytes(base_cfg(max_q_tokens=4))
    assert b - a >= 3 * 1024 * 24 * 130 * 4
    c = kvs.min_budget_bytes(base_cfg(max_q_tokens=4, group_pages=8))
    assert c < b
