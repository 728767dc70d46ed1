"""The seeded generator: workloads, determinism, residency patterns."""

import json
import os

import numpy as np

from kvs_synth import KVGeometry, WORKLOADS, layer_records, make_q, residency_mask
from kvs_synth.configs import _ten_percent_pages

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_ten_percent_residency_matches_page3():
    with open(os.path.join(GOLDEN, "page3_sizes.json")) as f:
        g = json.load(f)["residency"]
    for c in g["cases"]:
        assert _ten_percent_pages(c["n_ctx"]) * 256 == c["printed_resident_tokens"]


def test_workload_shapes():
    w = WORKLOADS
    assert w["tiny_decode"].n_pages == 4
    assert w["resident_decode_32k"].n_pages == 128
    assert w["streamed_decode_256k"].n_pages == 1024 and w["streamed_decode_256k"].resident_pages == 103
    assert w["spec_verify_160k"].n_pages == 640 and w["spec_verify_160k"].resident_pages == 180
    p = w["prefill_ubatch_128k"]
    assert p.n_pages == 513 and p.resident_pages == 52 and p.q_pos0 + p.n_q == p.n_kv


def test_generation_is_deterministic_and_slab_independent():
    geom = KVGeometry(2, 64, 16)
    a = layer_records(9, 3, 100, geom, slab_pages=64)
    b = layer_records(9, 3, 100, geom, slab_pages=1)
    assert np.array_equal(a, b)
    c = layer_records(9, 4, 100, geom)
    assert not np.array_equal(a, c)
    assert np.array_equal(make_q(9, 0, 2, 4, 64, "f32"), make_q(9, 0, 2, 4, 64, "f32"))


def test_residency_mask_recipe():
    m = residency_mask(3, 0, 1024, 103)
    assert m.sum() == 103 and np.all(m[-52:] == 1)
    m2 = residency_mask(5, 0, 513, 52, own_page=True)
    assert m2[-1] == 1 and m2.sum() == 53 and np.all(m2[-27:] == 1)
    assert np.array_equal(residency_mask(3, 0, 1024, 103), m)
    assert not np.array_equal(residency_mask(3, 1, 1024, 103), m)
    assert residency_mask(1, 0, 4, 4).sum() == 4
