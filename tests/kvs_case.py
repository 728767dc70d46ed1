"""Shared setup for GPU tests: seeded pages in pinned memory, a pool, and the
oracle's reference for the same bytes."""

import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import host_streamed_paged_amd as kvs
from kvs_synth import KVGeometry, layer_records, make_q, residency_mask
from oracle import attend_layer


def say(msg: str):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def normwise_error(out: np.ndarray, ref: np.ndarray) -> float:
    """max over rows (query token x head) of max_c |o - r| / max_c |r|."""
    num = np.max(np.abs(out.astype(np.float64) - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den))


class Case:
    """L layers of seeded pages, registered with a fresh pool."""

    def __init__(self, *, cid, n_layers, n_kv_heads, n_q_heads, n_kv, cfg_kw, resident_fn, slots=None,
                 tail="poison", threads=8, type_v="q4_0"):
        self.cid, self.L, self.Hkv, self.Hq, self.n_kv = cid, n_layers, n_kv_heads, n_q_heads, n_kv
        self.type_v = type_v
        self.geom = KVGeometry(n_kv_heads, 128, type_v=type_v)
        self.n_pages = -(-n_kv // 256)
        with ThreadPoolExecutor(threads) as ex:
            self.records = list(ex.map(lambda l: layer_records(cid, l, n_kv, self.geom, tail=tail), range(n_layers)))
        self.host = [torch.from_numpy(r).pin_memory() for r in self.records]
        self.masks = [np.asarray(resident_fn(l, self.n_pages), np.uint8) for l in range(n_layers)]
        cfg = dict(n_layers=n_layers, n_kv_heads=n_kv_heads, n_q_heads=n_q_heads, max_pages=max(1, self.n_pages),
                   type_v=kvs.TYPE_Q8_0 if type_v == "q8_0" else kvs.TYPE_Q4_0)
        cfg.update(cfg_kw)
        self.cfg = kvs.Config(**cfg)
        need = int(sum(m.sum() for m in self.masks))
        self.arena = kvs.Pool.arena_for(self.cfg, need if slots is None else slots)
        self.pool = kvs.Pool(self.cfg, self.arena)
        for l in range(n_layers):
            self.pool.host_pages_set(l, self.host[l])
            self.pool.page_table_set(l, self.masks[l])

    def close(self):
        self.pool.close()

    def queries(self, layer, n_q, dtype):
        return make_q(self.cid, layer, n_q, self.Hq, 128, dtype)

    def attend_all(self, qs, *, q_pos0, scale, causal, stream=None, prefetch=True):
        """Run kvs_attend for every layer in order; returns (out, lse) lists (numpy)."""
        outs, lses = [], []
        dq = [torch.from_numpy(q).cuda() for q in qs]
        res = []
        for l in range(self.L):
            if prefetch:
                self.pool.stream_enqueue(l)
            out = torch.empty(dq[l].shape, dtype=torch.float32, device="cuda")
            lse = torch.empty(dq[l].shape[:2], dtype=torch.float32, device="cuda")
            self.pool.attend(l, dq[l], self.n_kv, q_pos0, scale, causal, out, lse, stream=stream)
            res.append((out, lse))
        torch.cuda.synchronize()
        for out, lse in res:
            outs.append(out.cpu().numpy())
            lses.append(lse.cpu().numpy())
        return outs, lses

    def oracle(self, layer, q, *, q_pos0, scale, causal, heads=None):
        return attend_layer(self.records[layer], q, n_kv=self.n_kv, n_kv_heads=self.Hkv, head_dim=128,
                            scale=scale, causal=causal, q_pos0=q_pos0, heads=heads, type_v=self.type_v)


def mask_all(l, n):
    return np.ones(n, np.uint8)


def mask_none(l, n):
    return np.zeros(n, np.uint8)


def mask_random(frac, seed=0):
    def f(l, n):
        return residency_mask(1000 + seed, l, n, int(round(frac * n)))
    return f
