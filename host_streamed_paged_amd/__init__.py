"""Python binding of libkvs.so, the host-streamed paged attention library.

Argument marshalling only: every step of the path (ring copies, page
gathers, dequantization, attention, split-K combine) runs in the HIP library.
PyTorch only supplies device memory, pinned host memory and streams. If the
library is not built this module raises at first use; there is no fallback.

The C ABI is declared in include/kvs.h; the names here mirror it.
"""

import ctypes
import os
from dataclasses import dataclass

import numpy as np

import torch  # noqa: F401  (loads the HIP runtime the library binds to)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvs.so")

TYPE_F16, TYPE_Q4_0, TYPE_Q8_0 = 1, 2, 8
Q_F32, Q_F16 = 0, 1
FLAG_POISON_RING = 1
FLAG_ZERO_COPY = 2

OK = 0
ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_BUDGET, ERR_NO_SLOTS = -1, -2, -3, -4
ERR_BATCH_TOO_WIDE, ERR_NOT_READY, ERR_STATE, ERR_NOT_RESIDENT, ERR_HIP = -5, -6, -7, -8, -9
_ERR_NAMES = {
    -1: "INVALID_ARG", -2: "UNSUPPORTED", -3: "BUDGET", -4: "NO_SLOTS", -5: "BATCH_TOO_WIDE",
    -6: "NOT_READY", -7: "STATE", -8: "NOT_RESIDENT", -9: "HIP",
}

EXPORTS = [
    "kvs_type_pair_supported", "kvs_config_validate", "kvs_page_bytes", "kvs_min_budget_bytes",
    "kvs_slots_for_budget", "kvs_plan_layer", "kvs_pool_create", "kvs_pool_destroy", "kvs_host_pages_set",
    "kvs_page_table_set", "kvs_stream_enqueue", "kvs_attend", "kvs_status", "kvs_debug_gather",
    "kvs_debug_read_page", "kvs_last_error", "kvs_profile_enable", "kvs_profile_read", "kvs_append",
    "kvs_auto_resident_pages", "kvs_auto_stage_bytes", "kvs_auto_budget_bytes", "kvs_residency_promote_newest",
    "kvs_pool_pin_layer", "kvs_pool_reset_pinned", "kvs_debug_export_pages", "kvs_debug_stage",
    "kvs_attend_noalloc",
]

NOALLOC_SCRATCH_BYTES = 4 << 20   # KVS_NOALLOC_SCRATCH_BYTES

STAGED_TILE_BYTES = 135424   # KVS_STAGED_TILE_BYTES


class KvsError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{_ERR_NAMES.get(code, code)}: {message}")
        self.code = code


class KvsConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "n_kv_heads", "n_q_heads", "head_dim", "page_tokens", "type_k", "type_v",
        "max_pages", "max_q_tokens", "ring_pages", "chunk_pages", "group_pages")] + [
        ("flags", ctypes.c_uint32)]


class KvsPlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_groups", "n_streamed", "n_segs", "n_resident_segs", "n_chunks", "whole_groups")]


class KvsStatus(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "page_bytes", "slot_count", "slots_used", "ring_pages", "workspace_bytes", "bytes_h2d",
        "pages_streamed", "copies_issued", "kernels_launched", "resident_upload_bytes", "pinned_slots")]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libkvs.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(python -m host_streamed_paged_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, U64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
    cfgp = ctypes.POINTER(KvsConfig)
    sig = {
        "kvs_type_pair_supported": (ctypes.c_int, [I32, I32]),
        "kvs_config_validate": (ctypes.c_int, [cfgp]),
        "kvs_page_bytes": (U64, [cfgp]),
        "kvs_min_budget_bytes": (ctypes.c_int, [cfgp, ctypes.POINTER(U64)]),
        "kvs_slots_for_budget": (I64, [cfgp, U64]),
        "kvs_plan_layer": (ctypes.c_int, [cfgp, I32, P, ctypes.POINTER(KvsPlanInfo), P, I32, P, I32]),
        "kvs_pool_create": (ctypes.c_int, [cfgp, P, U64, ctypes.POINTER(P)]),
        "kvs_pool_destroy": (None, [P]),
        "kvs_host_pages_set": (ctypes.c_int, [P, I32, P, I32]),
        "kvs_page_table_set": (ctypes.c_int, [P, I32, I32, P, P]),
        "kvs_stream_enqueue": (ctypes.c_int, [P, I32]),
        "kvs_attend": (ctypes.c_int, [P, I32, P, I32, I32, I64, I64, F, I32, P, P, P]),
        "kvs_attend_noalloc": (ctypes.c_int, [P, I32, P, I32, I32, I64, I64, F, I32, P, P, P]),
        "kvs_status": (ctypes.c_int, [P, ctypes.POINTER(KvsStatus)]),
        "kvs_debug_gather": (ctypes.c_int, [P, I32, I64, I64, P, P, P]),
        "kvs_append": (ctypes.c_int, [P, I32, P, P, I32, I64, I32, P]),
        "kvs_auto_resident_pages": (I32, [I64]),
        "kvs_auto_stage_bytes": (U64, [I32, I64, U64]),
        "kvs_auto_budget_bytes": (ctypes.c_int, [cfgp, I64, ctypes.POINTER(U64)]),
        "kvs_residency_promote_newest": (ctypes.c_int, [P, I32, I32, I32, P]),
        "kvs_debug_read_page": (ctypes.c_int, [P, I32, I32, P]),
        "kvs_debug_export_pages": (ctypes.c_int, [P, I32, P, P]),
        "kvs_debug_stage": (ctypes.c_int, [P, I32, I64, P, P]),
        "kvs_pool_pin_layer": (ctypes.c_int, [P, I32, I32]),
        "kvs_pool_reset_pinned": (ctypes.c_int, [P]),
        "kvs_last_error": (ctypes.c_char_p, []),
        "kvs_profile_enable": (ctypes.c_int, [P, I32]),
        "kvs_profile_read": (ctypes.c_int, [P, I32, ctypes.POINTER(I64), ctypes.POINTER(ctypes.c_double), I32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype, fn.argtypes = res, args
    _lib = L
    return L


def _check(rc: int):
    if rc != OK:
        raise KvsError(rc, lib().kvs_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(s):
    if s is None:
        s = torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


@dataclass
class Config:
    n_layers: int
    n_kv_heads: int
    n_q_heads: int
    max_pages: int
    max_q_tokens: int = 1
    ring_pages: int = 16
    chunk_pages: int = 4
    group_pages: int = 1
    head_dim: int = 128
    page_tokens: int = 256
    type_k: int = TYPE_Q8_0
    type_v: int = TYPE_Q4_0
    flags: int = 0

    def c(self) -> KvsConfig:
        return KvsConfig(self.n_layers, self.n_kv_heads, self.n_q_heads, self.head_dim, self.page_tokens,
                         self.type_k, self.type_v, self.max_pages, self.max_q_tokens, self.ring_pages,
                         self.chunk_pages, self.group_pages, self.flags)


def type_pair_supported(type_k: int, type_v: int) -> bool:
    return bool(lib().kvs_type_pair_supported(type_k, type_v))


def config_validate(cfg: Config) -> int:
    return lib().kvs_config_validate(ctypes.byref(cfg.c()))


def page_bytes(cfg: Config) -> int:
    return lib().kvs_page_bytes(ctypes.byref(cfg.c()))


def min_budget_bytes(cfg: Config) -> int:
    out = ctypes.c_uint64(0)
    _check(lib().kvs_min_budget_bytes(ctypes.byref(cfg.c()), ctypes.byref(out)))
    return out.value


def slots_for_budget(cfg: Config, budget: int) -> int:
    return lib().kvs_slots_for_budget(ctypes.byref(cfg.c()), budget)


def auto_resident_pages(n_ctx: int) -> int:
    """Resident pages per layer under automatic sizing (kvs_auto_resident_pages)."""
    return lib().kvs_auto_resident_pages(n_ctx)


def auto_stage_bytes(n_layers: int, n_ctx: int, bytes_per_token: int) -> int:
    """The pages' automatic stage size (kvs_auto_stage_bytes)."""
    return lib().kvs_auto_stage_bytes(n_layers, n_ctx, bytes_per_token)


def auto_budget_bytes(cfg: Config, n_ctx: int) -> int:
    """This pool's budget for automatic residency (kvs_auto_budget_bytes)."""
    out = ctypes.c_uint64(0)
    _check(lib().kvs_auto_budget_bytes(ctypes.byref(cfg.c()), n_ctx, ctypes.byref(out)))
    return out.value


def residency_promote_newest(cur, n_new: int, max_resident: int):
    """The residency mask after the layer grows to n_new pages
    (kvs_residency_promote_newest)."""
    cur = np.ascontiguousarray(np.asarray(cur, dtype=np.uint8))
    out = np.zeros(max(1, n_new), np.uint8)
    cp = cur.ctypes.data_as(ctypes.c_void_p) if cur.size else None
    _check(lib().kvs_residency_promote_newest(cp, int(cur.size), n_new, max_resident,
                                              out.ctypes.data_as(ctypes.c_void_p)))
    return out[:n_new]


def plan_layer(cfg: Config, resident):
    """The launch plan for one layer (kvs_plan_layer): (info, segments, chunks)
    with segments as rows {group, first page, pages, flags} and chunks as rows
    {first streamed rank, pages, first segment, segments}."""
    res = np.ascontiguousarray(np.asarray(resident, dtype=np.uint8))
    n = int(res.shape[0])
    info = KvsPlanInfo()
    c = cfg.c()
    rp = res.ctypes.data_as(ctypes.c_void_p) if n else None
    _check(lib().kvs_plan_layer(ctypes.byref(c), n, rp, ctypes.byref(info), None, 0, None, 0))
    segs = np.zeros((max(1, info.n_segs), 4), np.int32)
    chunks = np.zeros((max(1, info.n_chunks), 4), np.int32)
    _check(lib().kvs_plan_layer(ctypes.byref(c), n, rp, ctypes.byref(info),
                                segs.ctypes.data_as(ctypes.c_void_p), segs.shape[0],
                                chunks.ctypes.data_as(ctypes.c_void_p), chunks.shape[0]))
    return info, segs[:info.n_segs], chunks[:info.n_chunks]


def last_error() -> str:
    return lib().kvs_last_error().decode()


class Pool:
    """A kvs_pool over a caller-owned device arena (a torch uint8 tensor)."""

    def __init__(self, cfg: Config, arena: torch.Tensor):
        assert arena.is_cuda and arena.dtype == torch.uint8 and arena.is_contiguous()
        self.cfg = cfg
        self.arena = arena
        self._h = ctypes.c_void_p()
        self._host = {}
        _check(lib().kvs_pool_create(ctypes.byref(cfg.c()), _ptr(arena), arena.numel(), ctypes.byref(self._h)))

    @staticmethod
    def arena_for(cfg: Config, resident_slots: int, device="cuda") -> torch.Tensor:
        budget = min_budget_bytes(cfg) + resident_slots * page_bytes(cfg)
        return torch.empty(budget, dtype=torch.uint8, device=device)

    def close(self):
        if self._h:
            lib().kvs_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def host_pages_set(self, layer: int, records: torch.Tensor):
        """records: pinned uint8 tensor [n_pages, page_bytes]."""
        assert records.dtype == torch.uint8 and records.is_contiguous() and records.dim() == 2
        self._host[layer] = records
        _check(lib().kvs_host_pages_set(self._h, layer, _ptr(records), records.shape[0]))

    def page_table_set(self, layer: int, resident, stream=None):
        import numpy as np
        mask = np.ascontiguousarray(np.asarray(resident, dtype=np.uint8))
        _check(lib().kvs_page_table_set(self._h, layer, int(mask.size), mask.ctypes.data_as(ctypes.c_void_p),
                                        _stream(stream)))

    def stream_enqueue(self, layer: int):
        _check(lib().kvs_stream_enqueue(self._h, layer))

    def attend(self, layer: int, q: torch.Tensor, n_kv: int, q_pos0: int, scale: float, causal: bool,
               out: torch.Tensor, lse: torch.Tensor | None = None, stream=None):
        if q.dtype == torch.float32:
            qd = Q_F32
        elif q.dtype == torch.float16:
            qd = Q_F16
        else:
            raise TypeError("q must be float32 or float16")
        assert q.is_contiguous() and out.is_contiguous() and out.dtype == torch.float32
        assert q.dim() == 3 and out.shape == q.shape
        if lse is not None:
            assert lse.dtype == torch.float32 and lse.is_contiguous() and lse.shape == q.shape[:2]
        _check(lib().kvs_attend(self._h, layer, _ptr(q), qd, q.shape[0], q_pos0, n_kv, float(scale),
                                1 if causal else 0, _ptr(out), _ptr(lse), _stream(stream)))

    def attend_noalloc(self, layer: int, q: torch.Tensor, n_kv: int, q_pos0: int, scale: float, causal: bool,
                       out: torch.Tensor, lse: torch.Tensor | None = None, stream=None):
        """kvs_attend_noalloc: kvs_attend with the split-K partials in the
        library's fixed scratch array (no allocation)."""
        if q.dtype == torch.float32:
            qd = Q_F32
        elif q.dtype == torch.float16:
            qd = Q_F16
        else:
            raise TypeError("q must be float32 or float16")
        assert q.is_contiguous() and out.is_contiguous() and out.dtype == torch.float32
        assert q.dim() == 3 and out.shape == q.shape
        if lse is not None:
            assert lse.dtype == torch.float32 and lse.is_contiguous() and lse.shape == q.shape[:2]
        _check(lib().kvs_attend_noalloc(self._h, layer, _ptr(q), qd, q.shape[0], q_pos0, n_kv, float(scale),
                                        1 if causal else 0, _ptr(out), _ptr(lse), _stream(stream)))

    def append(self, layer: int, k_new: torch.Tensor, v_new: torch.Tensor, pos0: int, stream=None):
        """Quantize new K and V rows [n_tok, Hkv, head_dim] (f32 or f16, on the
        device) into the layer's records at tokens pos0 .. pos0 + n_tok - 1."""
        if k_new.dtype != v_new.dtype or k_new.dtype not in (torch.float32, torch.float16):
            raise TypeError("k_new and v_new must both be float32 or both float16")
        assert k_new.is_contiguous() and v_new.is_contiguous() and k_new.shape == v_new.shape and k_new.dim() == 3
        dt = Q_F32 if k_new.dtype == torch.float32 else Q_F16
        _check(lib().kvs_append(self._h, layer, _ptr(k_new), _ptr(v_new), dt, pos0, k_new.shape[0], _stream(stream)))

    def status(self) -> KvsStatus:
        st = KvsStatus()
        _check(lib().kvs_status(self._h, ctypes.byref(st)))
        return st

    def debug_gather(self, layer: int, tok0: int, n_tok: int, k_out: torch.Tensor, v_out: torch.Tensor,
                     stream=None):
        _check(lib().kvs_debug_gather(self._h, layer, tok0, n_tok, _ptr(k_out), _ptr(v_out), _stream(stream)))

    def profile_enable(self, on: bool = True):
        _check(lib().kvs_profile_enable(self._h, 1 if on else 0))

    def profile_read(self, kind: int, reset: bool = True):
        """(launches, total_ms) of attention (kind 0) or combine (kind 1) kernels."""
        n, ms = ctypes.c_int64(0), ctypes.c_double(0.0)
        _check(lib().kvs_profile_read(self._h, kind, ctypes.byref(n), ctypes.byref(ms), 1 if reset else 0))
        return n.value, ms.value

    def pin_layer(self, layer: int, n_slots: int):
        """Reserve a pinned region of n_slots slots for one layer (kvs_pool_pin_layer)."""
        _check(lib().kvs_pool_pin_layer(self._h, layer, n_slots))

    def reset_pinned(self):
        """Return every pinned region to the pool (kvs_pool_reset_pinned)."""
        _check(lib().kvs_pool_reset_pinned(self._h))

    def debug_export_pages(self, layer: int, dst: torch.Tensor, stream=None):
        """Raw page records as the kernels read them, into dst (uint8, device,
        [n_pages, page_bytes]) (kvs_debug_export_pages)."""
        assert dst.is_cuda and dst.dtype == torch.uint8 and dst.is_contiguous()
        _check(lib().kvs_debug_export_pages(self._h, layer, _ptr(dst), _stream(stream)))

    def debug_stage(self, layer: int, n_kv: int, dst: torch.Tensor, stream=None):
        """Staged matrix-core operands of every page (kvs_debug_stage) into dst
        (uint8, device, [n_pages, n_kv_heads, STAGED_TILE_BYTES])."""
        assert dst.is_cuda and dst.dtype == torch.uint8 and dst.is_contiguous()
        _check(lib().kvs_debug_stage(self._h, layer, n_kv, _ptr(dst), _stream(stream)))

    def debug_read_page(self, layer: int, page: int):
        import numpy as np
        buf = np.empty(page_bytes(self.cfg), dtype=np.uint8)
        _check(lib().kvs_debug_read_page(self._h, layer, page, buf.ctypes.data_as(ctypes.c_void_p)))
        return buf
