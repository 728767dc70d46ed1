"""The five synthetic workloads: shapes, residency counts and query recipes.

Each workload mirrors a shape the pages measure on:
  * 32 Ki and 256 Ki contexts, page 1 "What it is useful for";
  * 16 streamed attention layers, page 3 "Diagnostic log";
  * about 10 % of the context resident, page 3 "--kv-stream auto";
  * about 160 K context with about 180 resident pages per layer, page 2
    "Results" (streaming onset);
  * draft length 3, so 4 verify tokens, page 1 "How engineers can use it";
  * a 256-token ubatch, page 2 "TLDR".
"""

from dataclasses import dataclass
import math


@dataclass(frozen=True)
class Workload:
    cid: int                 # seed component identifying the workload
    name: str
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_kv: int                # tokens in each layer's cache
    n_q: int                 # query tokens per call
    q_dtype: str             # "f32" or "f16"
    scale: float             # softmax scale applied to q.k
    causal: bool
    q_pos0: int              # position of the first query token
    resident_pages: int      # resident pages per layer (all pages if >= n_pages)
    own_page_resident: bool  # prefill: the ubatch's own page is always resident
    page_tokens: int = 256

    @property
    def n_pages(self) -> int:
        return -(-self.n_kv // self.page_tokens)


def _ten_percent_pages(n_tokens: int, page_tokens: int = 256) -> int:
    # 10 % of the context, rounded up to whole pages (page 3, "Diagnostic log":
    # 6656 tokens at 65536, 26368 at 262144).
    return -(-math.ceil(0.1 * n_tokens) // page_tokens)


WORKLOADS = {
    "tiny_decode": Workload(
        cid=1, name="tiny_decode", n_layers=1, n_q_heads=1, n_kv_heads=1, head_dim=128,
        n_kv=1024, n_q=1, q_dtype="f32", scale=1.0, causal=False, q_pos0=1023,
        resident_pages=4, own_page_resident=False),
    "resident_decode_32k": Workload(
        cid=2, name="resident_decode_32k", n_layers=16, n_q_heads=24, n_kv_heads=4,
        head_dim=128, n_kv=32768, n_q=1, q_dtype="f32", scale=1.0, causal=False,
        q_pos0=32767, resident_pages=128, own_page_resident=False),
    "streamed_decode_256k": Workload(
        cid=3, name="streamed_decode_256k", n_layers=16, n_q_heads=24, n_kv_heads=4,
        head_dim=128, n_kv=262144, n_q=1, q_dtype="f32", scale=1.0, causal=False,
        q_pos0=262143, resident_pages=_ten_percent_pages(262144), own_page_resident=False),
    "spec_verify_160k": Workload(
        cid=4, name="spec_verify_160k", n_layers=16, n_q_heads=24, n_kv_heads=4,
        head_dim=128, n_kv=163840, n_q=4, q_dtype="f32", scale=1.0, causal=True,
        q_pos0=163836, resident_pages=180, own_page_resident=False),
    "prefill_ubatch_128k": Workload(
        cid=5, name="prefill_ubatch_128k", n_layers=16, n_q_heads=24, n_kv_heads=4,
        head_dim=128, n_kv=131072 + 256, n_q=256, q_dtype="f16",
        scale=1.0 / math.sqrt(128.0), causal=True, q_pos0=131072,
        resident_pages=_ten_percent_pages(131072), own_page_resident=True),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]
