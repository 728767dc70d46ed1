"""Seeded synthetic inputs for the streamed paged attention library and its oracle.

This module is the one piece of Python that both sides use. It draws the
random numbers, encodes them into the Q8_0 / Q4_0 page records that the
library consumes, and picks the residency pattern. It holds none of the
arithmetic that the library computes: no dequantization, no scores, no
softmax. The oracle decodes the bytes produced here with its own code, and
the library decodes them with its own kernels.

Sources: the three pages collected on host-streamed paged KV (the
"Adaptive KV Streaming" llama.cpp forks). Page 1 ("Summary", "What it is
useful for") names the Q8_0 K / Q4_0 V cache; page 2 ("Dynamic draft eject")
fixes the 256-token page; page 3 ("Diagnostic log") fixes the 10 % residency,
rounded up to whole pages.
"""

from .configs import WORKLOADS, Workload, workload  # noqa: F401
from .gen import (  # noqa: F401
    KVGeometry,
    layer_records,
    make_q,
    residency_mask,
    quantize_q8_0,
    quantize_q4_0,
    pack_page_records,
    poison_tail,
    rng_for,
)
