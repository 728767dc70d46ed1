"""CPU oracle for streamed paged attention over a Q8_0-K / Q4_0-V cache.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports or calls this
package. Only the test suite, the smoke check in the graft entry module and the
`cpu_baseline` leg of bench.py may use it.

The oracle is plain float64 numpy. It shares no code with the HIP path and
never consults residency, rings or page tables. Streaming only moves bytes
(page 3, "KLD": the streamed and resident runs do the same math), so the oracle
computes ordinary softmax attention over the dequantized cache, read straight
from the host page records.

Parity status of each function (how it is pinned, in tests/test_oracle_*.py):
  f16_to_f64       pinned: all 65536 encodings against numpy's binary16 decode.
  dequant_q8_0     pinned: hand-built blocks with closed-form values; round trip.
  dequant_q4_0     pinned: hand-built blocks (nibble order, bias); round trip.
  gather_kv        pinned: hand-placed sentinel blocks at known (page, head, row).
  page_bytes       pinned: sizes printed on page 3 ("Diagnostic log").
  attend           pinned: mpmath brute force on tiny inputs, closed forms
                   (single key, zero scale, dominant key, GQA constants,
                   causal prefix means, ragged tails), LSE split invariance.
  quantize_q8_0_block, quantize_q4_0_block
                   pinned: dequantize-then-quantize returns the block for
                   every block whose extreme code is +-127 (Q8_0) or nibble 0
                   (Q4_0); hand-worked blocks (half-way codes, ties on the
                   largest magnitude, zero blocks, both scale signs); the
                   error bound of each rule on random blocks.
  append_rows      pinned: rows land at (page, head, row) as gather_kv reads
                   them back; bytes outside the appended rows are unchanged.
"""

from .kvs_oracle import (  # noqa: F401
    QK,
    Q8_0_BYTES,
    Q4_0_BYTES,
    F16_BYTES,
    f16_to_f64,
    dequant_q8_0,
    dequant_q4_0,
    page_bytes,
    gather_kv,
    attend,
    attend_layer,
    quantize_q8_0_block,
    quantize_q4_0_block,
    append_rows,
)
