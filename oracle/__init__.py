"""CPU oracle for the packed ternary-code matmul.

TEST INFRASTRUCTURE ONLY.  This package is imported by the tests, by the
smoke check and by the CPU-baseline leg of the benchmark, and by nothing else.
The HIP library never calls it, and it never calls the HIP library: the two
share no code, headers or tables.

Everything here is plain, slow and written to be checked by eye against the
pages it follows:

* "Does your weight format deserve a kernel?" (precisit.com, pack-unpack-run):
  the mean-abs ternary quantizer ("Three values and a shared scale"), the
  five-trits-per-byte packing ("Five trits in a byte") and the byte count
  ("Count the bytes you actually wrote").
* "A Discrete Weight Language for Large Language Models: Compressing Gemma 4
  31B with a 5-Step Ternary Route" (Route B): the 243-word code book (section
  3.2), the per-row scale (section 3.3), the fused LUT matmul semantics
  (section 4.2), per-head scales (section 8.2), the 7-bit truncated alphabet
  (section 8.1) and per-block code books (section 8.3).
* "FUCINA - a general ternary forge for Mixture-of-Experts models": the
  two-plane sum W ~ d1*T1 + d2*T2 ("The method") and the expert matmul.

Floating point is fp64 unless the pages fix a precision (fp16 group scales,
bf16 activations and reconstructions, fp32 code-book entries).

Parity status: every function is pinned by ``tests/test_oracle_pins.py``
against worked examples, closed forms, exact rational arithmetic or brute
force.  No function is "parity unpinned".
"""

from .fpround import (
    f64_to_f16_bits,
    f16_bits_to_f64,
    f64_to_bf16_bits,
    bf16_bits_to_f64,
    f64_to_f32,
)
from .ternary import (
    OracleDataError,
    bytes_per_group,
    bits_per_weight,
    quantize,
    pack,
    unpack,
    quantize_pack,
    two_plane,
)
from .routeb import (
    code_words,
    rb_block_scales,
    rb_encode,
    rb_table,
    rb_weights,
    rb_truncate,
    pack7,
    unpack7,
    rb_weights7,
)
from .matmul import (
    REL_BOUND,
    matmul_ref,
    ternary_weights,
    grouped_ref,
    hot_prefix_weights,
    check_bound,
)

__all__ = [
    "f64_to_f16_bits", "f16_bits_to_f64", "f64_to_bf16_bits", "bf16_bits_to_f64", "f64_to_f32",
    "OracleDataError", "bytes_per_group", "bits_per_weight", "quantize", "pack",
    "unpack", "quantize_pack", "two_plane",
    "code_words", "rb_block_scales", "rb_encode", "rb_table", "rb_weights",
    "rb_truncate", "pack7", "unpack7", "rb_weights7",
    "REL_BOUND", "matmul_ref", "ternary_weights", "grouped_ref", "hot_prefix_weights",
    "check_bound",
]
