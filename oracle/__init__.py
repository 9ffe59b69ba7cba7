"""CPU oracle for MLA decode with weight absorption.

TEST INFRASTRUCTURE ONLY. This package is imported only by the test suite,
by the smoke check in the repository's graft entry module and by the CPU
baseline leg of bench.py. The product path (the HIP library and its Python
binding) never imports, calls or links anything here, and this package never
imports the product path. Only the seeded input generator is shared.

All arithmetic is float64 numpy; the only rounding is the one the method
itself performs when a new row is stored in the cache (to the storage dtype).
"""
from .mla_oracle import (  # noqa: F401
    bf16_round, store_round, rope, rms_norm, compress_row, query,
    attend_unabsorbed, out_proj, absorb_q, attend_absorbed, expand_out,
    decode_step, decode_step_absorbed,
)
