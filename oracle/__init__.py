"""CPU oracle for the fused low-bit dequant-matmul path.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, calls or links
anything here; only the tests, the smoke check and the CPU-baseline leg of the
benchmark do.  The oracle shares no code with the GPU path: it has its own
bit-level packers and unpackers, its own bf16/fp16 handling and its own decode,
all in plain numpy with fp64 arithmetic.

Every decode below reaches its result exactly (decoded weights are exact in
fp64), so each function is the plain definition evaluated in fp64 and then a
library matrix product:

  lut6  - per-row LUT, 6-bit codes ("Qwen3.8-27B - BenQ 6-bit",
          "What BenQ stores": decode is the row-wise gather of the code into
          that row's 64-entry table; the table holds 32 negative levels in
          ascending order, then 32 positive).
  lut4  - the same with 4-bit codes and 16-entry tables (the 8-tier row of
          the card's "Why equal-width shells" placement table).
  fabq  - binary core with int4 rows, per-block scales and a residual
          codebook ("FABQ-RC" README "Key Ideas" and model card
          "How It Works" / "Quantization Details").
  mdbf  - multi-envelope double binary factorisation (OneCompression "MDBF",
          "Algorithm" and "Bit-width and rank").

Pins that tie each part to something other than itself live in
``tests/test_oracle_*.py``.  Parity status per function is stated in each
module header.
"""
from . import numerics, bits, lut6, lut4, fabq, mdbf, compare  # noqa: F401
