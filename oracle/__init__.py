"""CPU oracle for the fully-connected layer on GGUF Q4_K / Q5_K / Q6_K blocks.

TEST INFRASTRUCTURE ONLY.  Plain, slow, obviously correct NumPy code in
float64 (integer sums in int64), written from the method's description and
sharing nothing with the HIP path.  Only the test-suite, the smoke check of
the graft entry point and the CPU-baseline leg of the benchmark may import
it; the library's product path never does.

Modules
  kquant  block formats: decode to exact float64 weights, the Q6_K plane
          regroup and its inverse, and encoders for hand-built blocks.
  fc      Y = A.W^T (+R) in float64, the int8 activation quantisation, the
          integer sub-block dot sums, the exact emulation of the int8 decode
          path, and the MoE per-pair reference.

Every function is pinned by a `-m "not gpu"` test against closed forms,
invariants, exact rational arithmetic or brute force (see tests/test_oracle_*).
Compatibility of the bit layout with real GGUF files is parity unpinned:
no GGUF file or GGUF reader is available to compare against.
"""

from . import kquant, fc  # noqa: F401
