"""CPU oracle for the Load-as-Sparse, Compute-as-Dense sparse x skinny product.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls, links or
runs anything in this package: only the test suite, the smoke check in
`__graft_entry__.smoke()` and the CPU-baseline leg of `bench.py` may use it.
It shares no code, table or helper with the HIP library; the only thing both
sides take in common are the seeded inputs of `lscd_synth`.

What it computes, from the Flash-LLM pages:

* `tiled_csl` -- the Tiled-CSL sparse format (Flash-LLM paper review, xllm-io,
  section 3 "Tiled-CSL sparse encoding format"): the weight matrix is cut into
  tiles, each nonzero becomes one 32-bit word holding its fp16 value and its
  16-bit position inside the tile, the words are stored tile after tile and a
  per-tile offset array locates each tile.  `encode_canonical` builds the
  format with the nonzeros of a tile in ascending position order; `decode`
  turns any valid encoding back into the dense matrix and rejects invalid ones.
* `spmm` -- the product itself.  Load-as-Sparse / Compute-as-Dense changes how
  the weights are moved, not what is computed (same review, section 2
  "solution" and section 3 "core formulas": C = A x B with the sparse A
  decoded to dense); so the oracle is the plain definition
  C[n][i] = sum_k A[i][k] * B[n][k], accumulated in fp64.
* `bitmap` -- the bitmap-tile variant of the format (the pages' follow-up summary,
  section "Problematica": one bit per position instead of per-entry positions): per
  tile, 64 lane masks whose bits follow the matrix-core operand layout, then the kept
  values chunk by chunk.
* `loop` -- the same decode and product written again as plain C loops
  (`spmm_loop.c`: the fp64 triple loop with k ascending, OpenMP over rows), pinned
  to the modules above and timed as the CPU baseline.
* `accounting` -- the compute-intensity formula and the byte/flop counts used
  for effective bandwidth (same review, section 3 "core formulas").

Readings of points the pages leave open (bit order of a word, offset units,
padding, output rounding) are stated in the module that takes them.
"""
from . import accounting, bitmap, loop, spmm, tiled_csl  # noqa: F401
