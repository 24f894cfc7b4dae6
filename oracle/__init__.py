"""CPU oracle for Kronecker Product Attention (KPA) factor-cache decode.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link
or execute anything in this package: only the test-suite, the smoke check and
the CPU-baseline leg of the benchmark use it.  It shares no code, header,
table or constant generator with the HIP implementation.

Two implementations of the same definition, both in float64:

* ``kpa_ref``     -- the definitions written out literally with NumPy
                     (``np.kron`` for the Kronecker product, explicit rotation
                     matrices, textbook softmax).  Small shapes only.
* ``kpa_oracle``  -- a plain C version (``kpa_oracle.c``) of the same
                     definition, streamed one cached token at a time so that a
                     2^19-token context never materialises full K/V.  Used for
                     the full-size sampled parity checks and timed as the CPU
                     baseline.  It is itself checked against ``kpa_ref``.

Sources (cited by page title and section/equation):
  [KPA]  "Kronecker Product Attention: Memory-Efficient KV Compression via
         Structured Factorization" (arXiv 2610.12657).
  [TPA]  "Tensor Product Attention Is All You Need" (arXiv 2501.06425), as
         rendered and as summarised on the architecture-summary page.
"""
