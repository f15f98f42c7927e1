"""Oracle for the Hierarchical Sparse Attention (HSA) forward layer.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow CPU statement of
what the layer computes.  Only the test-suite, the package smoke check and the
benchmark's CPU-baseline leg may import it.  The product path (the HIP library
and its Python binding) never imports, calls or links anything in here, and
nothing in here imports the product path.

Modules
-------
hsa_oracle  numpy float64 implementation (landmarks, scores, top-k selection,
            in-chunk attention, fusion), plus the near-tie acceptance rule.
brute       pure-Python (math + fractions) restatement used on tiny inputs
            to pin ``hsa_oracle``.
"""
