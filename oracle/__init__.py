"""CPU oracle for the contextual-sparsity decode step -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (the HIP
library and its Python binding) never does, and the two share no code: only
the seeded input generators are common to both.

``ref``   -- the decode step in float64 NumPy, one function per step.
``bytes`` -- the byte account of a decode step, crossover and ideal speedups.

Pages cited (by title, then section / equation / table):
  DejaVu    = "Deja Vu: Contextual Sparsity for Efficient LLMs at Inference Time"
              (arXiv 2310.17157, the paper's own text).
  Explainer = the paper-graph explainer page of the same paper.
  ByteCross = "Where Activation Sparsity and KV-Cache Sparsity Cross in LLM
              Decoding" (arXiv 2609.33889v1, source-linked summary page).

Every function is pinned by a ``-m "not gpu"`` test against something other
than itself (see ``tests/test_oracle_pins.py`` and ``tests/test_bytes_pins.py``).
"""
