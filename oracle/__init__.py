"""CPU oracle for exact block-sparse masked ring attention (TEST INFRASTRUCTURE).

This package is the plain, slow, obviously-correct reference that the GPU path
is checked against.  It is test infrastructure only: it may be imported solely
by `tests/`, by `__graft_entry__.smoke()` and by the `cpu_baseline` leg of
`bench.py`.  The product library never imports, links or runs it, and it never
imports the product library; the two share nothing but the seeded input
generators in `workloads/`.

Contents (each function cites the passage of the pages it follows):
  mask       - the four-track mask predicate (MARBLE, section 01, mask code block)
  attention  - masked softmax attention in fp64 from its definition
               (ring-attention explainer, "The Long-Context Scaling Problem";
               Libra, section 2.2, Eq. 1), per sample
  ring       - the ring iteration with the unnormalized carried (m, l, O) state
               (ring-attention explainer, "Online Softmax Formulation" and
               "Execution Algorithm"; NumPy ring page, "The whole algorithm")
  backward   - the textbook gradients of masked softmax attention in fp64
  planner    - exact tile classification by enumeration, PTRR, per-step maps
               (MARBLE, section 03 "Block classification" and "PTRR")

Precision: fp64 unless a function says otherwise (the toy ring is fp32, as the
NumPy page runs it).

Parity pins: every function is pinned by a `-m "not gpu"` test against values
the pages print, closed forms, invariants or brute force; the pins are listed
in each module header.  Parity unpinned: none of the functions is unpinned; the
readings where the pages are silent (PTRR cost and tie order, the workload
recipes) are fixed readings, documented where they are implemented.
"""
