"""CPU oracle for SAGE's 2.25-bit spherical vector quantisation (TEST INFRASTRUCTURE ONLY).

Source: "SAGE: Pushing 2-Bit Vector-Quantized LLMs toward Real-World Usability" (called "the SAGE
paper" below), §3.1-§3.3 and Appendix A.6/A.7.

This package is the slow, obviously-correct reference that the HIP path is checked against. It is
plain NumPy in float64, written step by step from the paper's equations, and it shares no code,
constant tables or helpers with the GPU library. Only the test suite, the smoke check in
``__graft_entry__`` and the benchmark's ``cpu_baseline`` leg may import it; the product path never
calls it and has no CPU fallback.

Modules
  encoder  channel energies, ESG permutation, position weights, Eq. (6) assignment, weighted
           spherical k-means, radius grid, whole-matrix encoding and the ABS score/selection.
  decoder  decode of the stored fields to weights (float64 and RNE fp16), and the float64
           matrix-vector / matrix-matrix / grouped-expert products, plus the output tolerance.
  budget   bit-budget and storage-cost identities (Eq. (3), Eq. (15)).
  packing  our packed storage layout, written from its format description, for bit-exact checks.

Parity status per function is listed in each module's header.
"""
