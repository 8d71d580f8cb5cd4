"""CPU oracle of the batch-1 decode step and of the GEMV-tanh chain.

TEST INFRASTRUCTURE: a plain, slow float64 reference written from the pages
("7 - AMD et le monokernel", "8 - Ecrire son megakernel").  Only the tests, the
smoke check and the benchmark's CPU-baseline leg may import it; the product
path never does.  It shares no code with the HIP path.

Modules:
  decoder  KV-cached decoder (prefill by layer-major matrix products, decode by
           matrix-vector products), greedy and teacher-forced drivers.
  brute    independent full-recompute forward (no KV cache, complex-number RoPE,
           masked score matrix) used to pin ``decoder``.
  chain    the GEMV-tanh chain microbenchmark.
"""
