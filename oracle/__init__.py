"""CPU oracle for the LongFlow fused decode step.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and its
Python binding) imports, calls or links anything here; only the tests, the
smoke check and the benchmark's CPU-baseline leg do. The oracle shares no code
with the HIP path: not a kernel, header, helper, table or constant generator.
Both sides consume the same seeded inputs from the input-generator module,
which holds none of the method's arithmetic.

Modules:
  longflow_oracle  the step as the pages define it, in float64 (NumPy), with
                   the variants (l2 score, deferred order, one victim per
                   sequence) as options
"""
