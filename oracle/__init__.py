"""fp64 CPU oracle of the Gated DeltaNet layer: test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The HIP library never does.
"""
