"""CPU oracle for the CSA2 layer step -- test infrastructure only.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product (the HIP library and its Python binding) never
imports, links or runs anything here, and this package shares no code with it.
"""
