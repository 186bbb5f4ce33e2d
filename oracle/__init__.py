"""CPU oracle for the DCNv4 spatial-aggregation forward.

TEST INFRASTRUCTURE ONLY: the checker, not the product.  Only the test suite,
the smoke check and the benchmark's CPU-baseline leg may import this package.
It shares no code with the HIP library and never imports it.
"""
