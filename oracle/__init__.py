"""fp64 CPU oracle for the MoE layer with zero-computation experts.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import it; the product package never does.
"""
