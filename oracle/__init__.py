"""Plain CPU oracle for the NVFP4 block-scaled GEMM.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.
"""
