"""CPU oracle for the fused TP GEMM + reduction -- test infrastructure only.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path never does.
"""
