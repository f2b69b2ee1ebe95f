"""CPU oracle for the tiled dense GEMM (test infrastructure only).

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg;
never by the GPU library.
"""
