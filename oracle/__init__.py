"""FP64 CPU oracle for LeapQuant decoding (test infrastructure only).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package. It shares no code with the HIP path.
"""
