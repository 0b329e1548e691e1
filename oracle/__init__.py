"""fp64 CPU oracle for the NVFP4 MoE path. TEST INFRASTRUCTURE: only the tests, the smoke check
and the benchmark's CPU-baseline leg may import it; the HIP product path never does."""
