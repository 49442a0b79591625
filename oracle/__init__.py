"""CPU oracle (test infrastructure only: tests, the smoke check and the benchmark's
CPU-baseline leg use it; the product path never imports it)."""
