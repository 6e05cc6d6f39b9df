"""fp64 CPU oracle of the selective-recompute prefill layer.

Test infrastructure only: used by the tests, the package smoke check and the CPU
baseline of the benchmark, never by the product path."""
