"""Selective-recompute prefill ("KV cache fusor") for AMD MI355X (gfx950).

The layer runs in hand-written HIP kernels behind the C ABI of libsrp.so
(include/srp.h); this package holds the ctypes binding, the build step and the
seeded synthetic workload generator."""
__all__ = ["inputs"]
