"""MI355X-native load-balanced paged decode attention.

Three hand-written HIP kernels for gfx950 behind a C ABI (``include/lbsa.h``):
an assign kernel that builds the per-step task map, a persistent split kernel
that drains each workgroup's bin into partial outputs with their log-sum-exp,
and a combine kernel that merges them into bf16 output.  ``lbsa`` is the thin
ctypes binding; ``workload`` makes seeded synthetic batches.
"""
__all__ = ["lbsa", "workload"]
