"""LongSpark fixed-cost drafting path on MI355X (gfx950).

The compute lives in ``liblongspark.so`` (hand-written HIP kernels behind a C
ABI, declared in ``include/longspark.h``).  ``fixed_cost_drafter_amd.binding``
loads it and marshals arguments; importing this package alone loads nothing.
"""
__all__ = ["binding", "workload"]
