"""ReTopK decode-step attention on MI355X (gfx950).

The compute path is the HIP library ``libretopk.so`` (C ABI in
``include/retopk.h``); ``binding`` is its thin Python binding and
``workload`` draws the seeded synthetic inputs.
"""
__all__ = ["binding", "workload"]
