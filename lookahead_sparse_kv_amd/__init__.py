"""OasisKV decode hot path for MI355X (gfx950).

The compute lives in the HIP library ``liboasis.so`` (built from ``csrc/``);
``ops`` is its thin ctypes binding.  ``workload`` draws the seeded synthetic
inputs.
"""
__all__ = ["ops", "workload"]
