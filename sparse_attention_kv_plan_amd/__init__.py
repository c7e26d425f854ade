"""MI355X-native KV compressor: plan, write, c4/c128 compress and fused decode.

The compute path is the HIP library ``libkvc.so`` (built from ``csrc/``) behind
the C ABI declared in ``include/kvc.h``; ``kvc`` is its thin ctypes binding.
``workloads`` draws the seeded synthetic inputs.
"""
__all__ = ["kvc", "workloads"]
