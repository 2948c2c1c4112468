"""ReplaySSM decode hot path for AMD MI355X (gfx950).

The library is ``librss.so`` (C ABI in ``include/rss.h``, HIP kernels in
``csrc/``); ``recurrent_state_storage_amd.rss`` is its thin ctypes binding.
Importing this package loads nothing; the first library call loads
``librss.so`` and raises if it has not been built.
"""
__all__ = ["rss"]
