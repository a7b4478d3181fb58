"""MI355X-native paged KV decode attention.

The compute lives in ``libpagedattn.so`` (hand-written HIP for gfx950, C ABI
declared in ``include/pagedattn.h``).  ``ops`` is a thin ctypes binding that
passes torch tensors' device pointers and the current HIP stream; it loads the
library on first use and raises if it is missing.  ``inputs`` holds the
seeded synthetic workloads.
"""

__all__ = ["ops", "inputs"]
