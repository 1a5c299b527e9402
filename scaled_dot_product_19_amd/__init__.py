"""MI355X-native fused SDPA forward: THD ragged prefill and paged split-KV decode.

The compute path is the HIP library ``libsdpa.so`` (gfx950), reached through the
C-ABI declared in ``include/sdpa.h``; ``scaled_dot_product_19_amd.sdpa`` is its thin
ctypes binding.  Importing this package loads nothing; the first call into the
binding loads the library and raises if it is missing.
"""
