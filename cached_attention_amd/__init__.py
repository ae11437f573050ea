"""FlashBlock cached block-external attention for MI355X (gfx950).

The computation lives in the HIP library ``libflashblock.so`` behind the C ABI
declared in ``include/flashblock.h``; ``cached_attention_amd.flashblock`` is a
thin ctypes binding to it (argument marshalling only).  Importing this package
does not load the library; the binding loads it on first use and raises if it
has not been built.
"""
__all__ = ["workloads", "flashblock"]
