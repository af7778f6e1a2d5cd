"""q4_dequant_gemv_amd -- fused Q4_K dequantize-and-multiply for MI355X (gfx950).

The compute lives in ``libq4k.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/q4k.h``).  ``q4_dequant_gemv_amd.q4k`` is the thin
Python binding: it turns torch tensors into pointers and the current HIP
stream, calls the library, and raises on any error status.  Import of this
package itself loads nothing.
"""

__all__ = ["inputs", "q4k"]
