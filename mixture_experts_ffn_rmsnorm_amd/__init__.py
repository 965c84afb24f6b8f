"""Routed mixture-of-experts FFN layer with RMSNorm for AMD MI355X (gfx950).

The compute path lives in the HIP shared library ``libmoeffn.so`` behind the
C ABI declared in ``include/moe_ffn.h``; ``moe`` is its thin Python binding.
Importing this package loads nothing; ``moe`` loads the library on first use
and raises if it is missing.
"""

__all__ = ["inputs", "moe"]
