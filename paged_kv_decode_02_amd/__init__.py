"""Paged-KV attention for AMD Instinct MI355X (gfx950).

The compute lives in ``libpa.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/pa.h``); :mod:`paged_kv_decode_02_amd.pa` is its thin
ctypes binding and :mod:`paged_kv_decode_02_amd.build` compiles it in-tree.
Importing the package loads nothing; the first call into ``pa`` loads the
library and raises if it has not been built.
"""

__all__ = ["pa", "build", "roofline"]
