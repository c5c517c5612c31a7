"""fp64 CPU oracle for paged-KV attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product path (the HIP library
and its Python binding) never imports, calls or links it, and shares no code
with it: the only code both sides use is the seeded input generator in
``workloads``.

Pins (what fixes each function to something other than itself) are listed in
the headers of ``oracle/attention.py``, ``oracle/kv_append.py``,
``oracle/fp8.py`` and ``oracle/prefix_groups.py``; every
function is pinned, none is "parity unpinned".
"""

from .attention import (  # noqa: F401
    stored_to_f64,
    gather_rows,
    attend,
    lse_merge,
    paged_attention,
    decode,
    decode_multi_window,
    decode_window,
    prefix_cascade,
    mixed_chunk,
    check_block_tables,
)
from .kv_append import kv_append  # noqa: F401
from .fp8 import (  # noqa: F401
    decode_fp8,
    decode_multi_fp8,
    dequantize,
    e4m3_to_f64,
    kv_append_fp8,
    mixed_chunk_fp8,
    prefix_cascade_fp8,
    quantize_rows,
)
from .prefix_groups import detect_prefix_groups  # noqa: F401
