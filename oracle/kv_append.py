"""Reference for KV append: this step's new K/V rows into the paged cache.

TEST INFRASTRUCTURE ONLY (see the package docstring): the tests, the smoke
check and the benchmark's CPU-baseline leg are its only callers.

What it computes
----------------
The cache model is the one the SwiftLLM page describes in section 3.1
("PagedAttention and KV cache management"): a sequence's K/V rows live in
fixed-size blocks named by its block table, blocks being handed out as the
sequence grows.  Before attention runs, the rows of the tokens that this
step adds must be in those blocks (the attention layer of SwiftLLM page
section 5.1 reads them through the tables).  The pages do not spell out the
write; the plain reading, used here, is the inverse of the oracle's row
lookup in ``attention.gather_rows``:

segment s adds ``n = q_lens[s]`` tokens and holds ``L = context_lens[s]``
rows counting them, so its new token i (0-based, token ``cu[s] + i`` of the
batch) is row ``pos = L - n + i``; for every kv-head g,

    k_pool[bt[s][pos // BS], g, pos % BS, :] = k_new[cu[s] + i, g, :]

and the same for V.  Values are copied bit for bit (no arithmetic).  A
table entry outside ``[0, num_pages)`` names no page: that row is not
written (the library's documented behaviour for tables it cannot check on
the fast path).  All other pool rows are left as they were.

Pins (tests/test_oracle_pins.py): an element-by-element brute force written
from the definition above; untouched rows keep their bits (NaN poison
included); appending twice changes nothing more; the appended rows read
back through the attention oracle's own lookup equal the new rows; a round
trip -- appending a whole sequence into an empty pool, then the attention
oracle over it -- equals dense attention over the sequence's rows; planted
off-by-one positions and swapped kv-heads are caught.
"""

from __future__ import annotations

import numpy as np


def kv_append(k_pool, v_pool, k_new, v_new, block_tables, context_lens, q_lens, block_size: int):
    """Copies of ``k_pool`` and ``v_pool`` with the new rows written.

    ``k_pool``, ``v_pool``: [NP, Hkv, BS, D] stored values (float32, or bf16
    bit patterns as uint16); ``k_new``, ``v_new``: [T, Hkv, D] of the same
    kind, T = sum(q_lens); ``block_tables``: [S, MB]; ``context_lens``,
    ``q_lens``: [S].
    """
    kp = np.array(k_pool, copy=True)
    vp = np.array(v_pool, copy=True)
    ctx = np.asarray(context_lens, dtype=np.int64)
    ql = np.asarray(q_lens, dtype=np.int64)
    bt = np.asarray(block_tables)
    num_pages = kp.shape[0]
    if k_new.shape[0] != int(ql.sum()) or v_new.shape[0] != k_new.shape[0]:
        raise ValueError("new rows do not match the query lengths")
    t0 = 0
    for s in range(len(ctx)):
        L, n = int(ctx[s]), int(ql[s])
        if n < 0 or n > L:
            raise ValueError(f"segment {s}: need 0 <= q_len <= context_len")
        if (L + block_size - 1) // block_size > bt.shape[1]:
            raise ValueError(f"segment {s}: context longer than its table")
        for i in range(n):
            pos = L - n + i
            page = int(bt[s, pos // block_size])
            if 0 <= page < num_pages:
                kp[page, :, pos % block_size, :] = k_new[t0 + i]
                vp[page, :, pos % block_size, :] = v_new[t0 + i]
        t0 += n
    return kp, vp
