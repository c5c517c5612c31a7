"""fp64 reference for attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring): the tests, the smoke
check and the benchmark's CPU-baseline leg are its only callers.

What it computes
----------------
The cache model is PagedAttention as the SwiftLLM page describes it (section
3.1, "PagedAttention and KV cache management"): K and V live in fixed-size
blocks; a sequence's rows are found through its block table; blocks of a
shared prefix may be named by many tables.  The attention layer receives the
per-sequence block tables and context lengths (SwiftLLM page, section 5.1).
The pages do not print the attention formula itself; this oracle uses the
textbook definition.  For a sequence s with ``L`` rows in the pool and
``n`` query tokens this step, query token i of q-head h:

1. uses kv-head ``g = h // G`` (G = Hq / Hkv, contiguous head groups);
2. sees rows ``t < vis = L - n + i + 1`` (decode: n = 1, vis = L; a prefill
   chunk is causal inside itself, per the TokenSpeed deep-dive section 5.1
   chunked admission and the SwiftLLM page section 3.3 piggybacking);
3. row t lives at page ``bt[s][t // BS]``, slot ``t % BS``;
4. ``x_t = scale * <q, k_t>``; ``m = max x_t``; ``w_t = exp(x_t - m)``;
   ``out = sum w_t v_t / sum w_t``; ``lse = m + ln(sum w_t)`` (natural log).

Stored inputs are widened exactly to float64 (bf16 bit patterns or float32),
and ``scale`` is taken as the float32 value the GPU is handed.

The split-KV partials and their log-sum-exp merge (TokenSpeed deep-dive,
section 7 and 7.1: partial output plus LSE per split, reduced by a second
pass) are provided as :func:`attend` + :func:`lse_merge`; cascade /
Hydragen attention (Tokasaurus page, "dynamic prefix identification")
has the same definition as plain decode over the full table.

Pins (tests/test_oracle_pins.py):
* brute force: pure-Python loops over dense per-sequence K/V that the test
  itself scatters into pages (independent gather and arithmetic);
* closed forms: two-key softmax with weights 1/4, 3/4; one-row context
  returns its V row; constant V returns the constant; q = 0 returns the mean
  of the visible rows; lse of equal scores is ln(n);
* library routine: prefix-free causal chunk against
  ``torch.nn.functional.scaled_dot_product_attention`` in float64 on CPU;
* invariants: page relabelling, split/merge = unsplit, cascade = decode,
  GQA with G=1 equals per-head MHA, chunk decode rows equal decode;
* planted mistakes (a dropped scale, an off-by-one in visibility, a wrong
  kv-head mapping, a wrong lse log base) are each caught by one of the above.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np


def stored_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored values exactly to float64.

    ``dtype == "bf16"``: ``a`` holds bfloat16 bit patterns (uint16); a bf16
    value is the float32 whose upper 16 bits are those bits.
    ``dtype == "f32"``: ``a`` holds float32 values.
    """
    if dtype == "bf16":
        u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def gather_rows(pool, table_row, kv_head: int, n_rows: int, block_size: int, dtype: str):
    """Rows 0..n_rows-1 of one sequence's kv-head, found through its table.

    Row t is slot ``t % block_size`` of physical page ``table_row[t // block_size]``.
    """
    t = np.arange(n_rows)
    pages = np.asarray(table_row)[t // block_size]
    if n_rows and (pages.min() < 0 or pages.max() >= pool.shape[0]):
        raise IndexError("block table names a page outside the pool")
    slots = t % block_size
    return stored_to_f64(pool[pages, kv_head, slots, :], dtype)


def attend(qvec: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Softmax attention of one query over rows K, V (float64).

    Returns (out[D], lse) with lse in natural log.  An empty row set has no
    softmax; it returns (zeros, -inf), the identity of :func:`lse_merge`.
    """
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64), -math.inf
    x = float(scale) * (K @ qvec)
    m = float(np.max(x))
    w = np.exp(x - m)
    z = float(np.sum(w))
    return (w @ V) / z, m + math.log(z)


def lse_merge(parts: Sequence):
    """Combine (out_i, lse_i) partial results over disjoint row sets.

    With ``M = max lse_i`` over parts that saw rows, weights
    ``a_i = exp(lse_i - M)`` give ``out = sum a_i out_i / sum a_i`` and
    ``lse = M + ln(sum a_i)``.  Parts with lse = -inf (no rows) carry weight 0.
    """
    live = [(o, l) for o, l in parts if l != -math.inf]
    if not live:
        o0 = parts[0][0]
        return np.zeros_like(o0), -math.inf
    M = max(l for _, l in live)
    a = [math.exp(l - M) for _, l in live]
    den = sum(a)
    out = sum(ai * o for ai, (o, _) in zip(a, live)) / den
    return out, M + math.log(den)


def _widen_q(q, dtype):
    return stored_to_f64(q, dtype)


def paged_attention(
    q,
    k_pool,
    v_pool,
    block_tables,
    context_lens,
    q_lens,
    scale: float,
    num_kv_heads: int,
    block_size: int,
    dtype: str,
    seqs: Optional[Sequence[int]] = None,
):
    """General case: sequence s has ``q_lens[s]`` query tokens, the last
    ``q_lens[s]`` of its ``context_lens[s]`` pool rows.

    ``q``: [T, Hq, D] stored values, T = sum(q_lens).  Returns
    ``out`` [T, Hq, D] float64 and ``lse`` [T, Hq] float64.  If ``seqs`` is
    given only those sequences are computed (other rows stay NaN).
    """
    ctx = np.asarray(context_lens, dtype=np.int64)
    ql = np.asarray(q_lens, dtype=np.int64)
    T, Hq, D = q.shape
    if int(ql.sum()) != T:
        raise ValueError("q has the wrong number of tokens")
    if Hq % num_kv_heads:
        raise ValueError("q heads must be a multiple of kv heads")
    G = Hq // num_kv_heads
    sc = float(np.float32(scale))
    out = np.full((T, Hq, D), np.nan, dtype=np.float64)
    lse = np.full((T, Hq), np.nan, dtype=np.float64)
    starts = np.concatenate([[0], np.cumsum(ql)])
    todo = range(len(ctx)) if seqs is None else seqs
    for s in todo:
        L, n = int(ctx[s]), int(ql[s])
        if L < 1 or n < 1 or n > L:
            raise ValueError(f"sequence {s}: need 1 <= q_len <= context_len")
        qs = _widen_q(q[starts[s] : starts[s] + n], dtype)  # [n, Hq, D]
        for g in range(num_kv_heads):
            K = gather_rows(k_pool, block_tables[s], g, L, block_size, dtype)
            V = gather_rows(v_pool, block_tables[s], g, L, block_size, dtype)
            for i in range(n):
                vis = L - n + i + 1
                for h in range(g * G, (g + 1) * G):
                    o, l = attend(qs[i, h], K[:vis], V[:vis], sc)
                    out[starts[s] + i, h] = o
                    lse[starts[s] + i, h] = l
    return out, lse


def decode(q, k_pool, v_pool, block_tables, context_lens, scale, num_kv_heads, block_size, dtype, seqs=None):
    """One query token per sequence attending to all its ``context_lens[s]`` rows."""
    ones = np.ones(len(context_lens), dtype=np.int64)
    return paged_attention(
        q, k_pool, v_pool, block_tables, context_lens, ones, scale, num_kv_heads, block_size, dtype, seqs
    )


def decode_window(q, k_pool, v_pool, block_tables, context_lens, window, scale, num_kv_heads, block_size, dtype,
                  seqs=None):
    """Decode with a sliding window of ``window`` tokens: the query of a
    sequence with L rows sees rows ``[max(0, L - window), L)`` only.

    A sliding-window KV group declares its window size in tokens
    (``sliding_window_tokens``, TokenSpeed deep-dive section 4.1, the
    attention kinds table); its block table keeps the real blocks at the
    back and placeholder entries at the front for the blocks that fell out
    of the window (tokenspeed 딥다이브 section 6-3).  So only table entries
    from ``(L - window) // block_size`` on are looked up here: a placeholder
    is never read.
    """
    ctx = np.asarray(context_lens, dtype=np.int64)
    S, Hq, D = q.shape
    if S != len(ctx):
        raise ValueError("q must hold one token per sequence")
    if int(window) < 1:
        raise ValueError("window must be >= 1")
    G = Hq // num_kv_heads
    sc = float(np.float32(scale))
    out = np.full((S, Hq, D), np.nan, dtype=np.float64)
    lse = np.full((S, Hq), np.nan, dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        L = int(ctx[s])
        if L < 1:
            raise ValueError(f"sequence {s}: empty context")
        lo = max(0, L - int(window))
        t = np.arange(lo, L)
        pages = np.asarray(block_tables[s])[t // block_size]
        if pages.min() < 0 or pages.max() >= k_pool.shape[0]:
            raise IndexError("block table names a page outside the pool")
        qs = stored_to_f64(q[s], dtype)
        for g in range(num_kv_heads):
            K = stored_to_f64(k_pool[pages, g, t % block_size, :], dtype)
            V = stored_to_f64(v_pool[pages, g, t % block_size, :], dtype)
            for h in range(g * G, (g + 1) * G):
                out[s, h], lse[s, h] = attend(qs[h], K, V, sc)
    return out, lse


def decode_multi_window(q, k_pool, v_pool, block_tables, context_lens, q_len, window, scale, num_kv_heads,
                        block_size, dtype, seqs=None):
    """Multi-token decode over a sliding-window cache: sequence s brings its
    last ``q_len`` rows as new tokens; token i sits at position
    ``p = L - q_len + i`` and sees the rows ``[max(0, p + 1 - window), p]``:
    the causal rule of a multi-token step (each token sees the rows up to its
    own position; TokenSpeed deep-dive section 7.2 folds such tokens into
    one tile) with each token's own window of ``window`` tokens (TokenSpeed
    deep-dive section 4.1, ``sliding_window_tokens``).

    Token i of sequence s is row ``s * q_len + i`` of ``q`` / ``out``.
    Table entries before the earliest token's window,
    ``(L - q_len + 1 - window) // block_size``, may be placeholders
    (tokenspeed 딥다이브 section 6-3) and are never looked up.
    """
    ctx = np.asarray(context_lens, dtype=np.int64)
    n = int(q_len)
    W = int(window)
    T, Hq, D = q.shape
    if n < 1 or T != len(ctx) * n:
        raise ValueError("q must hold q_len tokens per sequence")
    if W < 1:
        raise ValueError("window must be >= 1")
    G = Hq // num_kv_heads
    sc = float(np.float32(scale))
    out = np.full((T, Hq, D), np.nan, dtype=np.float64)
    lse = np.full((T, Hq), np.nan, dtype=np.float64)
    for s in (range(len(ctx)) if seqs is None else seqs):
        L = int(ctx[s])
        if L < n:
            raise ValueError(f"sequence {s}: context shorter than q_len")
        lo0 = max(0, L - n + 1 - W)  # the earliest row any of the tokens sees
        t = np.arange(lo0, L)
        pages = np.asarray(block_tables[s])[t // block_size]
        if pages.min() < 0 or pages.max() >= k_pool.shape[0]:
            raise IndexError("block table names a page outside the pool")
        qs = stored_to_f64(q[s * n : (s + 1) * n], dtype)  # [n, Hq, D]
        for g in range(num_kv_heads):
            K = stored_to_f64(k_pool[pages, g, t % block_size, :], dtype)
            V = stored_to_f64(v_pool[pages, g, t % block_size, :], dtype)
            for i in range(n):
                p = L - n + i
                a, b = max(0, p + 1 - W) - lo0, p + 1 - lo0  # rows [a, b) of K, V
                for h in range(g * G, (g + 1) * G):
                    out[s * n + i, h], lse[s * n + i, h] = attend(qs[i, h], K[a:b], V[a:b], sc)
    return out, lse


def check_block_tables(
    block_tables,
    context_lens,
    num_pages: int,
    block_size: int,
    group_seq_offsets=None,
    prefix_lens=None,
):
    """Validate a batch's tables; returns a list of problems (empty = valid).

    Each sequence needs ``ceil(L/BS)`` in-range entries.  A physical page may
    be named by several tables only as part of a declared shared prefix: the
    first ``prefix_len / BS`` entries of every member of a group must be the
    same pages, and every other entry must be named exactly once.
    """
    problems = []
    bt = np.asarray(block_tables)
    ctx = np.asarray(context_lens)
    owner = {}
    prefix_pages_of = {}
    if group_seq_offsets is not None:
        offs = np.asarray(group_seq_offsets)
        for gi in range(len(offs) - 1):
            P = int(prefix_lens[gi])
            if P % block_size:
                problems.append(f"group {gi}: prefix length not a whole number of pages")
                continue
            npp = P // block_size
            ref = bt[offs[gi], :npp]
            for s in range(offs[gi], offs[gi + 1]):
                if P >= ctx[s]:
                    problems.append(f"group {gi}: prefix not shorter than sequence {s}")
                if not np.array_equal(bt[s, :npp], ref):
                    problems.append(f"group {gi}: sequence {s} does not share the prefix pages")
                prefix_pages_of[s] = npp
            for p in ref:
                owner[int(p)] = ("group", gi)
    for s in range(len(ctx)):
        L = int(ctx[s])
        n = (L + block_size - 1) // block_size
        if L < 1:
            problems.append(f"sequence {s}: empty context")
            continue
        if n > bt.shape[1]:
            problems.append(f"sequence {s}: table too short")
            continue
        for j in range(prefix_pages_of.get(s, 0), n):
            p = int(bt[s, j])
            if p < 0 or p >= num_pages:
                problems.append(f"sequence {s}: entry {j} out of range")
            elif p in owner:
                problems.append(f"sequence {s}: page {p} also used elsewhere")
            else:
                owner[p] = ("seq", s)
    return problems


def prefix_cascade(
    q,
    k_pool,
    v_pool,
    block_tables,
    context_lens,
    scale,
    num_kv_heads,
    block_size,
    dtype,
    group_seq_offsets,
    prefix_lens,
    seqs=None,
):
    """Shared-prefix (cascade / Hydragen) decode.

    The result is defined to be full attention over prefix + suffix, i.e.
    plain decode over each member's whole table (Tokasaurus page, "dynamic
    prefix identification"; the shared blocks of SwiftLLM page section 3.1).
    The group structure is checked first.
    """
    probs = check_block_tables(
        block_tables, context_lens, k_pool.shape[0], block_size, group_seq_offsets, prefix_lens
    )
    if probs:
        raise ValueError("; ".join(probs[:5]))
    return decode(q, k_pool, v_pool, block_tables, context_lens, scale, num_kv_heads, block_size, dtype, seqs)


def mixed_chunk(q, k_pool, v_pool, block_tables, context_lens, q_lens, scale, num_kv_heads, block_size, dtype, seqs=None):
    """Prefill chunks and decode tokens in one batch (SwiftLLM page section
    3.3, piggybacking): segment s's token i sees rows ``[0, L - n + i]``."""
    return paged_attention(
        q, k_pool, v_pool, block_tables, context_lens, q_lens, scale, num_kv_heads, block_size, dtype, seqs
    )
