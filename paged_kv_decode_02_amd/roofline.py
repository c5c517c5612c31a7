"""Algorithmic work of one call, for throughput and roofline figures.

Bytes count what the method must move at least once: every K and V row a
query sees, read once per kv-head (GQA heads share it), plus q, the output,
the block-table entries walked and the context lengths.  Workspace traffic
(split partials) is implementation overhead and is not counted.

The per-token KV size is the uncompressed MHA/GQA formula the tokenspeed
deep-dive (fiv.co.kr) gives in section 7-2: 2 x layers x kv_heads x head_dim
x tokens x bytes per element, here for one layer.
"""

from __future__ import annotations

import numpy as np

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
LLAMA8B_LAYERS = 32


def kv_cache_bytes(layers: int, kv_heads: int, head_dim: int, tokens: int, elem_bytes: int) -> int:
    """Size of an uncompressed K+V cache."""
    return 2 * layers * kv_heads * head_dim * tokens * elem_bytes


def decode_bytes(context_lens, num_q_heads, num_kv_heads, head_dim, elem_bytes, block_size=16) -> dict:
    ctx = np.asarray(context_lens, dtype=np.int64)
    S = ctx.size
    kv = kv_cache_bytes(1, num_kv_heads, head_dim, int(ctx.sum()), elem_bytes)
    qo = 2 * S * num_q_heads * head_dim * elem_bytes
    tables = 4 * int(((ctx + block_size - 1) // block_size).sum()) + 4 * S
    return {"kv": kv, "q_out": qo, "tables": tables, "total": kv + qo + tables}


def decode_fp8_bytes(context_lens, num_q_heads, num_kv_heads, head_dim, q_elem_bytes=2, block_size=16,
                     q_len=1) -> dict:
    """Decode over an fp8 cache: one byte per K and V element plus one
    float32 scale per K row and per V row (per token and kv-head); q and out
    of q_len tokens per sequence in their own (bf16) width; table entries as
    for :func:`decode_bytes`."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    S = ctx.size
    tokens = int(ctx.sum())
    kv = kv_cache_bytes(1, num_kv_heads, head_dim, tokens, 1)
    scales = 2 * num_kv_heads * tokens * 4
    qo = 2 * S * int(q_len) * num_q_heads * head_dim * q_elem_bytes
    tables = 4 * int(((ctx + block_size - 1) // block_size).sum()) + 4 * S
    return {"kv": kv, "scales": scales, "q_out": qo, "tables": tables, "total": kv + scales + qo + tables}


def decode_flops(context_lens, num_q_heads, head_dim) -> int:
    """2*D for q.k plus 2*D for p.v per (q-head, visible key)."""
    return int(4 * head_dim * num_q_heads * np.asarray(context_lens, dtype=np.int64).sum())


def cascade_bytes(context_lens, group_seq_offsets, prefix_lens, num_q_heads, num_kv_heads, head_dim, elem_bytes,
                  block_size=16, kv_fp8=False) -> dict:
    """Shared-prefix decode: each group's prefix K/V read once, every
    member's suffix once, plus q, out and table entries.  With kv_fp8 the
    K/V elements are one-byte codes and each K and V row (token, kv-head)
    adds a float32 scale; q and out keep elem_bytes."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    offs = np.asarray(group_seq_offsets, dtype=np.int64)
    pl = np.asarray(prefix_lens, dtype=np.int64)
    per_seq_prefix = np.repeat(pl, np.diff(offs))
    prefix_tokens = int(pl.sum())
    suffix_tokens = int((ctx - per_seq_prefix).sum())

    def kv_of(tokens):
        if kv_fp8:
            return kv_cache_bytes(1, num_kv_heads, head_dim, tokens, 1) + 2 * num_kv_heads * tokens * 4
        return kv_cache_bytes(1, num_kv_heads, head_dim, tokens, elem_bytes)

    kv = kv_of(prefix_tokens + suffix_tokens)
    S = ctx.size
    qo = 2 * S * num_q_heads * head_dim * elem_bytes
    tables = 4 * int(((ctx + block_size - 1) // block_size).sum()) + 4 * S
    return {"kv": kv, "q_out": qo, "tables": tables, "total": kv + qo + tables, "prefix_kv": kv_of(prefix_tokens)}


def prefix_flops(group_seq_offsets, prefix_lens, num_q_heads, head_dim) -> int:
    """q.k and p.v over the shared prefixes: 4*D per (member q-head, prefix key)."""
    offs = np.asarray(group_seq_offsets, dtype=np.int64)
    pl = np.asarray(prefix_lens, dtype=np.int64)
    return int(4 * head_dim * num_q_heads * (np.diff(offs) * pl).sum())


def mixed_bytes(context_lens, q_lens, num_q_heads, num_kv_heads, head_dim, elem_bytes, block_size=16,
                kv_fp8=False) -> dict:
    """Mixed batch: every segment's visible K/V read once per kv-head (a
    chunk's rows once for all its tokens), plus q and out for every token
    and the table entries walked.  With kv_fp8 the K/V elements are one-byte
    codes and each K and V row (token, kv-head) adds a float32 scale; q and
    out keep elem_bytes."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    ql = np.asarray(q_lens, dtype=np.int64)

    def kv_of(tokens):
        if kv_fp8:
            return kv_cache_bytes(1, num_kv_heads, head_dim, tokens, 1) + 2 * num_kv_heads * tokens * 4
        return kv_cache_bytes(1, num_kv_heads, head_dim, tokens, elem_bytes)

    kv = kv_of(int(ctx.sum()))
    qo = 2 * int(ql.sum()) * num_q_heads * head_dim * elem_bytes
    tables = 4 * int(((ctx + block_size - 1) // block_size).sum()) + 4 * (2 * ctx.size + 1)
    dec = ql == 1
    return {"kv": kv, "q_out": qo, "tables": tables, "total": kv + qo + tables, "decode_kv": kv_of(int(ctx[dec].sum()))}


def chunk_flops(context_lens, q_lens, num_q_heads, head_dim) -> int:
    """q.k and p.v of the prefill chunks (q_len > 1) under the causal mask:
    token i of a segment with L rows and n tokens sees L - n + i + 1 keys."""
    total = 0
    for L, n in zip(np.asarray(context_lens, dtype=np.int64), np.asarray(q_lens, dtype=np.int64)):
        if n > 1:
            total += int(n * (L - n) + n * (n + 1) // 2)
    return int(4 * head_dim * num_q_heads * total)
