"""Seeded synthetic paged-KV workloads.

A workload is a *layout* (how many sequences, their context lengths, which
physical pages each block table names) plus *values* (q, K, V).  Layouts are
drawn with numpy from ``SeedSequence(seed)``; values are drawn either with
numpy (host, any size that fits in RAM) or with torch's generator on a device
(large pools).  The two value routes give different numbers for the same seed;
each is a valid seeded input, and every comparison feeds the *same* arrays to
both sides.

Data layout (shared contract with the GPU library):

* ``q``            ``[T, Hq, D]``   T = sum of per-sequence query lengths
* ``k_pool/v_pool`` ``[num_pages, Hkv, block_size, D]``
* ``block_tables`` ``[S, max_blocks]`` int32, unused slots = -1
* ``context_lens`` ``[S]`` int32: KV rows already in the pool for sequence s,
  including this step's own tokens.
* ``q_lens``       ``[S]`` int32: query tokens of sequence s (1 for decode).

The paged cache model (fixed-size blocks, a per-request table of
non-contiguous blocks, shared-prefix blocks referenced by many tables) is the
one the SwiftLLM page describes in section 3.1 ("PagedAttention and KV cache
management").  Pages a table does not name, and rows past a sequence's last
token inside its last page, are filled with NaN so a stray read shows up.

The shapes of the five named workloads follow the statement of the problem:
a tiny fp32 case, a Llama-3-8B-shaped decode batch, a long-tail mixed-length
batch with one 32768-token sequence, a shared-prefix batch (16 groups x 64
sequences over a 2048-token prefix) and a chunked-prefill piggyback batch.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BF16_NAN_BITS = np.uint16(0x7FC0)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Inputs must be finite.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def pages_of(n_tokens: int, block_size: int) -> int:
    return (int(n_tokens) + block_size - 1) // block_size


@dataclasses.dataclass
class Layout:
    """Structure of one batch: everything except the q/K/V values."""

    name: str
    dtype: str  # "f32" or "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float  # softmax scale, stored exactly as float32
    value_std: float
    context_lens: np.ndarray  # int32 [S]
    q_lens: np.ndarray  # int32 [S]
    block_tables: np.ndarray  # int32 [S, MB]
    num_pages: int
    seed: int
    # cascade groups (contiguous sequence ranges sharing a prefix)
    group_seq_offsets: Optional[np.ndarray] = None  # int32 [NG+1]
    prefix_lens: Optional[np.ndarray] = None  # int32 [NG]
    # storage of the K/V pools: None = same as dtype; "fp8" = e4m3fn codes
    # with one float32 scale per (page, kv-head, slot), q and out in dtype
    kv_dtype: Optional[str] = None
    # sliding window in tokens (None = full history): sequence s keeps the
    # pages from (L - q_len + 1 - window) // block_size on (the earliest
    # new token's window); the entries before them are
    # placeholders naming page 0, which holds no sequence's rows
    window: Optional[int] = None

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def gqa_ratio(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def num_tokens(self) -> int:
        return int(self.q_lens.sum())

    @property
    def cu_q_lens(self) -> np.ndarray:
        cu = np.zeros(self.num_seqs + 1, dtype=np.int32)
        np.cumsum(self.q_lens, out=cu[1:])
        return cu

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def used_pages(self) -> np.ndarray:
        """Sorted distinct physical pages named by any table entry."""
        bt = self.block_tables
        return np.unique(bt[bt >= 0])


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed).spawn(stream + 1)[stream])


def _scale_f32(scale: float) -> float:
    return float(np.float32(scale))


def _fill_tables(page_lists, max_blocks) -> np.ndarray:
    bt = np.full((len(page_lists), max_blocks), -1, dtype=np.int32)
    for s, pl in enumerate(page_lists):
        bt[s, : len(pl)] = pl
    return bt


def decode_layout(
    context_lens,
    *,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    dtype: str,
    block_size: int = 16,
    num_pages: Optional[int] = None,
    pool_factor: float = 1.0,
    scale: Optional[float] = None,
    value_std: float = 0.5,
    seed: int = 0,
    name: str = "decode",
    q_lens=None,
    extra_blocks: int = 0,
) -> Layout:
    """One query token per sequence (or ``q_lens`` tokens), private pages.

    Physical placement: a seeded random permutation of the pool; sequence s
    takes the next ``ceil(L_s / block_size)`` entries of that permutation.
    """
    ctx = np.asarray(context_lens, dtype=np.int32)
    need = [pages_of(L, block_size) for L in ctx]
    total = int(sum(need))
    if num_pages is None:
        num_pages = max(total, int(math.ceil(pool_factor * total)))
    if num_pages < total:
        raise ValueError("pool too small for the requested contexts")
    perm = _rng(seed, 0).permutation(num_pages).astype(np.int32)
    lists, at = [], 0
    for n in need:
        lists.append(perm[at : at + n])
        at += n
    mb = max(need) + extra_blocks if need else 1
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    ql = np.ones_like(ctx) if q_lens is None else np.asarray(q_lens, dtype=np.int32)
    return Layout(
        name=name,
        dtype=dtype,
        num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads,
        head_dim=head_dim,
        block_size=block_size,
        scale=_scale_f32(scale),
        value_std=value_std,
        context_lens=ctx,
        q_lens=ql,
        block_tables=_fill_tables(lists, max(mb, 1)),
        num_pages=int(num_pages),
        seed=seed,
    )


def window_layout(
    context_lens,
    window: int,
    *,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    dtype: str,
    block_size: int = 16,
    scale: Optional[float] = None,
    value_std: float = 0.5,
    seed: int = 0,
    name: str = "window",
    q_len: int = 1,
) -> Layout:
    """q_len query tokens per sequence (the last q_len rows of its context;
    one for decode) over a sliding-window cache: sequence s holds only the
    pages from (L - q_len + 1 - window) // block_size on (the earliest
    token's window), in a seeded permutation of pages 1..; its table entries
    before them are placeholders naming page 0, which no sequence stores
    rows in (it stays NaN)."""
    ctx = np.asarray(context_lens, dtype=np.int32)
    if int(q_len) < 1 or (ctx < int(q_len)).any():
        raise ValueError("need 1 <= q_len <= every context length")
    firsts = [max(0, int(L) - int(q_len) + 1 - int(window)) // block_size for L in ctx]
    need = [pages_of(L, block_size) - f for L, f in zip(ctx, firsts)]
    num_pages = 1 + int(sum(need))
    perm = (1 + _rng(seed, 0).permutation(num_pages - 1)).astype(np.int32)
    mb = max(pages_of(L, block_size) for L in ctx)
    bt = np.full((len(ctx), mb), -1, dtype=np.int32)
    at = 0
    for s, (L, f, n) in enumerate(zip(ctx, firsts, need)):
        bt[s, :f] = 0
        bt[s, f : f + n] = perm[at : at + n]
        at += n
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return Layout(
        name=name,
        dtype=dtype,
        num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads,
        head_dim=head_dim,
        block_size=block_size,
        scale=_scale_f32(scale),
        value_std=value_std,
        context_lens=ctx,
        q_lens=np.full_like(ctx, int(q_len)),
        block_tables=bt,
        num_pages=num_pages,
        seed=seed,
        window=int(window),
    )


def cascade_layout(
    *,
    num_groups: int,
    seqs_per_group: int,
    prefix_len: int,
    suffix_lo: int,
    suffix_hi: int,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    dtype: str = "bf16",
    block_size: int = 16,
    value_std: float = 0.5,
    seed: int = 0,
    name: str = "shared_prefix",
    prefix_lens=None,
    suffix_lens=None,
) -> Layout:
    """Groups of sequences whose tables start with the same prefix pages.

    Each group's prefix pages are allocated once and named by every member's
    table (stored once, referenced many times); each member then gets private
    pages for its suffix of ``U[suffix_lo, suffix_hi]`` tokens.
    """
    if prefix_lens is None:
        prefix_lens = [prefix_len] * num_groups
    prefix_lens = np.asarray(prefix_lens, dtype=np.int32)
    if np.any(prefix_lens % block_size):
        raise ValueError("prefix lengths must be whole pages")
    n_seq = num_groups * seqs_per_group
    if suffix_lens is None:
        suffix_lens = _rng(seed, 1).integers(suffix_lo, suffix_hi + 1, size=n_seq)
    suffix_lens = np.asarray(suffix_lens, dtype=np.int32)
    pre_pages = [int(p) // block_size for p in prefix_lens]
    suf_pages = [pages_of(x, block_size) for x in suffix_lens]
    total = sum(pre_pages) + sum(suf_pages)
    perm = _rng(seed, 0).permutation(total).astype(np.int32)
    at = 0
    lists = []
    ctx = np.zeros(n_seq, dtype=np.int32)
    for g in range(num_groups):
        pre = perm[at : at + pre_pages[g]]
        at += pre_pages[g]
        for i in range(seqs_per_group):
            s = g * seqs_per_group + i
            suf = perm[at : at + suf_pages[s]]
            at += suf_pages[s]
            lists.append(np.concatenate([pre, suf]))
            ctx[s] = prefix_lens[g] + suffix_lens[s]
    offs = np.arange(num_groups + 1, dtype=np.int32) * seqs_per_group
    return Layout(
        name=name,
        dtype=dtype,
        num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads,
        head_dim=head_dim,
        block_size=block_size,
        scale=_scale_f32(1.0 / math.sqrt(head_dim)),
        value_std=value_std,
        context_lens=ctx,
        q_lens=np.ones(n_seq, dtype=np.int32),
        block_tables=_fill_tables(lists, max(len(x) for x in lists)),
        num_pages=int(total),
        seed=seed,
        group_seq_offsets=offs,
        prefix_lens=prefix_lens,
    )


def mixed_layout(
    *,
    chunk_prefixes,
    chunk_len: int,
    decode_ctx,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    dtype: str = "bf16",
    block_size: int = 16,
    value_std: float = 0.5,
    seed: int = 0,
    name: str = "chunked_piggyback",
) -> Layout:
    """Prefill chunks (``chunk_len`` new tokens after an existing prefix)
    followed by decode sequences (one new token), in one batch.

    ``context_lens`` counts every row already in the pool, the chunk's own
    new rows included; a chunk token i may see rows ``[0, prefix + i]``.
    """
    cp = [int(x) for x in chunk_prefixes]
    dc = [int(x) for x in decode_ctx]
    ctx = [p + chunk_len for p in cp] + dc
    ql = [chunk_len] * len(cp) + [1] * len(dc)
    lay = decode_layout(
        ctx,
        num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads,
        head_dim=head_dim,
        dtype=dtype,
        block_size=block_size,
        value_std=value_std,
        seed=seed,
        name=name,
        q_lens=ql,
    )
    return lay


# ----------------------------------------------------------------------------
# The named workloads.
# ----------------------------------------------------------------------------


def _tiny_f32(seed=0):
    return decode_layout(
        [17, 64, 100, 255],
        num_q_heads=8,
        num_kv_heads=2,
        head_dim=64,
        dtype="f32",
        num_pages=64,
        value_std=1.0,
        seed=seed,
        name="tiny_f32",
    )


def _llama8b_decode(seed=0):
    ctx = _rng(seed, 1).integers(512, 4097, size=64)
    return decode_layout(
        ctx,
        num_q_heads=32,
        num_kv_heads=8,
        head_dim=128,
        dtype="bf16",
        pool_factor=1.25,
        scale=1.0 / math.sqrt(128.0),
        seed=seed,
        name="llama8b_decode",
    )


def _longtail_splitkv(seed=0):
    r = _rng(seed, 1)
    u = r.uniform(math.log(16.0), math.log(32768.0), size=256)
    ctx = np.clip(np.floor(np.exp(u)), 16, 32768).astype(np.int32)
    ctx[int(r.integers(0, 256))] = 32768
    return decode_layout(
        ctx,
        num_q_heads=64,
        num_kv_heads=8,
        head_dim=128,
        dtype="bf16",
        seed=seed,
        name="longtail_splitkv",
    )


def _shared_prefix(seed=0):
    return cascade_layout(
        num_groups=16,
        seqs_per_group=64,
        prefix_len=2048,
        suffix_lo=1,
        suffix_hi=512,
        num_q_heads=32,
        num_kv_heads=8,
        head_dim=128,
        seed=seed,
    )


def _chunked_piggyback(seed=0):
    dc = _rng(seed, 1).integers(256, 8193, size=256)
    return mixed_layout(
        chunk_prefixes=[0, 1024, 4096, 8192],
        chunk_len=512,
        decode_ctx=dc,
        num_q_heads=32,
        num_kv_heads=8,
        head_dim=128,
        seed=seed,
    )


def _llama8b_decode_fp8(seed=0):
    lay = _llama8b_decode(seed)
    lay.name = "llama8b_decode_fp8"
    lay.kv_dtype = "fp8"
    return lay


def _llama8b_prefill_append(seed=0):
    """The Llama-shaped batch with every row new this step (a whole prefill
    written into the cache): the KV-append workload that moves enough bytes
    to be timed by its bandwidth."""
    lay = _llama8b_decode(seed)
    lay.name = "llama8b_prefill_append"
    lay.q_lens = lay.context_lens.copy()
    return lay


def _longtail_window4096(seed=0):
    """The long-tail batch's lengths and heads over a 4096-token sliding
    window (every sequence attends to at most its last 4096 rows)."""
    base = _longtail_splitkv(seed)
    return window_layout(base.context_lens, 4096, num_q_heads=base.num_q_heads, num_kv_heads=base.num_kv_heads,
                         head_dim=base.head_dim, dtype=base.dtype, seed=seed, name="longtail_window4096")


def _shared_prefix_fp8(seed=0):
    """The shared-prefix batch over an fp8 (e4m3fn) cache."""
    lay = _shared_prefix(seed)
    lay.name = "shared_prefix_fp8"
    lay.kv_dtype = "fp8"
    return lay


def _llama8b_multitoken4_window1024(seed=0):
    """The 4-token decode step of the Llama-shaped batch over a 1024-token
    sliding window: token i of a sequence with L rows sees the rows
    [L - 4 + i + 1 - 1024, L - 4 + i]."""
    base = _llama8b_decode(seed)
    return window_layout(base.context_lens, 1024, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                         seed=seed, name="llama8b_multitoken4_window1024", q_len=4)


def _llama8b_prefill_append_fp8(seed=0):
    """The whole-prefill append, quantised into an fp8 cache."""
    lay = _llama8b_prefill_append(seed)
    lay.name = "llama8b_prefill_append_fp8"
    lay.kv_dtype = "fp8"
    return lay


def _llama8b_multitoken4(seed=0):
    """The Llama-shaped batch decoding 4 tokens per sequence at once (a
    speculative-decoding step): 64 segments of q_len 4, causal among the 4."""
    base = _llama8b_decode(seed)
    prefixes = [int(L) - 4 for L in base.context_lens]
    return mixed_layout(chunk_prefixes=prefixes, chunk_len=4, decode_ctx=[], num_q_heads=32, num_kv_heads=8,
                        head_dim=128, seed=seed, name="llama8b_multitoken4")


def _llama8b_multitoken4_fp8(seed=0):
    """The 4-token decode step over an fp8 (e4m3fn) cache."""
    lay = _llama8b_multitoken4(seed)
    lay.name = "llama8b_multitoken4_fp8"
    lay.kv_dtype = "fp8"
    return lay


def _chunked_piggyback_fp8(seed=0):
    """The mixed batch (4 prefill chunks + 256 decode tokens) over an fp8
    (e4m3fn) cache."""
    lay = _chunked_piggyback(seed)
    lay.name = "chunked_piggyback_fp8"
    lay.kv_dtype = "fp8"
    return lay


WORKLOADS = {
    "tiny_f32": _tiny_f32,
    "chunked_piggyback_fp8": _chunked_piggyback_fp8,
    "llama8b_multitoken4_fp8": _llama8b_multitoken4_fp8,
    "llama8b_multitoken4": _llama8b_multitoken4,
    "llama8b_prefill_append_fp8": _llama8b_prefill_append_fp8,
    "longtail_window4096": _longtail_window4096,
    "llama8b_multitoken4_window1024": _llama8b_multitoken4_window1024,
    "shared_prefix_fp8": _shared_prefix_fp8,
    "llama8b_prefill_append": _llama8b_prefill_append,
    "llama8b_decode": _llama8b_decode,
    "llama8b_decode_fp8": _llama8b_decode_fp8,
    "longtail_splitkv": _longtail_splitkv,
    "shared_prefix": _shared_prefix,
    "chunked_piggyback": _chunked_piggyback,
}


def workload(name: str, seed: int = 0) -> Layout:
    return WORKLOADS[name](seed)


# ----------------------------------------------------------------------------
# Values.
# ----------------------------------------------------------------------------


def _valid_rows_mask(lay: Layout) -> np.ndarray:
    """bool [num_pages, block_size]: rows some sequence stores a token in
    (for a sliding window: the rows of the pages it still keeps)."""
    valid = np.zeros((lay.num_pages, lay.block_size), dtype=bool)
    bs = lay.block_size
    for s in range(lay.num_seqs):
        L = int(lay.context_lens[s])
        n = pages_of(L, bs)
        first = 0 if lay.window is None else max(0, L - int(lay.q_lens[s]) + 1 - lay.window) // bs
        pg = lay.block_tables[s, :n]
        valid[pg[first : n - 1]] = True
        last = L - (n - 1) * bs
        valid[pg[n - 1], :last] = True
    return valid


def values_numpy(lay: Layout, seed: Optional[int] = None):
    """Draw q, k_pool, v_pool on the host.

    f32 layouts give float32 arrays; bf16 layouts give uint16 bit patterns
    (rounded to nearest even from float32 draws).  Unused pages and the tail
    rows of each sequence's last page are NaN.
    """
    seed = lay.seed if seed is None else seed
    H, Hkv, D, BS = lay.num_q_heads, lay.num_kv_heads, lay.head_dim, lay.block_size
    shp = (lay.num_pages, Hkv, BS, D)
    arrs = []
    for i, shape in enumerate([(lay.num_tokens, H, D), shp, shp]):
        x = _rng(seed, 10 + i).standard_normal(size=shape, dtype=np.float32)
        if lay.value_std != 1.0:
            x *= np.float32(lay.value_std)
        arrs.append(x)
    q, k, v = arrs
    valid = _valid_rows_mask(lay)  # [NP, BS]
    bad = ~valid
    if lay.dtype == "bf16":
        q, k, v = (bf16_bits_from_f32(a) for a in (q, k, v))
        for a in (k, v):
            a.transpose(0, 2, 1, 3)[bad] = BF16_NAN_BITS
    else:
        for a in (k, v):
            a.transpose(0, 2, 1, 3)[bad] = np.nan
    return q, k, v


def values_torch(lay: Layout, device, seed: Optional[int] = None, chunk_pages: int = 4096):
    """Draw q, k_pool, v_pool directly on ``device`` with torch's generator.

    Returns torch tensors in float32 or bfloat16.  Same NaN poisoning as
    :func:`values_numpy`.  Used for pools too large to draw on the host.
    """
    import torch

    seed = lay.seed if seed is None else seed
    tdt = torch.float32 if lay.dtype == "f32" else torch.bfloat16
    H, Hkv, D, BS = lay.num_q_heads, lay.num_kv_heads, lay.head_dim, lay.block_size
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1000003 + 17)
    q = (torch.randn((lay.num_tokens, H, D), generator=gen, device=device) * lay.value_std).to(tdt)
    pools = []
    for _ in range(2):
        pool = torch.empty((lay.num_pages, Hkv, BS, D), dtype=tdt, device=device)
        for p0 in range(0, lay.num_pages, chunk_pages):
            p1 = min(lay.num_pages, p0 + chunk_pages)
            x = torch.randn((p1 - p0, Hkv, BS, D), generator=gen, device=device)
            pool[p0:p1] = (x * lay.value_std).to(tdt)
        pools.append(pool)
    bad = torch.from_numpy(~_valid_rows_mask(lay)).to(device)  # [NP, BS]
    for pool in pools:
        pool.masked_fill_(bad[:, None, :, None], float("nan"))
    return q, pools[0], pools[1]


def new_rows_numpy(lay: Layout, seed: Optional[int] = None):
    """This step's new K/V rows, ``[T, Hkv, D]`` each (T = sum of q_lens), on
    the host, in the layout's stored form (float32, or bf16 bit patterns),
    drawn N(0, value_std^2) from their own seeded streams."""
    seed = lay.seed if seed is None else seed
    shape = (lay.num_tokens, lay.num_kv_heads, lay.head_dim)
    out = []
    for i in range(2):
        x = _rng(seed, 20 + i).standard_normal(size=shape, dtype=np.float32)
        if lay.value_std != 1.0:
            x *= np.float32(lay.value_std)
        out.append(bf16_bits_from_f32(x) if lay.dtype == "bf16" else x)
    return out[0], out[1]


def new_rows_torch(lay: Layout, device, seed: Optional[int] = None):
    """As :func:`new_rows_numpy`, drawn on ``device`` with torch's generator."""
    import torch

    seed = lay.seed if seed is None else seed
    tdt = torch.float32 if lay.dtype == "f32" else torch.bfloat16
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1000003 + 29)
    shape = (lay.num_tokens, lay.num_kv_heads, lay.head_dim)
    return tuple((torch.randn(shape, generator=gen, device=device) * lay.value_std).to(tdt) for _ in range(2))


# ----------------------------------------------------------------------------
# fp8 (e4m3fn) pools.
# ----------------------------------------------------------------------------

FP8_CODE_STD = 128.0  # spread of the stored codes before the cast (|code| <= 448)
FP8_NAN_CODE = np.uint8(0x7F)


def fp8_values_torch(lay: Layout, device, seed: Optional[int] = None, chunk_pages: int = 4096):
    """q (bf16) and fp8 K/V pools drawn on ``device``.

    Codes: N(0, 1) * FP8_CODE_STD clamped to +-448 and cast to
    ``float8_e4m3fn`` by torch (the cast only turns the draw into valid
    codes); scales: value_std / FP8_CODE_STD * U[0.8, 1.2] per (page,
    kv-head, slot), float32, so read-back rows spread like the bf16
    workloads' N(0, value_std^2) values.  Unused pages and the tail rows of
    each last page hold the NaN code 0x7F and a NaN scale.  Returns q [T, Hq,
    D] bf16, k_codes, v_codes uint8 [NP, Hkv, BS, D], k_scales, v_scales
    float32 [NP, Hkv, BS].
    """
    import torch

    seed = lay.seed if seed is None else seed
    H, Hkv, D, BS = lay.num_q_heads, lay.num_kv_heads, lay.head_dim, lay.block_size
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) * 1000003 + 41)
    q = (torch.randn((lay.num_tokens, H, D), generator=gen, device=device) * lay.value_std).to(torch.bfloat16)
    bad = torch.from_numpy(~_valid_rows_mask(lay)).to(device)  # [NP, BS]
    out = []
    for _ in range(2):
        codes = torch.empty((lay.num_pages, Hkv, BS, D), dtype=torch.uint8, device=device)
        for p0 in range(0, lay.num_pages, chunk_pages):
            p1 = min(lay.num_pages, p0 + chunk_pages)
            x = torch.randn((p1 - p0, Hkv, BS, D), generator=gen, device=device) * FP8_CODE_STD
            codes[p0:p1] = x.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
        scales = (torch.rand((lay.num_pages, Hkv, BS), generator=gen, device=device) * 0.4 + 0.8) * (
            lay.value_std / FP8_CODE_STD)
        codes.masked_fill_(bad[:, None, :, None], int(FP8_NAN_CODE))
        scales.masked_fill_(bad[:, None, :], float("nan"))
        out += [codes, scales]
    return q, out[0], out[1], out[2], out[3]


def fp8_values_numpy(lay: Layout, seed: Optional[int] = None):
    """As :func:`fp8_values_torch`, on the host (q as bf16 bit patterns,
    codes uint8, scales float32 numpy arrays)."""
    import torch

    q, kc, ks, vc, vs = fp8_values_torch(lay, torch.device("cpu"), seed)
    return (q.view(torch.int16).numpy().view(np.uint16), kc.numpy(), ks.numpy(), vc.numpy(), vs.numpy())
