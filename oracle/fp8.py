"""fp64 reference for an fp8 (e4m3) paged KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes
----------------
The tokenspeed 딥다이브 page (section 6-4, GPU DSL and quantisation) describes
FP8 as a way to cut the cost of storing and moving numbers, and gives the
per-group recipe its token-group quantiser follows: the scale of a group is
its largest magnitude (at least 1e-10) divided by the largest finite value of
the 8-bit type; the group divided by the scale is clamped to that type's range
and converted to ``float8_e4m3fn``; a stored code is read back as its value
times the scale.

Readings (the page leaves these open):

* the group is one row of one kv-head for one token (``head_dim`` values) —
  the KV-cache form of a token group; each (page, kv-head, slot) carries one
  float32 scale for K and one for V;
* e4m3fn is the OCP 8-bit format with 4 exponent bits (bias 7), 3 mantissa
  bits, subnormals, no infinities, and NaN at the all-ones exponent+mantissa
  pattern; its largest finite value is 448;
* the division, the clamp and the scale are float32 (the quantiser's tensors
  are float32); the conversion rounds to nearest, ties to even;
* attention over an fp8 cache is the attention of ``oracle/attention.py``
  over the read-back (dequantised) K and V rows, computed in float64; with
  several new tokens per sequence (``decode_multi_fp8``) token i sees the
  rows up to its own position, as in a prefill chunk.

Pins (tests/test_fp8_pins.py):
* the code table against torch's own ``float8_e4m3fn`` conversion (a library
  routine) for all 256 codes, and closed forms (1.0, 448, the smallest
  subnormal 2^-9, the smallest normal 2^-6, signed zero, NaN);
* the quantiser against torch's float32 divide + clamp + ``float8_e4m3fn``
  cast, bit for bit; the row maximum maps to +-448; an all-zero row; the
  read-back error bound of round-to-nearest; sign symmetry;
* attention: with power-of-two scales the read-back rows are exact bf16
  values, and the result equals the (pinned) bf16 attention oracle on those
  values bit for bit; brute force on tiny inputs with Python loops;
* planted mistakes (scale ignored, K scale used for V, FNUZ bias 8) are each
  caught;
* multi-token decode: q_len 1 equals ``decode_fp8``; with power-of-two
  scales it equals the pinned chunk oracle (``oracle.mixed_chunk``) on the
  read-back bf16 values bit for bit; brute force with Python loops; a causal
  edge one row off and tokens read in the wrong order are caught;
* a mixed batch (``mixed_chunk_fp8``: prefill chunks and decode tokens,
  q_lens per segment): all-ones q_lens equal ``decode_fp8`` and a uniform
  q_len equals ``decode_multi_fp8`` bit for bit; with power-of-two scales a
  ragged batch equals the pinned chunk oracle on the read-back bf16 values
  bit for bit; brute force with Python loops; the causal mistakes above and
  segments read at the wrong offsets in q are caught;
* shared-prefix decode (``prefix_cascade_fp8``: the group check, then
  ``decode_fp8``): equal to the log-sum-exp merge of the fp8 attention over
  the prefix rows alone and over the suffix rows alone; a broken group is
  rejected; dropping the suffix, skipping the check and counting the prefix
  twice are each caught;
* the quantising append (``kv_append_fp8``: quantise each new row, then
  place codes and scale as ``oracle.kv_append`` places a row) against a
  brute-force element loop, and its read-back against the new rows within
  half a code step.
"""

from __future__ import annotations

import math

import numpy as np

from .attention import attend, check_block_tables, stored_to_f64

E4M3_MAX = 448.0
E4M3_BIAS = 7


def e4m3_value(code: int) -> float:
    """Value of one e4m3fn code (0..255) from the format's definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - E4M3_BIAS)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - E4M3_BIAS)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Read stored e4m3fn codes (uint8) exactly as float64."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def round_to_e4m3(y: np.ndarray) -> np.ndarray:
    """Round values already inside [-448, 448] to the nearest e4m3fn code,
    ties to the code with an even mantissa (its lowest bit clear).

    Brute force over the finite codes: the nearest value wins; a zero keeps
    its sign (+0 and -0 are equally near, the sign decides).
    """
    y = np.asarray(y, dtype=np.float64)
    flat = y.reshape(-1)
    if np.any(~((flat >= -E4M3_MAX) & (flat <= E4M3_MAX))):
        raise ValueError("value outside the e4m3fn range (or NaN); clamp first")
    codes = np.array([c for c in range(256) if not math.isnan(E4M3_TABLE[c])], dtype=np.int64)
    vals = E4M3_TABLE[codes]
    out = np.empty(flat.shape, dtype=np.uint8)
    for a in range(0, flat.size, 4096):
        v = flat[a : a + 4096]
        d = np.abs(vals[None, :] - v[:, None])
        cand = d == d.min(axis=1, keepdims=True)
        cand &= np.signbit(vals)[None, :] == np.signbit(v)[:, None]
        even = cand & ((codes & 1) == 0)[None, :]
        pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
        out[a : a + 4096] = codes[pick]
    return out.reshape(y.shape)


def quantize_rows(x: np.ndarray):
    """Quantise each row (last axis) of ``x`` to e4m3fn with one scale per
    row, as the token-group quantiser does.

    Returns ``(codes uint8, scales float32)`` with ``scales.shape ==
    x.shape[:-1]``; the read-back value of ``codes[..., d]`` is
    ``e4m3_to_f64(codes[..., d]) * scales[...]``.
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = (np.maximum(amax, np.float32(1e-10)) / np.float32(E4M3_MAX)).astype(np.float32)
    y = (x / scale[..., None]).astype(np.float32)
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return round_to_e4m3(y), scale


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Read-back rows: code value times the row's scale, in float64 (exact:
    4 significant bits times a 24-bit scale)."""
    return e4m3_to_f64(codes) * np.asarray(scales, dtype=np.float32).astype(np.float64)[..., None]


def _gather_fp8(codes_pool, scale_pool, table_row, kv_head: int, n_rows: int, block_size: int):
    t = np.arange(n_rows)
    pages = np.asarray(table_row)[t // block_size]
    if n_rows and (pages.min() < 0 or pages.max() >= codes_pool.shape[0]):
        raise IndexError("block table names a page outside the pool")
    slots = t % block_size
    return dequantize(codes_pool[pages, kv_head, slots, :], scale_pool[pages, kv_head, slots])


def decode_fp8(q, k_codes, k_scales, v_codes, v_scales, block_tables, context_lens, scale, num_kv_heads,
               block_size, q_dtype="bf16", seqs=None):
    """One query token per sequence over an fp8 cache.

    ``q`` [S, Hq, D] stored values of ``q_dtype``; ``k_codes``/``v_codes``
    [num_pages, Hkv, block_size, D] uint8 e4m3fn codes; ``k_scales``/
    ``v_scales`` [num_pages, Hkv, block_size] float32.  Returns out [S, Hq, D]
    and lse [S, Hq] in float64; sequences not in ``seqs`` stay NaN.
    """
    ctx = np.asarray(context_lens, dtype=np.int64)
    S, Hq, D = q.shape
    if S != len(ctx):
        raise ValueError("q must hold one token per sequence")
    if Hq % num_kv_heads:
        raise ValueError("q heads must be a multiple of kv heads")
    G = Hq // num_kv_heads
    sc = float(np.float32(scale))
    out = np.full((S, Hq, D), np.nan, dtype=np.float64)
    lse = np.full((S, Hq), np.nan, dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        L = int(ctx[s])
        if L < 1:
            raise ValueError(f"sequence {s}: empty context")
        qs = stored_to_f64(q[s], q_dtype)
        for g in range(num_kv_heads):
            K = _gather_fp8(k_codes, k_scales, block_tables[s], g, L, block_size)
            V = _gather_fp8(v_codes, v_scales, block_tables[s], g, L, block_size)
            for h in range(g * G, (g + 1) * G):
                out[s, h], lse[s, h] = attend(qs[h], K, V, sc)
    return out, lse


def prefix_cascade_fp8(q, k_codes, k_scales, v_codes, v_scales, block_tables, context_lens, scale, num_kv_heads,
                       block_size, group_seq_offsets, prefix_lens, q_dtype="bf16", seqs=None):
    """Shared-prefix (cascade) decode over an fp8 cache: as
    :func:`attention.prefix_cascade` -- defined as plain decode over each
    member's whole table, the prefix blocks shared by the group (Tokasaurus
    page, "dynamic prefix identification"; SwiftLLM page section 3.1) -- with
    the K and V rows read back from e4m3fn codes and their scales
    (tokenspeed 딥다이브 section 6-4), i.e. :func:`decode_fp8`.  The group
    structure is checked first."""
    probs = check_block_tables(block_tables, context_lens, k_codes.shape[0], block_size, group_seq_offsets,
                               prefix_lens)
    if probs:
        raise ValueError("; ".join(probs[:5]))
    return decode_fp8(q, k_codes, k_scales, v_codes, v_scales, block_tables, context_lens, scale, num_kv_heads,
                      block_size, q_dtype, seqs)


def _visible(L: int, q_len: int, i: int) -> int:
    """Rows new token i of a sequence with L rows (the last q_len new) sees:
    rows 0 .. L - q_len + i, its own position included."""
    return L - q_len + i + 1


def decode_multi_fp8(q, k_codes, k_scales, v_codes, v_scales, block_tables, context_lens, q_len, scale,
                     num_kv_heads, block_size, q_dtype="bf16", seqs=None):
    """q_len new tokens per sequence over an fp8 cache, causal among them
    (the chunk reading of the attention oracle: token i of a sequence with L
    rows sees rows up to its own position L - q_len + i).

    ``q`` [S * q_len, Hq, D] stored values, token i of sequence s at row
    s * q_len + i; pools and scales as :func:`decode_fp8`.  Returns out and
    lse of the same leading shape in float64; sequences not in ``seqs`` stay
    NaN.
    """
    ctx = np.asarray(context_lens, dtype=np.int64)
    n = int(q_len)
    T, Hq, D = q.shape
    if n < 1 or T != n * len(ctx):
        raise ValueError("q must hold q_len tokens per sequence")
    if Hq % num_kv_heads:
        raise ValueError("q heads must be a multiple of kv heads")
    G = Hq // num_kv_heads
    sc = float(np.float32(scale))
    out = np.full((T, Hq, D), np.nan, dtype=np.float64)
    lse = np.full((T, Hq), np.nan, dtype=np.float64)
    for s in (range(len(ctx)) if seqs is None else seqs):
        L = int(ctx[s])
        if L < n:
            raise ValueError(f"sequence {s}: fewer rows than new tokens")
        for g in range(num_kv_heads):
            K = _gather_fp8(k_codes, k_scales, block_tables[s], g, L, block_size)
            V = _gather_fp8(v_codes, v_scales, block_tables[s], g, L, block_size)
            for i in range(n):
                row = s * n + i
                qs = stored_to_f64(q[row], q_dtype)
                vis = _visible(L, n, i)
                for h in range(g * G, (g + 1) * G):
                    out[row, h], lse[row, h] = attend(qs[h], K[:vis], V[:vis], sc)
    return out, lse


def _segment_starts(q_lens) -> np.ndarray:
    """First row in q of each segment: the segments' tokens are stored one
    segment after another, so segment s starts at q_lens[0] + .. + q_lens[s-1]."""
    ql = np.asarray(q_lens, dtype=np.int64)
    starts = np.zeros(ql.size + 1, dtype=np.int64)
    np.cumsum(ql, out=starts[1:])
    return starts


def mixed_chunk_fp8(q, k_codes, k_scales, v_codes, v_scales, block_tables, context_lens, q_lens, scale,
                    num_kv_heads, block_size, q_dtype="bf16", seqs=None):
    """Prefill chunks and decode tokens in one batch over an fp8 cache: the
    piggybacked batch of the SwiftLLM page (section 3.3) with K and V rows
    read back from e4m3fn codes and their scales (tokenspeed 딥다이브 section
    6-4).  Segment s has q_lens[s] new tokens, its last rows; token i of a
    segment with L rows and n new tokens sees rows 0 .. L - n + i (a decode
    token, n = 1, sees all L).

    ``q`` [sum(q_lens), Hq, D] stored values of ``q_dtype``, segment after
    segment; pools and scales as :func:`decode_fp8`.  Returns out and lse of
    q's leading shape in float64; segments not in ``seqs`` stay NaN.
    """
    ctx = np.asarray(context_lens, dtype=np.int64)
    ql = np.asarray(q_lens, dtype=np.int64)
    T, Hq, D = q.shape
    if ql.size != ctx.size or (ql < 1).any():
        raise ValueError("one q_len >= 1 per segment")
    starts = _segment_starts(ql)
    if T != int(ql.sum()):
        raise ValueError("q must hold sum(q_lens) tokens")
    if Hq % num_kv_heads:
        raise ValueError("q heads must be a multiple of kv heads")
    G = Hq // num_kv_heads
    sc = float(np.float32(scale))
    out = np.full((T, Hq, D), np.nan, dtype=np.float64)
    lse = np.full((T, Hq), np.nan, dtype=np.float64)
    for s in (range(ctx.size) if seqs is None else seqs):
        L, n = int(ctx[s]), int(ql[s])
        if L < n:
            raise ValueError(f"segment {s}: fewer rows than new tokens")
        for g in range(num_kv_heads):
            K = _gather_fp8(k_codes, k_scales, block_tables[s], g, L, block_size)
            V = _gather_fp8(v_codes, v_scales, block_tables[s], g, L, block_size)
            for i in range(n):
                row = int(starts[s]) + i
                qs = stored_to_f64(q[row], q_dtype)
                vis = _visible(L, n, i)
                for h in range(g * G, (g + 1) * G):
                    out[row, h], lse[row, h] = attend(qs[h], K[:vis], V[:vis], sc)
    return out, lse


def kv_append_fp8(k_codes, k_scales, v_codes, v_scales, k_new, v_new, block_tables, context_lens, q_lens,
                  block_size, new_dtype="bf16"):
    """KV append into an fp8 cache: each new K and V row of each kv-head is
    quantised on its own (the token-group recipe above, group = the row) and
    its codes and scale are written where ``oracle.kv_append`` writes a row.

    ``k_new``, ``v_new``: [T, Hkv, D] stored values of ``new_dtype`` (bf16
    bit patterns or float32), widened exactly to float32 before the
    quantiser.  Returns new (k_codes, k_scales, v_codes, v_scales).
    """
    from .attention import stored_to_f64
    from .kv_append import kv_append

    kx = stored_to_f64(k_new, new_dtype).astype(np.float32)
    vx = stored_to_f64(v_new, new_dtype).astype(np.float32)
    kc_new, ks_new = quantize_rows(kx)
    vc_new, vs_new = quantize_rows(vx)
    kc, vc = kv_append(k_codes, v_codes, kc_new, vc_new, block_tables, context_lens, q_lens, block_size)
    ks, vs = kv_append(np.asarray(k_scales)[..., None], np.asarray(v_scales)[..., None], ks_new[..., None],
                       vs_new[..., None], block_tables, context_lens, q_lens, block_size)
    return kc, ks[..., 0], vc, vs[..., 0]
