"""Pins for the sliding-window decode oracles (one token per sequence, and
q_len tokens per sequence with a window each): brute force, closed forms,
reductions to plain decode / multi-token decode, and planted mistakes (an
off-by-one window edge, one window for all of a sequence's tokens, reading
the placeholder entries)."""

import math

import numpy as np
import pytest

import oracle
from oracle import attention as opa
from workloads import values_numpy, window_layout


def small(window, ctx=(1, 5, 16, 17, 40, 100, 333), hq=4, hkv=2, d=8, dtype="f32", seed=1):
    lay = window_layout(list(ctx), window, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype, seed=seed)
    return lay, values_numpy(lay)


def run_window(lay, vals):
    q, k, v = vals
    return oracle.decode_window(q, k, v, lay.block_tables, lay.context_lens, lay.window, lay.scale,
                                lay.num_kv_heads, lay.block_size, lay.dtype)


def pin_bruteforce():
    """Python loops: look each window row up in the table by hand, softmax
    with math.exp."""
    fails = []
    for window in (1, 7, 16, 50):
        lay, (q, k, v) = small(window)
        out, lse = run_window(lay, (q, k, v))
        G = lay.num_q_heads // lay.num_kv_heads
        sc = float(np.float32(lay.scale))
        for s, L in enumerate(lay.context_lens):
            L = int(L)
            for h in range(lay.num_q_heads):
                g = h // G
                xs, vs = [], []
                for t in range(max(0, L - window), L):
                    p, r = int(lay.block_tables[s, t // 16]), t % 16
                    xs.append(sc * sum(float(q[s, h, j]) * float(k[p, g, r, j]) for j in range(lay.head_dim)))
                    vs.append([float(v[p, g, r, j]) for j in range(lay.head_dim)])
                m = max(xs)
                w = [math.exp(x - m) for x in xs]
                z = sum(w)
                o = [sum(w[i] * vs[i][j] for i in range(len(w))) / z for j in range(lay.head_dim)]
                if not (np.max(np.abs(np.array(o) - out[s, h])) <= 1e-12 and abs(m + math.log(z) - lse[s, h]) <= 1e-12):
                    fails.append(f"window {window} seq {s} head {h}")
    return fails


def pin_closed_forms():
    """Window 1: the last row's V exactly, lse = its score."""
    lay, (q, k, v) = small(1)
    out, lse = run_window(lay, (q, k, v))
    fails = []
    sc = float(np.float32(lay.scale))
    for s, L in enumerate(lay.context_lens):
        t = int(L) - 1
        p, r = int(lay.block_tables[s, t // 16]), t % 16
        for h in range(lay.num_q_heads):
            g = h // (lay.num_q_heads // lay.num_kv_heads)
            if not np.array_equal(out[s, h], v[p, g, r].astype(np.float64)):
                fails.append(f"seq {s}: window 1 is not the last V row")
            x = sc * float(np.dot(q[s, h].astype(np.float64), k[p, g, r].astype(np.float64)))
            if not abs(lse[s, h] - x) <= 1e-12:
                fails.append(f"seq {s}: window 1 lse is not the last score")
    return fails


def pin_reductions():
    """A window covering every sequence equals plain decode; a page-aligned
    window equals plain decode over a table that starts at the window."""
    fails = []
    lay, vals = small(10_000, seed=4)
    q, k, v = vals
    out, lse = run_window(lay, vals)
    ro, rl = oracle.decode(q, k, v, lay.block_tables, lay.context_lens, lay.scale, lay.num_kv_heads, 16, lay.dtype)
    if not (np.array_equal(out, ro) and np.array_equal(lse, rl)):
        fails.append("a window longer than every context differs from decode")
    lay, vals = small(32, ctx=(48, 64, 100, 333), seed=5)
    q, k, v = vals
    out, lse = run_window(lay, vals)
    bt = np.full_like(lay.block_tables, -1)
    ctx = lay.context_lens.copy()
    for s, L in enumerate(lay.context_lens):
        lo = int(L) - 32
        f = lo // 16
        n = (int(L) + 15) // 16
        bt[s, : n - f] = lay.block_tables[s, f:n]
        ctx[s] = int(L) - f * 16
    # the shifted table starts at the window's first page; where the window
    # starts on a page boundary the two must agree bit for bit
    ro, rl = oracle.decode(q, k, v, bt, ctx, lay.scale, lay.num_kv_heads, 16, lay.dtype)
    aligned = [s for s, L in enumerate(lay.context_lens) if (int(L) - 32) % 16 == 0]
    if not aligned:
        fails.append("no page-aligned window in the case")
    for s in aligned:
        if not (np.array_equal(out[s], ro[s]) and np.array_equal(lse[s], rl[s])):
            fails.append(f"seq {s}: page-aligned window differs from decode over the shifted table")
    return fails


def pin_placeholders_are_never_read():
    """The placeholder page is NaN: every output stays finite."""
    lay, vals = small(20, ctx=(100, 333, 1000), dtype="bf16", d=16, seed=6)
    out, lse = run_window(lay, vals)
    return [] if np.isfinite(out).all() and np.isfinite(lse).all() else ["a placeholder row reached the result"]


ALL_PINS = [pin_bruteforce, pin_closed_forms, pin_reductions, pin_placeholders_are_never_read]


# -- q_len tokens per sequence, each with its own window ---------------------


def small_multi(window, q_len, ctx=(4, 5, 16, 17, 40, 100, 333), hq=4, hkv=2, d=8, dtype="f32", seed=1):
    lay = window_layout(list(ctx), window, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype, seed=seed,
                        q_len=q_len)
    return lay, values_numpy(lay)


def run_multi(lay, vals, q_len):
    q, k, v = vals
    return oracle.decode_multi_window(q, k, v, lay.block_tables, lay.context_lens, q_len, lay.window, lay.scale,
                                      lay.num_kv_heads, lay.block_size, lay.dtype)


def pin_multi_bruteforce():
    """Python loops: token i of sequence s (position L - n + i) against the
    rows of its own window, looked up in the table by hand, math.exp."""
    fails = []
    for window, n in ((1, 2), (7, 3), (16, 4), (50, 4)):
        lay, (q, k, v) = small_multi(window, n)
        out, lse = run_multi(lay, (q, k, v), n)
        G = lay.num_q_heads // lay.num_kv_heads
        sc = float(np.float32(lay.scale))
        for s, L in enumerate(lay.context_lens):
            L = int(L)
            for i in range(n):
                pos = L - n + i
                for h in range(lay.num_q_heads):
                    g = h // G
                    xs, vs = [], []
                    for t in range(max(0, pos + 1 - window), pos + 1):
                        p, r = int(lay.block_tables[s, t // 16]), t % 16
                        xs.append(sc * sum(float(q[s * n + i, h, j]) * float(k[p, g, r, j])
                                           for j in range(lay.head_dim)))
                        vs.append([float(v[p, g, r, j]) for j in range(lay.head_dim)])
                    m = max(xs)
                    w = [math.exp(x - m) for x in xs]
                    z = sum(w)
                    o = np.array([sum(w[u] * vs[u][j] for u in range(len(w))) / z for j in range(lay.head_dim)])
                    row = s * n + i
                    if not (np.max(np.abs(o - out[row, h])) <= 1e-12 and abs(m + math.log(z) - lse[row, h]) <= 1e-12):
                        fails.append(f"window {window} q_len {n} seq {s} token {i} head {h}")
    return fails


def pin_multi_window_one():
    """Window 1: each token returns its own row's V exactly and lse = its own
    score (so the windows move with the token)."""
    n = 3
    lay, (q, k, v) = small_multi(1, n)
    out, lse = run_multi(lay, (q, k, v), n)
    sc = float(np.float32(lay.scale))
    G = lay.num_q_heads // lay.num_kv_heads
    fails = []
    for s, L in enumerate(lay.context_lens):
        for i in range(n):
            t = int(L) - n + i
            p, r = int(lay.block_tables[s, t // 16]), t % 16
            for h in range(lay.num_q_heads):
                g = h // G
                if not np.array_equal(out[s * n + i, h], v[p, g, r].astype(np.float64)):
                    fails.append(f"seq {s} token {i}: window 1 is not its own V row")
                x = sc * float(np.dot(q[s * n + i, h].astype(np.float64), k[p, g, r].astype(np.float64)))
                if not abs(lse[s * n + i, h] - x) <= 1e-12:
                    fails.append(f"seq {s} token {i}: window 1 lse is not its own score")
    return fails


def pin_multi_reductions():
    """q_len 1 equals the one-token window oracle; a window covering every
    context equals multi-token decode (the chunk definition with q_len
    tokens per sequence); both bit for bit."""
    fails = []
    lay, vals = small_multi(20, 1, seed=7)
    q, k, v = vals
    out, lse = run_multi(lay, vals, 1)
    ro, rl = oracle.decode_window(q, k, v, lay.block_tables, lay.context_lens, 20, lay.scale, lay.num_kv_heads, 16,
                                  lay.dtype)
    if not (np.array_equal(out, ro) and np.array_equal(lse, rl)):
        fails.append("q_len 1 differs from the one-token window oracle")
    n = 4
    lay, vals = small_multi(10_000, n, seed=8)
    q, k, v = vals
    out, lse = run_multi(lay, vals, n)
    ro, rl = oracle.paged_attention(q, k, v, lay.block_tables, lay.context_lens, lay.q_lens, lay.scale,
                                    lay.num_kv_heads, 16, lay.dtype)
    if not (np.array_equal(out, ro) and np.array_equal(lse, rl)):
        fails.append("a window longer than every context differs from multi-token decode")
    return fails


def pin_multi_placeholders_are_never_read():
    """Placeholders (the NaN page) before the earliest token's window: every
    output stays finite."""
    n = 4
    lay, vals = small_multi(20, n, ctx=(100, 333, 1000), dtype="bf16", d=16, seed=9)
    out, lse = run_multi(lay, vals, n)
    return [] if np.isfinite(out).all() and np.isfinite(lse).all() else ["a placeholder row reached the result"]


MULTI_PINS = [pin_multi_bruteforce, pin_multi_window_one, pin_multi_reductions,
              pin_multi_placeholders_are_never_read]


@pytest.mark.parametrize("pin", MULTI_PINS, ids=lambda p: p.__name__)
def test_multi_pin(pin):
    fails = pin()
    assert not fails, fails[:5]


def _multi_window_plus(delta):
    orig = opa.decode_multi_window

    def wrong(q, k, v, bt, ctx, q_len, window, *a, **kw):
        return orig(q, k, v, bt, ctx, q_len, max(1, window + delta), *a, **kw)

    return wrong


def _multi_last_token_window(q, k, v, bt, ctx, q_len, window, scale, hkv, bs, dtype, seqs=None):
    # every token gets the last token's window (the earlier tokens then see
    # rows after their own position)
    out = np.full((q.shape[0], q.shape[1], q.shape[2]), np.nan)
    lse = np.full((q.shape[0], q.shape[1]), np.nan)
    for i in range(q_len):
        o, l = opa.decode_window(q[i::q_len], k, v, bt, ctx, window, scale, hkv, bs, dtype, seqs)
        out[i::q_len], lse[i::q_len] = o, l
    return out, lse


def _multi_reads_placeholders(q, k, v, bt, ctx, q_len, window, scale, hkv, bs, dtype, seqs=None):
    # "forgets" the windows: plain multi-token decode through the placeholders
    ql = np.full(len(ctx), q_len)
    return opa.paged_attention(q, k, v, bt, ctx, ql, scale, hkv, bs, dtype, seqs)


@pytest.mark.parametrize("name,fn", [("window+1", _multi_window_plus(1)), ("window-1", _multi_window_plus(-1)),
                                     ("last token's window for all", _multi_last_token_window),
                                     ("reads placeholders", _multi_reads_placeholders)])
def test_multi_planted_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(oracle, "decode_multi_window", fn)
    assert any(p() for p in MULTI_PINS), f"no pin noticed: {name}"


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    fails = pin()
    assert not fails, fails[:5]


def _window_plus(delta):
    orig = opa.decode_window

    def wrong(q, k, v, bt, ctx, window, *a, **kw):
        return orig(q, k, v, bt, ctx, max(1, window + delta), *a, **kw)

    return wrong


def _reads_placeholders(q, k, v, bt, ctx, window, scale, hkv, bs, dtype, seqs=None):
    # "forgets" the window: attends from row 0, through the placeholders
    return opa.decode(q, k, v, bt, ctx, scale, hkv, bs, dtype, seqs)


@pytest.mark.parametrize("name,fn", [("window+1", _window_plus(1)), ("window-1", _window_plus(-1)),
                                     ("reads placeholders", _reads_placeholders)])
def test_planted_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(oracle, "decode_window", fn)
    assert any(p() for p in ALL_PINS), f"no pin noticed: {name}"
