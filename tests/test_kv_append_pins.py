"""Pins for the KV-append oracle (``oracle.kv_append``).

Each ``pin_*`` takes an implementation with the oracle's signature and
returns a list of failure strings, so that the planted-mistake test at the
bottom can run every pin against deliberately broken copies and require
that some pin notices.  Nothing here compares the oracle with itself.
"""

import math

import numpy as np
import pytest

import oracle

BS = 16


def make_case(rng, hkv=2, d=8, n_seqs=5, dtype=np.float32, max_ctx=70, pool_extra=4):
    """Random segments (decode tokens and chunks), a random page placement,
    pools with random values in every row named by a table and NaN
    elsewhere.  Returns a dict of the oracle's arguments."""
    ctx = rng.integers(1, max_ctx + 1, size=n_seqs).astype(np.int32)
    ql = np.array([1 if rng.random() < 0.5 else int(rng.integers(1, L + 1)) for L in ctx], dtype=np.int32)
    pages_needed = [(int(L) + BS - 1) // BS for L in ctx]
    num_pages = sum(pages_needed) + pool_extra
    perm = list(rng.permutation(num_pages))
    mb = max(pages_needed)
    bt = np.full((n_seqs, mb), -1, dtype=np.int32)
    for s, n in enumerate(pages_needed):
        for j in range(n):
            bt[s, j] = perm.pop()
    kp = rng.standard_normal((num_pages, hkv, BS, d)).astype(np.float32)
    vp = rng.standard_normal((num_pages, hkv, BS, d)).astype(np.float32)
    named = np.zeros(num_pages, dtype=bool)
    named[bt[bt >= 0]] = True
    kp[~named] = np.nan
    vp[~named] = np.nan
    T = int(ql.sum())
    kn = rng.standard_normal((T, hkv, d)).astype(np.float32)
    vn = rng.standard_normal((T, hkv, d)).astype(np.float32)
    if dtype == np.uint16:  # bf16 bit patterns: any 16-bit values are fine to copy
        kp, vp, kn, vn = (rng.integers(0, 1 << 16, size=a.shape).astype(np.uint16) for a in (kp, vp, kn, vn))
    return dict(k_pool=kp, v_pool=vp, k_new=kn, v_new=vn, block_tables=bt, context_lens=ctx, q_lens=ql,
                block_size=BS)


def same_bits(a, b):
    a, b = np.asarray(a), np.asarray(b)
    if a.dtype == np.float32:
        return a.shape == b.shape and np.array_equal(a.view(np.uint32), b.view(np.uint32))
    return a.shape == b.shape and np.array_equal(a, b)


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------


def pin_bruteforce(fn):
    """Element-by-element writes from the definition, pure Python loops."""
    fails = []
    rng = np.random.default_rng(1)
    for trial in range(4):
        c = make_case(rng, dtype=np.uint16 if trial % 2 else np.float32)
        kp = c["k_pool"].copy()
        vp = c["v_pool"].copy()
        t = 0
        for s in range(len(c["context_lens"])):
            L, n = int(c["context_lens"][s]), int(c["q_lens"][s])
            for i in range(n):
                row = L - n + i
                page = int(c["block_tables"][s][row // BS])
                for g in range(kp.shape[1]):
                    for j in range(kp.shape[3]):
                        kp[page][g][row % BS][j] = c["k_new"][t + i][g][j]
                        vp[page][g][row % BS][j] = c["v_new"][t + i][g][j]
            t += n
        gk, gv = fn(**c)
        if not (same_bits(gk, kp) and same_bits(gv, vp)):
            fails.append(f"brute force trial {trial}")
    return fails


def pin_untouched_rows(fn):
    """Rows that no new token maps to keep their bits, NaN poison included."""
    fails = []
    rng = np.random.default_rng(2)
    c = make_case(rng, n_seqs=7)
    gk, gv = fn(**c)
    touched = np.zeros(c["k_pool"].shape[0:1] + (BS,), dtype=bool)
    for s in range(len(c["context_lens"])):
        L, n = int(c["context_lens"][s]), int(c["q_lens"][s])
        for row in range(L - n, L):
            touched[c["block_tables"][s][row // BS], row % BS] = True
    for a, b in ((gk, c["k_pool"]), (gv, c["v_pool"])):
        keep_a = a.transpose(0, 2, 1, 3)[~touched]
        keep_b = b.transpose(0, 2, 1, 3)[~touched]
        if not same_bits(keep_a, keep_b):
            fails.append("a row no token maps to changed")
    return fails


def pin_idempotent(fn):
    """Appending the same rows a second time changes nothing."""
    rng = np.random.default_rng(3)
    c = make_case(rng)
    k1, v1 = fn(**c)
    c2 = dict(c, k_pool=k1, v_pool=v1)
    k2, v2 = fn(**c2)
    return [] if same_bits(k1, k2) and same_bits(v1, v2) else ["second append changed the pools"]


def pin_readback(fn):
    """The attention oracle's own row lookup returns the appended rows."""
    fails = []
    rng = np.random.default_rng(4)
    c = make_case(rng, n_seqs=6)
    gk, gv = fn(**c)
    t = 0
    for s in range(len(c["context_lens"])):
        L, n = int(c["context_lens"][s]), int(c["q_lens"][s])
        for g in range(gk.shape[1]):
            K = oracle.gather_rows(gk, c["block_tables"][s], g, L, BS, "f32")
            V = oracle.gather_rows(gv, c["block_tables"][s], g, L, BS, "f32")
            if not (np.array_equal(K[L - n:], c["k_new"][t:t + n, g].astype(np.float64))
                    and np.array_equal(V[L - n:], c["v_new"][t:t + n, g].astype(np.float64))):
                fails.append(f"segment {s} kv-head {g}: rows read back differ")
        t += n
    return fails


def pin_roundtrip_attention(fn):
    """A whole sequence appended into an empty pool, then the attention
    oracle, equals dense softmax attention over the sequence's rows
    (numpy, written here)."""
    fails = []
    rng = np.random.default_rng(5)
    hkv, d, G = 2, 8, 2
    ctx = np.array([1, 16, 17, 40], dtype=np.int32)
    npg = [(int(L) + BS - 1) // BS for L in ctx]
    num_pages = sum(npg) + 3
    perm = list(rng.permutation(num_pages))
    bt = np.full((len(ctx), max(npg)), -1, dtype=np.int32)
    for s, n in enumerate(npg):
        for j in range(n):
            bt[s, j] = perm.pop()
    dense_k = [rng.standard_normal((int(L), hkv, d)).astype(np.float32) for L in ctx]
    dense_v = [rng.standard_normal((int(L), hkv, d)).astype(np.float32) for L in ctx]
    empty = np.full((num_pages, hkv, BS, d), np.nan, dtype=np.float32)
    kp, vp = fn(empty, empty, np.concatenate(dense_k), np.concatenate(dense_v), bt, ctx, ctx, BS)
    q = rng.standard_normal((len(ctx), hkv * G, d)).astype(np.float32)
    scale = 0.3
    out, lse = oracle.decode(q, kp, vp, bt, ctx, scale, hkv, BS, "f32")
    for s in range(len(ctx)):
        for h in range(hkv * G):
            K = dense_k[s][:, h // G].astype(np.float64)
            V = dense_v[s][:, h // G].astype(np.float64)
            x = float(np.float32(scale)) * (K @ q[s, h].astype(np.float64))
            w = np.exp(x - x.max())
            want = (w @ V) / w.sum()
            if not np.allclose(out[s, h], want, rtol=1e-12, atol=1e-12):
                fails.append(f"sequence {s} head {h}: attention over appended rows differs")
            if not math.isclose(lse[s, h], x.max() + math.log(w.sum()), rel_tol=1e-12, abs_tol=1e-12):
                fails.append(f"sequence {s} head {h}: lse differs")
    return fails


def pin_invalid_entries_skipped(fn):
    """A table entry outside the pool names no page: nothing is written
    through it, and every row that no valid entry maps to keeps its bits."""
    rng = np.random.default_rng(6)
    c = make_case(rng, n_seqs=3)
    L = int(c["context_lens"][0])
    c["block_tables"] = c["block_tables"].copy()
    c["block_tables"][0, (L - 1) // BS] = -1  # the page holding segment 0's last new row
    gk, gv = fn(**c)
    tgt = np.zeros(c["k_pool"].shape[0:1] + (BS,), dtype=bool)
    for s in range(3):
        Ls, ns = int(c["context_lens"][s]), int(c["q_lens"][s])
        for row in range(Ls - ns, Ls):
            p = int(c["block_tables"][s][row // BS])
            if p >= 0:
                tgt[p, row % BS] = True
    fails = []
    for got, old in ((gk, c["k_pool"]), (gv, c["v_pool"])):
        if not same_bits(got.transpose(0, 2, 1, 3)[~tgt], old.transpose(0, 2, 1, 3)[~tgt]):
            fails.append("a row no valid entry maps to changed")
    return fails


ALL_PINS = [pin_bruteforce, pin_untouched_rows, pin_idempotent, pin_readback, pin_roundtrip_attention,
            pin_invalid_entries_skipped]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_passes_pin(pin):
    assert pin(oracle.kv_append) == []


# ---------------------------------------------------------------------------
# planted mistakes (test-owned broken copies of the definition)
# ---------------------------------------------------------------------------


def _mutant(row_of=None, head_of=None, swap_kv=False, skip_last=False):
    def fn(k_pool, v_pool, k_new, v_new, block_tables, context_lens, q_lens, block_size):
        kp, vp = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
        hkv = kp.shape[1]
        t0 = 0
        for s in range(len(context_lens)):
            L, n = int(context_lens[s]), int(q_lens[s])
            for i in range(n - (1 if skip_last and n > 1 else 0)):
                pos = row_of(L, n, i) if row_of else L - n + i
                pos = min(max(pos, 0), L - 1)
                page = int(block_tables[s][pos // block_size])
                if not 0 <= page < kp.shape[0]:
                    continue
                for g in range(hkv):
                    gs = head_of(g, hkv) if head_of else g
                    kk, vv = (v_new, k_new) if swap_kv else (k_new, v_new)
                    kp[page, gs, pos % block_size] = kk[t0 + i, g]
                    vp[page, gs, pos % block_size] = vv[t0 + i, g]
            t0 += n
        return kp, vp
    return fn


@pytest.mark.parametrize(
    "name,fn",
    [
        ("position off by one", _mutant(row_of=lambda L, n, i: L - n + i + 1)),
        ("position from the front", _mutant(row_of=lambda L, n, i: i)),
        ("kv-heads swapped", _mutant(head_of=lambda g, h: (g + 1) % h)),
        ("K and V swapped", _mutant(swap_kv=True)),
        ("last new token dropped", _mutant(skip_last=True)),
    ],
)
def test_planted_mistake_is_caught(name, fn):
    fails = []
    for pin in ALL_PINS:
        try:
            fails += pin(fn)
        except Exception as e:  # a crash also counts as caught
            fails.append(f"{pin.__name__} raised {e!r}")
    assert fails, f"no pin noticed: {name}"
