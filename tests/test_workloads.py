"""The seeded input generator: determinism and layout sanity for every
named workload (host only)."""

import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, pages_of, values_numpy, window_layout, workload


def kept_tables(lay):
    """For a sliding-window layout: each row's kept entries moved to the
    front and the lengths cut to match (a valid plain table), after checking
    that the entries before them are placeholders naming page 0, which no
    kept entry uses.  Other layouts pass through."""
    if lay.window is None:
        return lay.block_tables, lay.context_lens
    bt = np.full_like(lay.block_tables, -1)
    ctx = lay.context_lens.copy()
    for s, L in enumerate(lay.context_lens):
        f = max(0, int(L) - int(lay.q_lens[s]) + 1 - lay.window) // lay.block_size  # the earliest token's window
        n = pages_of(L, lay.block_size)
        assert (lay.block_tables[s, :f] == 0).all()
        bt[s, : n - f] = lay.block_tables[s, f:n]
        ctx[s] = L - f * lay.block_size
        assert (bt[s, : n - f] != 0).all()
    return bt, ctx


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_layout_is_valid(name):
    lay = workload(name, seed=0)
    kw = {}
    if lay.group_seq_offsets is not None:
        kw = dict(group_seq_offsets=lay.group_seq_offsets, prefix_lens=lay.prefix_lens)
    bt, ctx = kept_tables(lay)
    assert oracle.check_block_tables(bt, ctx, lay.num_pages, lay.block_size, **kw) == []
    assert (lay.q_lens >= 1).all() and (lay.q_lens <= lay.context_lens).all()
    for s in range(lay.num_seqs):
        n = pages_of(lay.context_lens[s], lay.block_size)
        assert (lay.block_tables[s, :n] >= 0).all() and (lay.block_tables[s, n:] == -1).all()


def test_named_shapes():
    c1 = workload("tiny_f32")
    assert c1.context_lens.tolist() == [17, 64, 100, 255] and c1.num_pages == 64
    assert (c1.num_q_heads, c1.num_kv_heads, c1.head_dim, c1.dtype) == (8, 2, 64, "f32")
    assert len(c1.used_pages()) == 2 + 4 + 7 + 16
    c2 = workload("llama8b_decode")
    assert c2.num_seqs == 64 and c2.context_lens.min() >= 512 and c2.context_lens.max() <= 4096
    assert c2.num_pages == int(np.ceil(1.25 * len(c2.used_pages())))
    assert abs(c2.scale - 1 / np.sqrt(128)) < 1e-7
    c3 = workload("longtail_splitkv")
    assert c3.num_seqs == 256 and (c3.context_lens == 32768).sum() >= 1
    assert c3.context_lens.min() >= 16 and c3.gqa_ratio == 8
    c4 = workload("shared_prefix")
    assert c4.num_seqs == 1024 and c4.group_seq_offsets.tolist() == list(range(0, 1025, 64))
    assert (c4.prefix_lens == 2048).all()
    suf = c4.context_lens - 2048
    assert suf.min() >= 1 and suf.max() <= 512
    # the prefix is stored once: 16 groups x 128 pages, plus private suffix pages
    assert c4.num_pages == 16 * 128 + sum(pages_of(x, 16) for x in suf)
    c5 = workload("chunked_piggyback")
    assert c5.q_lens[:4].tolist() == [512] * 4 and (c5.q_lens[4:] == 1).all()
    assert (c5.context_lens[:4] - 512).tolist() == [0, 1024, 4096, 8192]
    assert c5.num_seqs == 260 and c5.context_lens[4:].min() >= 256 and c5.context_lens[4:].max() <= 8192


def test_values_are_deterministic_and_poisoned():
    lay = workload("tiny_f32")
    a = values_numpy(lay)
    b = values_numpy(lay)
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)
    q, k, v = a
    used = lay.used_pages()
    unused = np.setdiff1d(np.arange(lay.num_pages), used)
    assert np.isnan(k[unused]).all() and np.isnan(v[unused]).all()
    # tail rows of the 17-token sequence's second page are poisoned, its first row is not
    p = lay.block_tables[0, 1]
    assert not np.isnan(k[p, :, 0]).any() and np.isnan(k[p, :, 1:]).all()
    assert np.isfinite(q).all()
    c = values_numpy(lay, seed=1)
    assert not np.array_equal(c[0], q)


def test_window_layout_keeps_only_the_window_pages():
    lay = workload("longtail_window4096")
    assert lay.window == 4096 and lay.num_seqs == 256
    kept = sum(pages_of(L, 16) - max(0, int(L) - 4096) // 16 for L in lay.context_lens)
    assert lay.num_pages == 1 + kept  # page 0 is the placeholder target
    small = window_layout([5, 40, 100, 333], 50, num_q_heads=4, num_kv_heads=2, head_dim=64, dtype="f32", seed=3)
    bt, ctx = kept_tables(small)
    assert ctx.tolist() == [5, 40, 100 - 48, 333 - 272]
    q, k, v = values_numpy(small)
    assert np.isnan(k[0]).all() and np.isnan(v[0]).all()
    # the kept rows of every sequence are finite, from the window's first page on
    for s, L in enumerate(small.context_lens):
        f = max(0, int(L) - 50) // 16
        for t in range(f * 16, int(L)):
            assert np.isfinite(k[small.block_tables[s, t // 16], :, t % 16]).all()
