"""The seeded input generator: determinism and layout sanity for every
named workload (host only)."""

import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, pages_of, values_numpy, workload


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_layout_is_valid(name):
    lay = workload(name, seed=0)
    kw = {}
    if lay.group_seq_offsets is not None:
        kw = dict(group_seq_offsets=lay.group_seq_offsets, prefix_lens=lay.prefix_lens)
    assert oracle.check_block_tables(lay.block_tables, lay.context_lens, lay.num_pages, lay.block_size, **kw) == []
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
