"""The sharded oracle runner (oracle.parallel) gives the direct oracle's
results bit for bit: it only splits a batch into (sequence, kv-head) units
and relabels each unit's pages 0..n-1, which the oracle pins show changes
nothing."""

import numpy as np
import pytest

import oracle
from oracle import parallel
from workloads import decode_layout, fp8_values_numpy, mixed_layout, values_numpy, window_layout


def host_fetch(lay, q, k, v, ks=None, vs=None):
    cu = lay.cu_q_lens

    def fetch(s):
        L = int(lay.context_lens[s])
        W = lay.window
        lo = L - int(lay.q_lens[s]) + 1 - W if W is not None else 0  # the earliest row a token sees
        first = lo // 16 if lo > 0 else 0
        pages = lay.block_tables[s, first:(L + 15) // 16]
        got = (q[cu[s]:cu[s + 1]], k[pages], v[pages])
        return got + (ks[pages], vs[pages]) if ks is not None else got

    return fetch


def run_all(lay, fetch, **kw):
    T = lay.num_tokens
    out = np.full((T, lay.num_q_heads, lay.head_dim), np.nan)
    lse = np.full((T, lay.num_q_heads), np.nan)
    cu = lay.cu_q_lens
    seen = []
    for s, o, l in parallel.batch_attention(fetch, range(lay.num_seqs), lay.context_lens, lay.q_lens,
                                            lay.num_kv_heads, lay.scale, lay.dtype, **kw):
        out[cu[s]:cu[s + 1]], lse[cu[s]:cu[s + 1]] = o, l
        seen.append(s)
    assert sorted(seen) == list(range(lay.num_seqs))
    return out, lse


@pytest.fixture(scope="module", params=[0, 2], ids=["in-process", "two-workers"])
def pool(request):
    if request.param:
        parallel.start_pool(request.param)
    yield request.param
    parallel.stop_pool()


def test_mixed_batch_bit_identical(pool):
    lay = mixed_layout(chunk_prefixes=[0, 37], chunk_len=9, decode_ctx=[5, 70, 17], num_q_heads=8, num_kv_heads=2,
                       head_dim=64, dtype="f32", seed=3)
    q, k, v = values_numpy(lay)
    want = oracle.mixed_chunk(q, k, v, lay.block_tables, lay.context_lens, lay.q_lens, lay.scale, 2, 16, "f32")
    got = run_all(lay, host_fetch(lay, q, k, v))
    for g, w in zip(got, want):
        assert np.array_equal(g, w)


def test_bf16_decode_bit_identical(pool):
    lay = decode_layout([1, 16, 33, 300], num_q_heads=16, num_kv_heads=4, head_dim=64, dtype="bf16", seed=1,
                        pool_factor=1.5)
    q, k, v = values_numpy(lay)
    want = oracle.decode(q, k, v, lay.block_tables, lay.context_lens, lay.scale, 4, 16, "bf16")
    got = run_all(lay, host_fetch(lay, q, k, v))
    for g, w in zip(got, want):
        assert np.array_equal(g, w)


def test_window_bit_identical(pool):
    lay = window_layout([10, 100, 257], 40, num_q_heads=8, num_kv_heads=2, head_dim=64, dtype="f32", seed=2)
    q, k, v = values_numpy(lay)
    want = oracle.decode_window(q, k, v, lay.block_tables, lay.context_lens, 40, lay.scale, 2, 16, "f32")
    got = run_all(lay, host_fetch(lay, q, k, v), window=40)
    for g, w in zip(got, want):
        assert np.array_equal(g, w)


def test_multi_token_window_bit_identical(pool):
    lay = window_layout([4, 37, 100, 257], 40, num_q_heads=8, num_kv_heads=2, head_dim=64, dtype="f32", seed=4,
                        q_len=4)
    q, k, v = values_numpy(lay)
    want = oracle.decode_multi_window(q, k, v, lay.block_tables, lay.context_lens, 4, 40, lay.scale, 2, 16, "f32")
    got = run_all(lay, host_fetch(lay, q, k, v), window=40)
    for g, w in zip(got, want):
        assert np.array_equal(g, w)


def test_fp8_bit_identical(pool):
    lay = decode_layout([3, 40, 129], num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16", seed=6)
    lay.kv_dtype = "fp8"
    q, kc, ks, vc, vs = fp8_values_numpy(lay)
    want = oracle.decode_fp8(q, kc, ks, vc, vs, lay.block_tables, lay.context_lens, lay.scale, 2, 16, "bf16")
    got = run_all(lay, host_fetch(lay, q, kc, vc, ks, vs), fp8_kv=True)
    for g, w in zip(got, want):
        assert np.array_equal(g, w)
