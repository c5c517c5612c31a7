"""Byte accounting used by the benchmark, pinned to the worked example the
tokenspeed deep-dive prints (section 7-2)."""

import json
import os

import numpy as np

from paged_kv_decode_02_amd import roofline

HERE = os.path.dirname(os.path.abspath(__file__))


def test_kv_bytes_worked_example():
    g = json.load(open(os.path.join(HERE, "golden", "kv_bytes_llama8b.json")))
    got = roofline.kv_cache_bytes(g["layers"], g["kv_heads"], g["head_dim"], g["tokens"], g["bytes_per_element"])
    assert got == g["kv_bytes"] == 512 * 2**20


def test_decode_bytes_counts_kv_once_per_kv_head():
    b = roofline.decode_bytes([4096], num_q_heads=32, num_kv_heads=8, head_dim=128, elem_bytes=2)
    assert b["kv"] * 32 == 536870912  # one layer of the worked example
    b4 = roofline.decode_bytes([4096], num_q_heads=8, num_kv_heads=8, head_dim=128, elem_bytes=2)
    assert b4["kv"] == b["kv"]  # GQA does not multiply KV traffic
    assert b["tables"] == 4 * 256 + 4
    assert b["q_out"] == 2 * 32 * 128 * 2
    assert roofline.decode_flops(np.array([10, 20]), 32, 128) == 4 * 128 * 32 * 30


def test_cascade_accounting_on_the_shared_prefix_workload():
    from workloads import workload

    lay = workload("shared_prefix")
    f = roofline.prefix_flops(lay.group_seq_offsets, lay.prefix_lens, lay.num_q_heads, lay.head_dim)
    assert f == 4 * 128 * 32 * 64 * 2048 * 16  # 34.36 GFLOP
    b = roofline.cascade_bytes(lay.context_lens, lay.group_seq_offsets, lay.prefix_lens, 32, 8, 128, 2)
    assert b["prefix_kv"] == 16 * 2048 * 4096
    naive = roofline.decode_bytes(lay.context_lens, 32, 8, 128, 2)
    assert naive["kv"] - b["kv"] == 63 * 16 * 2048 * 4096  # the prefix is read once per group, not per member


def test_mixed_accounting_on_the_chunked_piggyback_workload():
    from workloads import workload

    lay = workload("chunked_piggyback")
    f = roofline.chunk_flops(lay.context_lens, lay.q_lens, 32, 128)
    # token i of a 512-token chunk after prefix p sees p + i + 1 keys
    want = 4 * 128 * 32 * sum(512 * p + 512 * 513 // 2 for p in (0, 1024, 4096, 8192))
    assert f == want  # 120.27 GFLOP
    assert abs(f / 1e9 - 120.27) < 0.01
    # brute-force the causal count on one small segment
    assert roofline.chunk_flops([7], [3], 1, 1) == 4 * (5 + 6 + 7)
    assert roofline.chunk_flops([9], [1], 1, 1) == 0  # decode tokens are not chunk work
    b = roofline.mixed_bytes(lay.context_lens, lay.q_lens, 32, 8, 128, 2)
    assert b["kv"] == 2 * 8 * 128 * 2 * int(lay.context_lens.sum())
    assert b["decode_kv"] == 2 * 8 * 128 * 2 * int(lay.context_lens[4:].sum())
    assert b["q_out"] == 2 * 2304 * 32 * 128 * 2


def test_fp8_decode_bytes():
    b = roofline.decode_fp8_bytes([4096], num_q_heads=32, num_kv_heads=8, head_dim=128)
    bf = roofline.decode_bytes([4096], num_q_heads=32, num_kv_heads=8, head_dim=128, elem_bytes=2)
    assert 2 * b["kv"] == bf["kv"]  # one byte per element instead of two
    assert b["scales"] == 2 * 8 * 4096 * 4  # a float32 scale per K row and per V row
    assert b["q_out"] == bf["q_out"] and b["tables"] == bf["tables"]


def test_fp8_bytes_count_every_new_token():
    one = roofline.decode_fp8_bytes([100, 2000], 32, 8, 128)
    four = roofline.decode_fp8_bytes([100, 2000], 32, 8, 128, q_len=4)
    assert four["q_out"] == 4 * one["q_out"]
    assert four["total"] - one["total"] == 3 * one["q_out"]


def test_fp8_cascade_and_mixed_bytes():
    """Over an fp8 cache the cascade and mixed byte counts take one byte per
    K/V element plus a float32 scale per K row and per V row, in the same
    places the bf16 counts take two bytes per element."""
    from workloads import workload

    lay = workload("shared_prefix")
    b = roofline.cascade_bytes(lay.context_lens, lay.group_seq_offsets, lay.prefix_lens, 32, 8, 128, 2)
    f = roofline.cascade_bytes(lay.context_lens, lay.group_seq_offsets, lay.prefix_lens, 32, 8, 128, 2, kv_fp8=True)
    tokens = b["kv"] // (2 * 8 * 128 * 2)  # K/V rows read: each prefix once, every suffix
    assert f["kv"] == 2 * 8 * 128 * tokens + 2 * 8 * tokens * 4
    assert f["prefix_kv"] == 16 * 2048 * (2 * 8 * 128 + 2 * 8 * 4)
    assert f["q_out"] == b["q_out"] and f["tables"] == b["tables"]
    lay = workload("chunked_piggyback")
    b = roofline.mixed_bytes(lay.context_lens, lay.q_lens, 32, 8, 128, 2)
    f = roofline.mixed_bytes(lay.context_lens, lay.q_lens, 32, 8, 128, 2, kv_fp8=True)
    n = int(lay.context_lens.sum())
    assert f["kv"] == 2 * 8 * 128 * n + 2 * 8 * n * 4
    assert f["decode_kv"] == roofline.decode_fp8_bytes(lay.context_lens[4:], 32, 8, 128)["kv"] + \
        roofline.decode_fp8_bytes(lay.context_lens[4:], 32, 8, 128)["scales"]
    assert f["q_out"] == b["q_out"] and f["tables"] == b["tables"]
