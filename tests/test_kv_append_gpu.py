"""Parity of pa_kv_append (HIP, through the C ABI) against the oracle: the
pools after the call must equal the oracle's bit for bit; then attention
over the appended pools must match the attention oracle."""

import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_util import LSE_TOL, assert_close, out_to_f64, to_device_values, to_host_values
from workloads import decode_layout, mixed_layout, new_rows_numpy, new_rows_torch, values_numpy, values_torch, workload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def conv(lay, a):
    if lay.dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def run_append(pa, lay, kp, vp, kn, vn, bt_host=None):
    bt = torch.from_numpy(lay.block_tables if bt_host is None else bt_host).cuda()
    cu = torch.from_numpy(lay.cu_q_lens.astype(np.int32)).cuda()
    ctx = torch.from_numpy(lay.context_lens).cuda()
    pa.kv_append(kp, vp, kn, vn, bt, cu, lay.cu_q_lens, ctx, lay.context_lens)
    torch.cuda.synchronize()


def bits(lay, t):
    """Host copy of a device tensor as raw bits (NaN-safe comparison)."""
    h = to_host_values(lay, t)
    return h.view(np.uint32) if h.dtype == np.float32 else h


def check_whole_pools(pa, lay, bt_host=None):
    kh, vh = values_numpy(lay)[1:]
    kn, vn = new_rows_numpy(lay)
    bt = lay.block_tables if bt_host is None else bt_host
    want_k, want_v = oracle.kv_append(kh, vh, kn, vn, bt, lay.context_lens, lay.q_lens, lay.block_size)
    kp, vp = conv(lay, kh), conv(lay, vh)
    run_append(pa, lay, kp, vp, conv(lay, kn), conv(lay, vn), bt_host)
    for name, got, want in (("k_pool", kp, want_k), ("v_pool", vp, want_v)):
        w = want.view(np.uint32) if want.dtype == np.float32 else want
        assert np.array_equal(bits(lay, got), w), f"{lay.name}: {name} differs from the oracle"


def test_small_f32_whole_pools(gpu_lib):
    say("case append f32 D=64 Hkv=2 chunks [0, 5, 33] x 20 + 5 decode")
    lay = mixed_layout(chunk_prefixes=[0, 5, 33], chunk_len=20, decode_ctx=[1, 16, 17, 40, 100], num_q_heads=4,
                       num_kv_heads=2, head_dim=64, dtype="f32", name="append_f32")
    check_whole_pools(gpu_lib, lay)


def test_small_bf16_llama_heads_whole_pools(gpu_lib):
    say("case append bf16 D=128 Hkv=8 chunks [0, 16, 100] x 37 + 7 decode")
    lay = mixed_layout(chunk_prefixes=[0, 16, 100], chunk_len=37, decode_ctx=[1, 2, 15, 16, 17, 255, 513],
                       num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16", name="append_bf16")
    check_whole_pools(gpu_lib, lay)


def test_many_segments_and_empty_ones(gpu_lib):
    # More segments than one coarse search step covers (S > 64), some adding
    # no token at all, whole-sequence appends (q_len = context) among them.
    say("case append bf16 S=300 with empty segments")
    rng = np.random.default_rng(11)
    ctx = rng.integers(1, 90, size=300).astype(np.int32)
    ql = np.array([0 if i % 7 == 3 else (int(L) if i % 11 == 5 else min(int(L), 1 + i % 4))
                   for i, L in enumerate(ctx)], dtype=np.int32)
    lay = decode_layout(ctx, num_q_heads=8, num_kv_heads=4, head_dim=128, dtype="bf16", q_lens=ql,
                        name="append_many")
    check_whole_pools(gpu_lib, lay)


def test_entries_outside_the_pool_are_not_written(gpu_lib):
    say("case append bf16 with -1 and out-of-pool table entries")
    lay = mixed_layout(chunk_prefixes=[0, 40], chunk_len=30, decode_ctx=[5, 33, 64, 65], num_q_heads=8,
                       num_kv_heads=2, head_dim=128, dtype="bf16", name="append_invalid")
    bt = lay.block_tables.copy()
    for s, v in ((0, -1), (1, lay.num_pages), (3, 1 << 30)):
        L = int(lay.context_lens[s])
        bt[s, (L - 1) // 16] = v  # the page of the segment's last new row
    check_whole_pools(gpu_lib, lay, bt)


def test_chunked_piggyback_size(gpu_lib):
    # Full size (2,304 new tokens, 8 kv-heads, ~2.2 GB pools drawn on the
    # device): the pages the new rows land in are checked against the
    # oracle bit for bit; every other row of both pools must keep its bits.
    lay = workload("chunked_piggyback")
    say("case append chunked_piggyback full size")
    _, kp, vp = values_torch(lay, "cuda")
    kn, vn = new_rows_torch(lay, "cuda")
    touched = []
    for s in range(lay.num_seqs):
        L, n = int(lay.context_lens[s]), int(lay.q_lens[s])
        for row in range(L - n, L):
            touched.append((int(lay.block_tables[s, row // 16]), row % 16))
    pages = np.unique(np.array([p for p, _ in touched], dtype=np.int64))
    idx = torch.from_numpy(pages).cuda()
    k_before, v_before = kp.clone(), vp.clone()
    run_append(gpu_lib, lay, kp, vp, kn, vn)
    # the oracle on the touched pages only (renumbered 0..n-1)
    remap = {int(p): i for i, p in enumerate(pages)}
    bt_sub = np.vectorize(lambda p: remap.get(int(p), -1))(lay.block_tables).astype(np.int32)
    want_k, want_v = oracle.kv_append(to_host_values(lay, k_before.index_select(0, idx)),
                                      to_host_values(lay, v_before.index_select(0, idx)),
                                      to_host_values(lay, kn), to_host_values(lay, vn), bt_sub, lay.context_lens,
                                      lay.q_lens, 16)
    assert np.array_equal(bits(lay, kp.index_select(0, idx)), want_k)
    assert np.array_equal(bits(lay, vp.index_select(0, idx)), want_v)
    mask = torch.zeros((lay.num_pages, 16), dtype=torch.bool, device="cuda")
    tp = torch.tensor([p for p, _ in touched], device="cuda")
    ts = torch.tensor([r for _, r in touched], device="cuda")
    mask[tp, ts] = True
    keep = ~mask
    for got, before in ((kp, k_before), (vp, v_before)):
        g = got.view(torch.int16).transpose(1, 2)[keep]
        b = before.view(torch.int16).transpose(1, 2)[keep]
        assert torch.equal(g, b), "a row that no new token maps to changed"


def test_whole_prefill_write(gpu_lib):
    # The Llama-shaped batch with every row new (148,663 tokens, 1.2 GB
    # moved): the rows read back through each table, in order, must be the
    # new rows bit for bit (the oracle's definition, checked as a property
    # at this size), and the rows past each sequence's end keep their bits.
    lay = workload("llama8b_prefill_append")
    say("case append llama8b_prefill_append full size")
    _, kp, vp = values_torch(lay, "cuda")
    kn, vn = new_rows_torch(lay, "cuda")
    k_before, v_before = kp.clone(), vp.clone()
    run_append(gpu_lib, lay, kp, vp, kn, vn)
    rows_page, rows_slot = [], []
    for s in range(lay.num_seqs):
        t = np.arange(int(lay.context_lens[s]))
        rows_page.append(lay.block_tables[s, t // 16])
        rows_slot.append(t % 16)
    rp = torch.from_numpy(np.concatenate(rows_page).astype(np.int64)).cuda()
    rs = torch.from_numpy(np.concatenate(rows_slot).astype(np.int64)).cuda()
    for got, new, before in ((kp, kn, k_before), (vp, vn, v_before)):
        back = got.view(torch.int16)[rp, :, rs, :]  # [T, Hkv, D] in token order
        assert torch.equal(back, new.view(torch.int16)), "a row read back differs from the new row"
        mask = torch.ones((lay.num_pages, 16), dtype=torch.bool, device="cuda")
        mask[rp, rs] = False
        assert torch.equal(got.view(torch.int16).transpose(1, 2)[mask],
                           before.view(torch.int16).transpose(1, 2)[mask]), "a row no token maps to changed"


def test_append_then_mixed_attention(gpu_lib):
    # End to end: the rows of this step's tokens start as NaN in the pools,
    # pa_kv_append writes them, then pa_mixed_chunk attends over the pools;
    # the oracle does the same with oracle.kv_append + oracle.mixed_chunk.
    say("case append then pa_mixed_chunk, bf16 Llama heads")
    lay = mixed_layout(chunk_prefixes=[0, 48], chunk_len=64, decode_ctx=[1, 17, 200, 333], num_q_heads=32,
                       num_kv_heads=8, head_dim=128, dtype="bf16", name="append_attend")
    qh, kh, vh = values_numpy(lay)
    for s in range(lay.num_seqs):
        L, n = int(lay.context_lens[s]), int(lay.q_lens[s])
        for row in range(L - n, L):
            kh[lay.block_tables[s, row // 16], :, row % 16, :] = 0x7FC0
            vh[lay.block_tables[s, row // 16], :, row % 16, :] = 0x7FC0
    kn, vn = new_rows_numpy(lay)
    ko, vo = oracle.kv_append(kh, vh, kn, vn, lay.block_tables, lay.context_lens, lay.q_lens, 16)
    ro, rl = oracle.mixed_chunk(qh, ko, vo, lay.block_tables, lay.context_lens, lay.q_lens, lay.scale,
                                lay.num_kv_heads, 16, "bf16")
    q, kp, vp = to_device_values(lay, qh, kh, vh)
    run_append(gpu_lib, lay, kp, vp, conv(lay, kn), conv(lay, vn))
    T, Hq, D = q.shape
    bt = torch.from_numpy(lay.block_tables).cuda()
    ctx = torch.from_numpy(lay.context_lens).cuda()
    cu = torch.from_numpy(lay.cu_q_lens.astype(np.int32)).cuda()
    out = torch.empty_like(q)
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    total = int(((lay.context_lens + 15) // 16).sum())
    ws = torch.empty(gpu_lib.mixed_chunk_workspace_size(T, lay.num_seqs, 8, 4, D, total), dtype=torch.uint8,
                     device="cuda")
    gpu_lib.mixed_chunk(out, q, kp, vp, bt, cu, lay.cu_q_lens, ctx, lay.context_lens, lay.scale, ws, lse_out=lse)
    torch.cuda.synchronize()
    assert_close(lay, out_to_f64(out), ro, "append then mixed attention")
    assert np.abs(lse.cpu().numpy() - rl).max() < LSE_TOL
