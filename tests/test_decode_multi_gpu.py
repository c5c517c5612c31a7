"""Parity of pa_decode_multi (HIP, through the C ABI) against the fp64
oracle: every sequence brings q_len new tokens, causal among them, folded
into the rows of the decode waves.  Cases span folds that fill a wave,
folds with idle rows, several passes, the shortest legal contexts
(L == q_len), and splits that leave some folded rows with no visible row in
a wave's part of a sequence."""

import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, oracle_full, out_to_f64, tables_to_device, to_device_values, to_host_values
from workloads import decode_layout, values_numpy, values_torch, workload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_multi(pa, lay, q, k, v, q_len, split_pages=0):
    bt, ctx = tables_to_device(lay)
    T, Hq, D = q.shape
    S = lay.num_seqs
    out = torch.empty_like(q)
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    total = int(((lay.context_lens + 15) // 16).sum())
    # workspace poisoned with NaN bytes: nothing may be read before it is written
    ws = torch.full((pa.decode_multi_workspace_size(S, q_len, lay.num_kv_heads, lay.gqa_ratio, D, total, split_pages),),
                    0xFF, dtype=torch.uint8, device="cuda")
    pa.decode_multi(out, q, k, v, bt, ctx, lay.context_lens, lay.scale, q_len, ws, lse_out=lse,
                    split_pages=split_pages)
    torch.cuda.synchronize()
    return out, lse


def multi_layout(ctx, q_len, hq, hkv, d, dtype, seed):
    return decode_layout(list(ctx), num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype, seed=seed,
                         value_std=1.0 if dtype == "f32" else 0.5, q_lens=[q_len] * len(ctx), name="multi_token")


def oracle_multi(lay, qh, kh, vh, seqs=None):
    return oracle.mixed_chunk(qh, kh, vh, lay.block_tables, lay.context_lens, lay.q_lens, lay.scale,
                              lay.num_kv_heads, 16, lay.dtype, seqs)


def ctx_for(q_len):
    # the shortest legal context, the page edges around it, ragged middles
    # and one long sequence that several waves share
    return sorted({q_len, q_len + 1, 15, 16, 17, 31, 33, 64, 65, 100, 257, 1000, 2100})


@pytest.mark.parametrize("dtype,d,hq,hkv", [("bf16", 128, 32, 8), ("f32", 64, 8, 2), ("bf16", 64, 16, 2),
                                            ("bf16", 128, 8, 8), ("bf16", 128, 64, 4), ("f32", 64, 32, 2)])
@pytest.mark.parametrize("q_len", [2, 3, 4, 5, 8])
def test_ragged_batches(gpu_lib, dtype, d, hq, hkv, q_len):
    ctx = [L for L in ctx_for(q_len) if L >= q_len]
    lay = multi_layout(ctx, q_len, hq, hkv, d, dtype, seed=q_len * 7 + hq)
    say(f"case multi q_len={q_len} {dtype} d={d} hq={hq} hkv={hkv}")
    qh, kh, vh = values_numpy(lay)
    q, k, v = to_device_values(lay, qh, kh, vh)
    ro, rl = oracle_multi(lay, qh, kh, vh)
    for sp in (0, 1, 3):
        out, lse = run_multi(gpu_lib, lay, q, k, v, q_len, split_pages=sp)
        assert_close(lay, out_to_f64(out), ro, f"q_len {q_len} split_pages={sp}")
        assert np.abs(lse.cpu().numpy() - rl).max() < (1e-4 if dtype == "f32" else 1e-3)


@pytest.mark.parametrize("q_len,hq,split", [(4, 32, 0), (4, 32, 5), (2, 32, 3), (3, 8, 0), (2, 128, 0)])
def test_many_shared_sequences(gpu_lib, q_len, hq, split):
    """64 sequences of 20..400 rows: every wave leaves partials of several
    sequences (both partial slots in use), so the partial rows of the
    folded passes fill the whole workspace carve-up."""
    ctx = [int(x) for x in np.random.default_rng(q_len * 31 + split).integers(20, 400, size=64)]
    lay = multi_layout(ctx, q_len, hq, 8, 128, "bf16", seed=split + 3)
    say(f"case multi shared q_len={q_len} hq={hq} split={split}")
    qh, kh, vh = values_numpy(lay)
    q, k, v = to_device_values(lay, qh, kh, vh)
    ro, rl = oracle_multi(lay, qh, kh, vh)
    out, lse = run_multi(gpu_lib, lay, q, k, v, q_len, split_pages=split)
    assert_close(lay, out_to_f64(out), ro, f"q_len {q_len} hq {hq} split {split}")
    assert np.abs(lse.cpu().numpy() - rl).max() < 1e-3


def test_causal_edge_is_exact(gpu_lib):
    """The newest row of each sequence (token q_len-1's own key) scores far
    above the rest for every query: token q_len-1 must return exactly that
    V row, every earlier token must not see it (their output equals the
    oracle's without the planted row's weight)."""
    q_len, hq, hkv = 4, 32, 8
    ctx = [4, 5, 17, 20, 64, 65, 300]
    lay = multi_layout(ctx, q_len, hq, hkv, 64, "f32", seed=5)
    qh, kh, vh = values_numpy(lay)
    G = hq // hkv
    for s, L in enumerate(ctx):
        p = lay.block_tables[s, (L - 1) // 16]
        for g in range(hkv):
            j = (s * 8 + g) % 64
            kh[p, g, (L - 1) % 16, :] = 0.0
            kh[p, g, (L - 1) % 16, j] = 64.0
            for t in range(q_len):
                qh[s * q_len + t, g * G:(g + 1) * G, j] = 64.0
    ro, _ = oracle_multi(lay, qh, kh, vh)
    q, k, v = to_device_values(lay, qh, kh, vh)
    for sp in (0, 1):
        out, _ = run_multi(gpu_lib, lay, q, k, v, q_len, split_pages=sp)
        got = out_to_f64(out)
        assert_close(lay, got, ro, f"causal edge split {sp}")
        for s, L in enumerate(ctx):
            p = lay.block_tables[s, (L - 1) // 16]
            for g in range(hkv):
                want = vh[p, g, (L - 1) % 16].astype(np.float64)
                last = got[s * q_len + q_len - 1, g * G:(g + 1) * G]
                assert np.abs(last - want).max() < 1e-5, f"seq {s}: newest token does not pick its own row"


def test_q_len_one_is_decode(gpu_lib):
    """q_len 1 takes the plain decode path: bit for bit pa_decode."""
    lay = multi_layout([1, 17, 100, 1000, 3000], 1, 32, 8, 128, "bf16", seed=2)
    qh, kh, vh = values_numpy(lay)
    q, k, v = to_device_values(lay, qh, kh, vh)
    out_m, lse_m = run_multi(gpu_lib, lay, q, k, v, 1)
    bt, ctx = tables_to_device(lay)
    out = torch.empty_like(q)
    lse = torch.empty_like(lse_m)
    total = int(((lay.context_lens + 15) // 16).sum())
    ws = torch.empty(gpu_lib.decode_workspace_size(lay.num_seqs, 8, 4, 128, total, 0), dtype=torch.uint8,
                     device="cuda")
    gpu_lib.decode(out, q, k, v, bt, ctx, lay.context_lens, lay.scale, ws, lse_out=lse)
    torch.cuda.synchronize()
    assert torch.equal(out_m.view(torch.int16), out.view(torch.int16)) and torch.equal(lse_m, lse)


def test_agrees_with_mixed_chunk(gpu_lib):
    """The same batch through pa_mixed_chunk (every segment a 4-token
    chunk): both within the bf16 bar of each other."""
    lay = multi_layout([4, 40, 333, 1200], 4, 32, 8, 128, "bf16", seed=9)
    qh, kh, vh = values_numpy(lay)
    q, k, v = to_device_values(lay, qh, kh, vh)
    out_m, _ = run_multi(gpu_lib, lay, q, k, v, 4)
    bt, ctx = tables_to_device(lay)
    cu = torch.from_numpy(lay.cu_q_lens.astype(np.int32)).cuda()
    out_c = torch.empty_like(q)
    total = int(((lay.context_lens + 15) // 16).sum())
    ws = torch.empty(gpu_lib.mixed_chunk_workspace_size(lay.num_tokens, lay.num_seqs, 8, 4, 128, total),
                     dtype=torch.uint8, device="cuda")
    gpu_lib.mixed_chunk(out_c, q, k, v, bt, cu, lay.cu_q_lens, ctx, lay.context_lens, lay.scale, ws)
    torch.cuda.synchronize()
    assert_close(lay, out_to_f64(out_m), out_to_f64(out_c), "decode_multi vs mixed_chunk")


def test_llama8b_multitoken4_full(gpu_lib):
    """The full-size speculative-decoding step (64 sequences x 4 tokens,
    Llama-8B heads), in the launch configuration the benchmark times: every
    token against the oracle."""
    lay = workload("llama8b_multitoken4")
    say("case llama8b_multitoken4 seed 0 (device values, every token)")
    q, k, v = values_torch(lay, "cuda")
    out, lse = run_multi(gpu_lib, lay, q, k, v, 4)
    assert torch.isfinite(out.float()).all()
    ro, rl = oracle_full(lay, q, k, v)
    assert_close(lay, out_to_f64(out), ro, "llama8b_multitoken4, every token")
    assert np.abs(lse.cpu().numpy() - rl).max() < 1e-3


def test_context_shorter_than_q_len_is_rejected(gpu_lib):
    lay = multi_layout([10, 20], 4, 8, 2, 64, "f32", seed=0)
    qh, kh, vh = values_numpy(lay)
    q, k, v = to_device_values(lay, qh, kh, vh)
    bt, ctx = tables_to_device(lay)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    bad = np.array([3, 20], dtype=np.int32)
    with pytest.raises(gpu_lib.PAError) as e:
        gpu_lib.decode_multi(torch.empty_like(q), q, k, v, bt, ctx, bad, lay.scale, 4, ws)
    assert e.value.code == gpu_lib.PA_EINVAL
