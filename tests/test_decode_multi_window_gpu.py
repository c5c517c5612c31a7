"""Parity of pa_decode_multi_window (HIP, through the C ABI) against the fp64
oracle (oracle.decode_multi_window): q_len new tokens per sequence, token i
at position p = L - q_len + i seeing rows max(0, p + 1 - window) .. p, the
tokens folded into the decode waves' rows.  Tables hold placeholders (the
NaN page 0) before the earliest token's window, so a read of one shows up
as NaN.  Cases: ragged batches on both stream kernels (float32 and 1-2
q-heads per kv-head on the vector kernel, 4-16 bf16 rows on the matrix
cores), window edges planted so that a row is inside some tokens' windows
and outside the next token's, the reductions to pa_decode_window (q_len 1)
and pa_decode_multi (a window past every context), and the full Llama-shaped
4-token step over a 1024-token window."""

import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_util import LSE_TOL, assert_close, oracle_full, out_to_f64, tables_to_device, to_device_values
from workloads import values_numpy, values_torch, window_layout, workload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_mw(pa, lay, q, k, v, q_len, window, split_pages=0):
    bt, ctx = tables_to_device(lay)
    T, Hq, D = q.shape
    S = lay.num_seqs
    out = torch.empty_like(q)
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    total = int(((lay.context_lens + 15) // 16).sum())
    # workspace poisoned with NaN bytes: nothing may be read before it is written
    ws = torch.full((pa.decode_multi_workspace_size(S, q_len, lay.num_kv_heads, lay.gqa_ratio, D, total, split_pages),),
                    0xFF, dtype=torch.uint8, device="cuda")
    pa.decode_multi_window(out, q, k, v, bt, ctx, lay.context_lens, lay.scale, q_len, window, ws, lse_out=lse,
                           split_pages=split_pages)
    torch.cuda.synchronize()
    return out, lse


def mw_layout(ctx, q_len, window, hq, hkv, d, dtype, seed):
    return window_layout(list(ctx), window, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype, seed=seed,
                         value_std=1.0 if dtype == "f32" else 0.5, q_len=q_len, name="multi_window")


def oracle_mw(lay, qh, kh, vh, q_len):
    return oracle.decode_multi_window(qh, kh, vh, lay.block_tables, lay.context_lens, q_len, lay.window, lay.scale,
                                      lay.num_kv_heads, 16, lay.dtype)


def ctx_for(q_len):
    return sorted({q_len, q_len + 1, 15, 16, 17, 31, 33, 64, 65, 100, 257, 1000, 2100})


@pytest.mark.parametrize("dtype,d,hq,hkv", [("bf16", 128, 32, 8), ("f32", 64, 8, 2), ("bf16", 64, 16, 2),
                                            ("bf16", 128, 8, 8), ("bf16", 128, 64, 4)])
@pytest.mark.parametrize("q_len,window", [(2, 1), (3, 16), (4, 37), (5, 100), (4, 700)])
def test_ragged_batches(gpu_lib, dtype, d, hq, hkv, q_len, window):
    ctx = [L for L in ctx_for(q_len) if L >= q_len]
    lay = mw_layout(ctx, q_len, window, hq, hkv, d, dtype, seed=q_len * 11 + window + hq)
    say(f"case multi_window q_len={q_len} window={window} {dtype} d={d} hq={hq} hkv={hkv}")
    qh, kh, vh = values_numpy(lay)
    q, k, v = to_device_values(lay, qh, kh, vh)
    ro, rl = oracle_mw(lay, qh, kh, vh, q_len)
    for sp in (0, 1, 3):
        out, lse = run_mw(gpu_lib, lay, q, k, v, q_len, window, split_pages=sp)
        assert torch.isfinite(out.float()).all(), "a placeholder row reached the result"
        assert_close(lay, out_to_f64(out), ro, f"q_len {q_len} window {window} split_pages={sp}")
        assert np.abs(lse.cpu().numpy() - rl).max() < (1e-4 if dtype == "f32" else LSE_TOL)


@pytest.mark.parametrize("dtype,d,hq,hkv", [("f32", 64, 8, 2), ("bf16", 128, 32, 8), ("bf16", 128, 128, 8)])
def test_window_edges_are_exact(gpu_lib, dtype, d, hq, hkv):
    """Row r = L - q_len + 2 - window scores far above the rest for every
    query: it is the first row of token 1's window, inside token 0's and
    outside token 2's and later.  Tokens 0 and 1 must return exactly its V
    row; later tokens must not see it (their outputs match the oracle, which
    then gives the row no weight)."""
    q_len, window = 4, 40
    ctx = [44, 45, 60, 64, 65, 100, 300]
    lay = mw_layout(ctx, q_len, window, hq, hkv, d, dtype, seed=13)
    qh, kh, vh = values_numpy(lay)
    G = hq // hkv
    hot = 64.0 if dtype == "f32" else 48.0
    for s, L in enumerate(ctx):
        r = L - q_len + 2 - window
        p = lay.block_tables[s, r // 16]
        for g in range(hkv):
            j = (s * 5 + g) % d
            if dtype == "f32":
                kh[p, g, r % 16, :] = 0.0
                kh[p, g, r % 16, j] = hot
                for t in range(q_len):
                    qh[s * q_len + t, g * G:(g + 1) * G, j] = hot
            else:
                from workloads import bf16_bits_from_f32

                row = np.zeros(d, np.float32)
                row[j] = hot
                kh[p, g, r % 16, :] = bf16_bits_from_f32(row)
                for t in range(q_len):
                    qh[s * q_len + t, g * G:(g + 1) * G, j] = bf16_bits_from_f32(np.array([hot], np.float32))[0]
    ro, _ = oracle_mw(lay, qh, kh, vh, q_len)
    q, k, v = to_device_values(lay, qh, kh, vh)
    for sp in (0, 1):
        out, _ = run_mw(gpu_lib, lay, q, k, v, q_len, window, split_pages=sp)
        got = out_to_f64(out)
        assert_close(lay, got, ro, f"window edges split {sp}")
        for s, L in enumerate(ctx):
            r = L - q_len + 2 - window
            p = lay.block_tables[s, r // 16]
            for g in range(hkv):
                if dtype == "f32":
                    want = vh[p, g, r % 16].astype(np.float64)
                else:
                    want = oracle.stored_to_f64(vh[p, g, r % 16], "bf16")
                for t in (0, 1):
                    row = got[s * q_len + t, g * G:(g + 1) * G]
                    assert np.abs(row - want).max() == 0.0, f"seq {s} token {t}: not exactly the hot row"


def test_q_len_one_is_window_decode(gpu_lib):
    """q_len 1 is pa_decode_window, bit for bit."""
    lay = mw_layout([1, 17, 100, 1000, 3000], 1, 64, 32, 8, 128, "bf16", seed=2)
    qh, kh, vh = values_numpy(lay)
    q, k, v = to_device_values(lay, qh, kh, vh)
    out_m, lse_m = run_mw(gpu_lib, lay, q, k, v, 1, 64)
    bt, ctx = tables_to_device(lay)
    out = torch.empty_like(q)
    lse = torch.empty_like(lse_m)
    total = int(((lay.context_lens + 15) // 16).sum())
    ws = torch.empty(gpu_lib.decode_workspace_size(lay.num_seqs, 8, 4, 128, total, 0), dtype=torch.uint8,
                     device="cuda")
    gpu_lib.decode_window(out, q, k, v, bt, ctx, lay.context_lens, lay.scale, 64, ws, lse_out=lse)
    torch.cuda.synchronize()
    assert torch.equal(out_m.view(torch.int16), out.view(torch.int16)) and torch.equal(lse_m, lse)


@pytest.mark.parametrize("q_len", [2, 4])
def test_window_past_every_context_is_multi(gpu_lib, q_len):
    """A window longer than every context: pa_decode_multi, bit for bit."""
    ctx = [q_len, 17, 100, 1000, 2500]
    lay = mw_layout(ctx, q_len, 4096, 32, 8, 128, "bf16", seed=3)
    qh, kh, vh = values_numpy(lay)
    q, k, v = to_device_values(lay, qh, kh, vh)
    out_w, lse_w = run_mw(gpu_lib, lay, q, k, v, q_len, 4096)
    bt, ctx_d = tables_to_device(lay)
    out = torch.empty_like(q)
    lse = torch.empty_like(lse_w)
    total = int(((lay.context_lens + 15) // 16).sum())
    ws = torch.empty(gpu_lib.decode_multi_workspace_size(lay.num_seqs, q_len, 8, 4, 128, total, 0),
                     dtype=torch.uint8, device="cuda")
    gpu_lib.decode_multi(out, q, k, v, bt, ctx_d, lay.context_lens, lay.scale, q_len, ws, lse_out=lse)
    torch.cuda.synchronize()
    assert torch.equal(out_w.view(torch.int16), out.view(torch.int16)) and torch.equal(lse_w, lse)


def test_llama8b_multitoken4_window1024_full(gpu_lib):
    """The Llama-shaped 4-token step over a 1024-token window, in the launch
    configuration the benchmark times: every token against the oracle."""
    lay = workload("llama8b_multitoken4_window1024")
    say("case llama8b_multitoken4_window1024 seed 0 (device values, every token)")
    q, k, v = values_torch(lay, "cuda")
    out, lse = run_mw(gpu_lib, lay, q, k, v, 4, lay.window)
    assert torch.isfinite(out.float()).all()
    ro, rl = oracle_full(lay, q, k, v)
    assert_close(lay, out_to_f64(out), ro, "llama8b_multitoken4_window1024, every token")
    assert np.abs(lse.cpu().numpy() - rl).max() < LSE_TOL


def test_window_must_be_positive(gpu_lib):
    lay = mw_layout([10, 20], 2, 5, 8, 2, 64, "f32", seed=0)
    qh, kh, vh = values_numpy(lay)
    q, k, v = to_device_values(lay, qh, kh, vh)
    bt, ctx = tables_to_device(lay)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(gpu_lib.PAError) as e:
        gpu_lib.decode_multi_window(torch.empty_like(q), q, k, v, bt, ctx, lay.context_lens, lay.scale, 2, 0, ws)
    assert e.value.code == gpu_lib.PA_EINVAL
