"""Parity of pa_decode_window (HIP, through the C ABI) against the fp64
oracle: each query sees only the last `window` rows of its sequence, and the
placeholder table entries before the window (naming a NaN page) are never
read."""

import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, oracle_full, out_to_f64, tables_to_device, to_device_values, to_host_values
from workloads import bf16_bits_from_f32, values_numpy, values_torch, window_layout, workload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_window(pa, lay, q, k, v, split_pages=0):
    bt, ctx = tables_to_device(lay)
    S, Hq, D = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((S, Hq), dtype=torch.float32, device="cuda")
    total_pages = int(sum((int(L) + 15) // 16 for L in lay.context_lens))
    ws = torch.empty(pa.decode_workspace_size(S, lay.num_kv_heads, lay.gqa_ratio, D, total_pages, split_pages),
                     dtype=torch.uint8, device="cuda")
    pa.decode_window(out, q, k, v, bt, ctx, lay.context_lens, lay.scale, lay.window, ws, lse_out=lse,
                     split_pages=split_pages)
    torch.cuda.synchronize()
    return out, lse


def oracle_window(lay, q, k, v, seqs=None):
    return oracle.decode_window(q, k, v, lay.block_tables, lay.context_lens, lay.window, lay.scale,
                                lay.num_kv_heads, lay.block_size, lay.dtype, seqs)


CTX = [1, 15, 16, 17, 40, 63, 64, 65, 100, 257, 1000, 2049]


@pytest.mark.parametrize("dtype,d,hq,hkv", [("bf16", 128, 32, 8), ("bf16", 128, 64, 8), ("bf16", 128, 128, 8),
                                            ("bf16", 64, 8, 2),
                                            ("f32", 64, 8, 2)])
@pytest.mark.parametrize("window", [1, 15, 16, 17, 100, 1000])
def test_ragged_windows(gpu_lib, dtype, d, hq, hkv, window):
    lay = window_layout(CTX, window, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype,
                        seed=window + hq, value_std=1.0 if dtype == "f32" else 0.5)
    say(f"case window {window} {dtype} d={d} hq={hq} hkv={hkv}")
    qh, kh, vh = values_numpy(lay)
    q, k, v = to_device_values(lay, qh, kh, vh)
    ro, rl = oracle_window(lay, qh, kh, vh)
    for sp in [0, 1, 3]:
        out, lse = run_window(gpu_lib, lay, q, k, v, split_pages=sp)
        assert_close(lay, out_to_f64(out), ro, f"window {window} split_pages={sp}")
        assert np.abs(lse.cpu().numpy() - rl).max() < (1e-4 if dtype == "f32" else 1e-3)


def test_window_edge_needle_is_bit_exact(gpu_lib):
    """Row L - W (the first one the query sees) scores 362 above the other
    visible rows, so its weight is exactly 1 and the output is its V row;
    row L - W - 1, just outside the window on the same or the previous page,
    scores twice as high and must not count."""
    ctx = [20, 33, 64, 100, 257, 1000, 3000]
    for window in (5, 16, 17, 50):
        lay = window_layout(ctx, window, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16", seed=window)
        say(f"case window needle W={window}")
        qh, kh, vh = values_numpy(lay)
        kk = np.where(np.isnan(oracle.stored_to_f64(kh, "bf16")), kh, np.uint16(0)).astype(np.uint16)
        qf = np.zeros((lay.num_seqs, 32, 128), dtype=np.float32)
        want = np.zeros((lay.num_seqs, 32, 128), dtype=np.uint16)
        big = bf16_bits_from_f32(np.array([64.0, 128.0], dtype=np.float32))
        for s, L in enumerate(ctx):
            lo = max(0, L - window)
            for g in range(8):
                j = (s * 8 + g) % 128
                p = lay.block_tables[s, lo // 16]
                kk[p, g, lo % 16, j] = big[0]
                # the stronger row just outside the window, where its page is
                # still kept (page 0 is the placeholder: never written)
                if lo > 0 and lay.block_tables[s, (lo - 1) // 16] != 0:
                    kk[lay.block_tables[s, (lo - 1) // 16], g, (lo - 1) % 16, j] = big[1]
                qf[s, g * 4:(g + 1) * 4, j] = 64.0
                want[s, g * 4:(g + 1) * 4] = vh[p, g, lo % 16]
        qq = bf16_bits_from_f32(qf)
        ro, _ = oracle_window(lay, qq, kk, vh)
        ref = bf16_bits_from_f32(ro.astype(np.float32))
        assert np.array_equal(ref, want), f"W={window}: oracle disagrees with the needle"
        q, k, v = to_device_values(lay, qq, kk, vh)
        for sp in (0, 1):
            out, _ = run_window(gpu_lib, lay, q, k, v, split_pages=sp)
            assert np.array_equal(to_host_values(lay, out), ref), f"W={window} split {sp}: window edge mismatch"


def test_window_longer_than_every_context_is_decode(gpu_lib):
    lay = window_layout(CTX, 100_000, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16", seed=2)
    qh, kh, vh = values_numpy(lay)
    q, k, v = to_device_values(lay, qh, kh, vh)
    out_w, lse_w = run_window(gpu_lib, lay, q, k, v)
    bt, ctx = tables_to_device(lay)
    out = torch.empty_like(q)
    lse = torch.empty_like(lse_w)
    total_pages = int(sum((int(L) + 15) // 16 for L in CTX))
    ws = torch.empty(gpu_lib.decode_workspace_size(len(CTX), 8, 4, 128, total_pages, 0), dtype=torch.uint8,
                     device="cuda")
    gpu_lib.decode(out, q, k, v, bt, ctx, lay.context_lens, lay.scale, ws, lse_out=lse)
    torch.cuda.synchronize()
    assert torch.equal(out_w.view(torch.int16), out.view(torch.int16)) and torch.equal(lse_w, lse)


def test_longtail_window_full(gpu_lib):
    """The long-tail batch over a 4096-token window, in the launch
    configuration the benchmark times: every sequence against the oracle."""
    lay = workload("longtail_window4096")
    say("case longtail_window4096 seed 0 (device values, every sequence)")
    q, k, v = values_torch(lay, "cuda")
    out, lse = run_window(gpu_lib, lay, q, k, v)
    assert torch.isfinite(out.float()).all()
    ro, rl = oracle_full(lay, q, k, v)
    assert_close(lay, out_to_f64(out), ro, "longtail_window4096, every sequence")
    assert np.abs(lse.cpu().numpy() - rl).max() < 1e-3


def test_window_must_be_positive(gpu_lib):
    lay = window_layout([10, 20], 5, num_q_heads=8, num_kv_heads=2, head_dim=64, dtype="f32", seed=0)
    qh, kh, vh = values_numpy(lay)
    q, k, v = to_device_values(lay, qh, kh, vh)
    bt, ctx = tables_to_device(lay)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(gpu_lib.PAError) as e:
        gpu_lib.decode_window(torch.empty_like(q), q, k, v, bt, ctx, lay.context_lens, lay.scale, 0, ws)
    assert e.value.code == gpu_lib.PA_EINVAL
