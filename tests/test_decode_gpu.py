"""Parity of pa_decode (HIP, through the C ABI) against the fp64 oracle."""

import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (LSE_TOL, assert_close, device_inputs, oracle_full, out_to_f64, tables_to_device,
                      to_device_values, to_host_values)
from workloads import bf16_bits_from_f32, decode_layout, values_numpy, workload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_decode(pa, lay, q, k, v, split_pages=0, want_lse=True):
    bt, ctx = tables_to_device(lay)
    S, Hq, D = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((S, Hq), dtype=torch.float32, device="cuda") if want_lse else None
    total_pages = int(sum((int(L) + 15) // 16 for L in lay.context_lens))
    ws = torch.empty(pa.decode_workspace_size(S, lay.num_kv_heads, lay.gqa_ratio, D, total_pages, split_pages),
                     dtype=torch.uint8, device="cuda")
    pa.decode(out, q, k, v, bt, ctx, lay.context_lens, lay.scale, ws, lse_out=lse, split_pages=split_pages)
    torch.cuda.synchronize()
    return out, lse


def oracle_decode(lay, qh, kh, vh, seqs=None):
    return oracle.decode(qh, kh, vh, lay.block_tables, lay.context_lens, lay.scale, lay.num_kv_heads,
                         lay.block_size, lay.dtype, seqs)


def test_tiny_f32_full(gpu_lib):
    lay = workload("tiny_f32")
    say("case tiny_f32 seed 0")
    (q, k, v), (qh, kh, vh) = device_inputs(lay)
    ro, rl = oracle_decode(lay, qh, kh, vh)
    for sp in [0, 1, 2, 5]:
        out, lse = run_decode(gpu_lib, lay, q, k, v, split_pages=sp)
        assert_close(lay, out_to_f64(out), ro, f"tiny_f32 split_pages={sp}")
        assert np.abs(lse.cpu().numpy() - rl).max() < 1e-4


def test_llama8b_full(gpu_lib):
    lay = workload("llama8b_decode")
    say("case llama8b_decode seed 0 (full)")
    (q, k, v), (qh, kh, vh) = device_inputs(lay)
    ro, rl = oracle_decode(lay, qh, kh, vh)
    out, lse = run_decode(gpu_lib, lay, q, k, v)
    err, rel = assert_close(lay, out_to_f64(out), ro, "llama8b_decode")
    say(f"  max-abs {err:.2e} rel-L2 {rel:.2e}")
    assert np.abs(lse.cpu().numpy() - rl).max() < 1e-3


def test_longtail_full(gpu_lib):
    """The long-tail batch (256 sequences, 16 to 32768 rows, 8 q-heads per
    kv-head) in the launch configuration the benchmark times: every
    sequence against the oracle."""
    lay = workload("longtail_splitkv")
    say("case longtail_splitkv seed 0 (device values, every sequence)")
    q, k, v = device_inputs(lay, host_values=False)[0]
    out, lse = run_decode(gpu_lib, lay, q, k, v)
    # every row of the batch is finite (no NaN poison leaked anywhere)
    assert torch.isfinite(out.float()).all()
    ro, rl = oracle_full(lay, q, k, v)
    err, rel = assert_close(lay, out_to_f64(out), ro, "longtail_splitkv, every sequence")
    say(f"  max-abs {err:.2e} rel-L2 {rel:.2e}")
    assert np.abs(lse.cpu().numpy() - rl).max() < LSE_TOL


@pytest.mark.parametrize("total_pages", [1290, 1300, 2611, 5000])
def test_automatic_plan_paired_runs(gpu_lib, total_pages):
    """Automatic plans of the matrix-core kernel over bf16 pools pair the
    runs (the even wave of each pair takes a few pages more than the odd
    one) and add one empty wave when the run count is odd; with 8 kv-heads
    on 256 CUs these totals give runs of 11 to 40 pages and both parities
    of the run count.  Every sequence still matches the oracle."""
    rng = np.random.default_rng(total_pages)
    n = 24
    cuts = np.sort(rng.choice(np.arange(1, total_pages), n - 1, replace=False))
    pages = np.diff(np.concatenate([[0], cuts, [total_pages]]))
    ctx = [int(16 * p - rng.integers(0, 16)) for p in pages]  # ragged last page, same page count
    lay = decode_layout(ctx, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16", pool_factor=1.2, seed=7,
                        value_std=0.5)
    say(f"case paired runs: {total_pages} pages over {n} sequences")
    (q, k, v), (qh, kh, vh) = device_inputs(lay)
    ro, rl = oracle_decode(lay, qh, kh, vh)
    out, lse = run_decode(gpu_lib, lay, q, k, v)
    assert_close(lay, out_to_f64(out), ro, f"paired runs, {total_pages} pages")
    assert np.abs(lse.cpu().numpy() - rl).max() < 1e-3


@pytest.mark.parametrize("dtype,d,hq,hkv", [("bf16", 128, 8, 8), ("bf16", 128, 16, 8), ("bf16", 128, 128, 8),
                                            ("bf16", 64, 8, 2), ("bf16", 64, 32, 4), ("bf16", 64, 32, 2),
                                            ("f32", 64, 4, 4),
                                            ("f32", 64, 16, 2)])
def test_shapes_and_ragged_lengths(gpu_lib, dtype, d, hq, hkv):
    ctx = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 511, 512, 513, 1000, 2049]
    lay = decode_layout(ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype, pool_factor=1.3,
                        seed=5, value_std=1.0 if dtype == "f32" else 0.5)
    say(f"case shapes {dtype} D={d} Hq={hq} Hkv={hkv}")
    (q, k, v), (qh, kh, vh) = device_inputs(lay)
    ro, rl = oracle_decode(lay, qh, kh, vh)
    for sp in [0, 1, 3, 8]:
        out, lse = run_decode(gpu_lib, lay, q, k, v, split_pages=sp)
        assert_close(lay, out_to_f64(out), ro, f"{dtype} D={d} G={hq // hkv} split={sp}")
        assert np.abs(lse.cpu().numpy() - rl).max() < (1e-4 if dtype == "f32" else 1e-3)


# (dtype, head_dim, q-heads, kv-heads): 4 bf16 q-heads per kv-head run on
# the matrix-core stream kernel; float32 (the tiny workload's shape) and 1 or
# 2 bf16 q-heads per kv-head on the vector stream kernel.
NEEDLE_SHAPES = [("bf16", 128, 32, 8), ("f32", 64, 8, 2), ("bf16", 128, 8, 8), ("bf16", 128, 16, 8),
                 ("bf16", 64, 16, 8), ("f32", 64, 4, 4)]


def _stored(lay, x):
    """float32 values -> the layout's stored form (bf16 bits or float32)."""
    x = np.asarray(x, dtype=np.float32)
    return bf16_bits_from_f32(x) if lay.dtype == "bf16" else x


@pytest.mark.parametrize("dtype,d,hq,hkv", NEEDLE_SHAPES)
def test_one_row_context_returns_v_row(gpu_lib, dtype, d, hq, hkv):
    lay = decode_layout([1] * 9, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype, seed=2,
                        value_std=1.0 if dtype == "f32" else 0.5)
    say(f"case one-row context {dtype} D={d} Hq={hq} Hkv={hkv}")
    (q, k, v), (qh, kh, vh) = device_inputs(lay)
    out, _ = run_decode(gpu_lib, lay, q, k, v)
    got = to_host_values(lay, out)  # bf16 bits or float32 [S, Hq, D]
    G = hq // hkv
    for s in range(lay.num_seqs):
        p = lay.block_tables[s, 0]
        for h in range(hq):
            assert np.array_equal(got[s, h].view(np.uint32) if dtype == "f32" else got[s, h],
                                  vh[p, h // G, 0].view(np.uint32) if dtype == "f32" else vh[p, h // G, 0]), (s, h)


@pytest.mark.parametrize("dtype,d,hq,hkv", NEEDLE_SHAPES)
def test_needle_gather_is_bit_exact(gpu_lib, dtype, d, hq, hkv):
    """Each (sequence, kv-head) has one key aligned with q and far above the
    rest (a score of at least 362 against 0), so softmax puts weight exactly
    1 on it and the output must be that row's V bits: table lookup and gather
    indexing are checked bit-exactly, at first/last rows and page
    boundaries, on both stream kernels."""
    rng = np.random.default_rng(9)
    ctx = [1, 16, 17, 64, 65, 100, 255, 256, 257, 1000, 4096, 3000]
    G = hq // hkv
    lay = decode_layout(ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype, pool_factor=1.5, seed=4,
                        value_std=1.0 if dtype == "f32" else 0.5)
    say(f"case needle {dtype} D={d} Hq={hq} Hkv={hkv}")
    qh, kh, vh = values_numpy(lay)
    widen = (lambda a: oracle.stored_to_f64(a, "bf16")) if dtype == "bf16" else (lambda a: a.astype(np.float64))
    zero_k = np.where(np.isnan(widen(kh)), kh, _stored(lay, 0.0)).astype(kh.dtype)
    big = _stored(lay, np.array([64.0]))[0]  # score 64 * 64 * scale >= 362 (D <= 128)
    for trial in range(3):
        kk = zero_k.copy()
        qf = np.zeros((lay.num_seqs, hq, d), dtype=np.float32)
        want = np.zeros((lay.num_seqs, hq, d), dtype=vh.dtype)
        for s, L in enumerate(ctx):
            for g in range(hkv):
                if trial == 0:
                    t = [0, L - 1][g % 2]
                elif trial == 1:
                    t = [min(15, L - 1), min(16, L - 1)][g % 2]
                else:
                    t = int(rng.integers(0, L))
                j = (s * hkv + g) % d
                p = lay.block_tables[s, t // 16]
                kk[p, g, t % 16, j] = big
                qf[s, g * G:(g + 1) * G, j] = 64.0
                want[s, g * G:(g + 1) * G] = vh[p, g, t % 16]
        qq = _stored(lay, qf)
        qd, kd, vd = to_device_values(lay, qq, kk, vh)
        out, _ = run_decode(gpu_lib, lay, qd, kd, vd, split_pages=[0, 1, 3][trial])
        got = to_host_values(lay, out)
        ro, _ = oracle_decode(lay, qq, kk, vh)
        ref = _stored(lay, ro)
        bits = (lambda a: a.view(np.uint32)) if dtype == "f32" else (lambda a: a)
        assert np.array_equal(bits(ref), bits(want)), f"trial {trial}: oracle disagrees with the needle"
        assert np.array_equal(bits(got), bits(ref)), f"trial {trial}: gather mismatch against the oracle"


def test_page_relabelling_gives_identical_bits(gpu_lib):
    lay = workload("llama8b_decode", seed=3)
    (q, k, v), _ = device_inputs(lay)
    out1, lse1 = run_decode(gpu_lib, lay, q, k, v)
    pi = np.random.default_rng(1).permutation(lay.num_pages)
    pit = torch.from_numpy(np.argsort(pi)).cuda()
    k2 = k.index_select(0, pit)
    v2 = v.index_select(0, pit)  # new page pi[p] holds old page p
    lay2 = dataclasses.replace(
        lay, block_tables=np.where(lay.block_tables >= 0, pi[np.maximum(lay.block_tables, 0)], -1).astype(np.int32))
    out2, lse2 = run_decode(gpu_lib, lay2, q, k2, v2)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1, lse2)


def test_constant_v_and_peaked_scores(gpu_lib):
    ctx = [5, 300, 4000, 129]
    lay = decode_layout(ctx, num_q_heads=16, num_kv_heads=2, head_dim=128, dtype="bf16", seed=8)
    qh, kh, vh = values_numpy(lay)
    vconst = vh.copy()
    vconst[~np.isnan(opa_widen(vh))] = bf16_bits_from_f32(np.array([0.375], dtype=np.float32))[0]
    qd, kd, vd = to_device_values(lay, qh, kh, vconst)
    out, _ = run_decode(gpu_lib, lay, qd, kd, vd, split_pages=2)
    assert np.all(out.float().cpu().numpy() == 0.375)
    # peaked scores (q x 16) exercise the running-max rescale
    q16 = bf16_bits_from_f32(opa_widen(qh).astype(np.float32) * 16)
    qd, kd, vd = to_device_values(lay, q16, kh, vh)
    ro, _ = oracle_decode(lay, q16, kh, vh)
    for sp in [0, 1]:
        out, _ = run_decode(gpu_lib, lay, qd, kd, vd, split_pages=sp)
        assert_close(lay, out_to_f64(out), ro, f"peaked split={sp}")


def opa_widen(bits):
    return oracle.stored_to_f64(bits, "bf16")


def test_errors_launch_nothing(gpu_lib):
    lay = workload("tiny_f32")
    (q, k, v), _ = device_inputs(lay)
    bt, ctx = tables_to_device(lay)
    out = torch.full_like(q, 7.0)
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(gpu_lib.PAError) as e:
        gpu_lib.decode(out, q, k, v, bt, ctx, lay.context_lens, lay.scale, ws, split_pages=1)
    assert e.value.code == gpu_lib.PA_EWORKSPACE
    bad = lay.context_lens.copy()
    bad[2] = 0
    with pytest.raises(gpu_lib.PAError) as e:
        gpu_lib.decode(out, q, k, v, bt, ctx, bad, lay.scale, ws)
    assert e.value.code == gpu_lib.PA_EINVAL
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
