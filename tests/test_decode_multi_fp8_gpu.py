"""Parity of pa_decode_multi_fp8 (HIP, through the C ABI) against the fp64
oracle: q_len new tokens per sequence, causal among them, over an fp8
(e4m3fn) cache, every folded pass on the matrix cores."""

import sys

import numpy as np
import pytest
import torch

from gpu_util import assert_close, out_to_f64, tables_to_device
from oracle import fp8 as of8
from workloads import decode_layout, fp8_values_numpy

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def multi_fp8_layout(ctx, q_len, hq, hkv, seed):
    lay = decode_layout(list(ctx), num_q_heads=hq, num_kv_heads=hkv, head_dim=128, dtype="bf16", pool_factor=1.3,
                        seed=seed, q_lens=[q_len] * len(ctx), name="multi_token_fp8")
    lay.kv_dtype = "fp8"
    return lay


def to_dev(q, kc, ks, vc, vs):
    qd = torch.from_numpy(q.view(np.int16)).cuda().view(torch.bfloat16)
    return qd, torch.from_numpy(kc).cuda(), torch.from_numpy(ks).cuda(), torch.from_numpy(vc).cuda(), \
        torch.from_numpy(vs).cuda()


def run_multi_fp8(pa, lay, q_len, q, kc, ks, vc, vs, split_pages=0):
    bt, ctx = tables_to_device(lay)
    T, Hq, D = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    total = int(((lay.context_lens + 15) // 16).sum())
    # workspace poisoned with NaN bytes: nothing may be read before it is written
    ws = torch.full((pa.decode_multi_workspace_size(lay.num_seqs, q_len, lay.num_kv_heads, lay.gqa_ratio, D, total,
                                                    split_pages),), 0xFF, dtype=torch.uint8, device="cuda")
    pa.decode_multi_fp8(out, q, kc, vc, ks, vs, bt, ctx, lay.context_lens, lay.scale, q_len, ws, lse_out=lse,
                        split_pages=split_pages)
    torch.cuda.synchronize()
    return out, lse


def oracle_multi_fp8(lay, q_len, q, kc, ks, vc, vs):
    return of8.decode_multi_fp8(q, kc, ks, vc, vs, lay.block_tables, lay.context_lens, q_len, lay.scale,
                                lay.num_kv_heads, lay.block_size, "bf16")


@pytest.mark.parametrize("hq,hkv", [(32, 8), (8, 8), (64, 8), (128, 8), (16, 2)])
@pytest.mark.parametrize("q_len", [2, 3, 4, 5])
def test_ragged_batches(gpu_lib, hq, hkv, q_len):
    ctx = sorted({q_len, q_len + 1, 15, 16, 17, 33, 64, 65, 100, 257, 1000, 2100})
    lay = multi_fp8_layout(ctx, q_len, hq, hkv, seed=q_len * 13 + hq)
    say(f"case multi fp8 q_len={q_len} hq={hq} hkv={hkv}")
    vals = fp8_values_numpy(lay)
    ro, rl = oracle_multi_fp8(lay, q_len, *vals)
    dev = to_dev(*vals)
    for sp in (0, 1, 3):
        out, lse = run_multi_fp8(gpu_lib, lay, q_len, *dev, split_pages=sp)
        assert_close(lay, out_to_f64(out), ro, f"fp8 q_len {q_len} split_pages={sp}")
        assert np.abs(lse.cpu().numpy() - rl).max() < 1e-3


def test_q_len_one_is_decode_fp8(gpu_lib):
    """q_len 1 takes the plain fp8 decode path: bit for bit pa_decode_fp8."""
    lay = multi_fp8_layout([1, 17, 100, 1000, 3000], 1, 32, 8, seed=4)
    q, kc, ks, vc, vs = to_dev(*fp8_values_numpy(lay))
    out_m, lse_m = run_multi_fp8(gpu_lib, lay, 1, q, kc, ks, vc, vs)
    bt, ctx = tables_to_device(lay)
    out = torch.empty_like(q)
    lse = torch.empty_like(lse_m)
    total = int(((lay.context_lens + 15) // 16).sum())
    ws = torch.empty(gpu_lib.decode_workspace_size(lay.num_seqs, 8, 4, 128, total, 0), dtype=torch.uint8,
                     device="cuda")
    gpu_lib.decode_fp8(out, q, kc, vc, ks, vs, bt, ctx, lay.context_lens, lay.scale, ws, lse_out=lse)
    torch.cuda.synchronize()
    assert torch.equal(out_m.view(torch.int16), out.view(torch.int16)) and torch.equal(lse_m, lse)


@pytest.mark.parametrize("q_len,hq", [(4, 32), (2, 128)])
def test_power_of_two_scales_match_bf16_multi(gpu_lib, q_len, hq):
    """Power-of-two scales make every read-back value a bf16 value: the fp8
    call computes the products of pa_decode_multi on the read-back bf16
    pools (both on the matrix cores, same operand order): outputs agree to
    one bf16 rounding step, lse to 1e-5."""
    rng = np.random.default_rng(17)
    ctx = [4, 33, 100, 640, 1500]
    lay = multi_fp8_layout(ctx, q_len, hq, 8, seed=19)
    q, kc, ks0, vc, vs0 = fp8_values_numpy(lay)
    valid = np.isfinite(ks0)
    ks = np.where(valid, 2.0 ** rng.integers(-10, -4, size=ks0.shape), np.nan).astype(np.float32)
    vs = np.where(valid, 2.0 ** rng.integers(-10, -4, size=vs0.shape), np.nan).astype(np.float32)
    from workloads import bf16_bits_from_f32
    kb = bf16_bits_from_f32(np.nan_to_num(of8.dequantize(kc, ks)).astype(np.float32))
    vb = bf16_bits_from_f32(np.nan_to_num(of8.dequantize(vc, vs)).astype(np.float32))
    qd, kcd, ksd, vcd, vsd = to_dev(q, kc, ks, vc, vs)
    out8, lse8 = run_multi_fp8(gpu_lib, lay, q_len, qd, kcd, ksd, vcd, vsd, split_pages=2)
    bt, ctxd = tables_to_device(lay)
    kbd = torch.from_numpy(kb.view(np.int16)).cuda().view(torch.bfloat16)
    vbd = torch.from_numpy(vb.view(np.int16)).cuda().view(torch.bfloat16)
    out16 = torch.empty_like(qd)
    lse16 = torch.empty_like(lse8)
    total = int(((lay.context_lens + 15) // 16).sum())
    ws = torch.empty(gpu_lib.decode_multi_workspace_size(len(ctx), q_len, 8, hq // 8, 128, total, 2),
                     dtype=torch.uint8, device="cuda")
    gpu_lib.decode_multi(out16, qd, kbd, vbd, bt, ctxd, lay.context_lens, lay.scale, q_len, ws, lse_out=lse16,
                         split_pages=2)
    torch.cuda.synchronize()
    a, b = out8.float(), out16.float()
    assert torch.all((a - b).abs() <= b.abs() * 2.0 ** -7 + 1e-6), float((a - b).abs().max())
    assert float((lse8 - lse16).abs().max()) <= 1e-5
