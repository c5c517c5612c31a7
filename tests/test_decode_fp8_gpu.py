"""Parity of pa_decode_fp8 (HIP, through the C ABI) against the fp64 oracle
for an e4m3fn KV cache with one float32 scale per (page, kv-head, slot)."""

import sys

import numpy as np
import pytest
import torch

from gpu_util import assert_close, out_to_f64, tables_to_device
from oracle import fp8 as of8
from workloads import bf16_bits_from_f32, decode_layout, fp8_values_numpy, workload

pytestmark = pytest.mark.gpu

LSE_TOL = 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(q, kc, ks, vc, vs):
    qd = torch.from_numpy(q.view(np.int16)).cuda().view(torch.bfloat16)
    return qd, torch.from_numpy(kc).cuda(), torch.from_numpy(ks).cuda(), torch.from_numpy(vc).cuda(), \
        torch.from_numpy(vs).cuda()


def run_fp8(pa, lay, q, kc, ks, vc, vs, split_pages=0):
    bt, ctx = tables_to_device(lay)
    S, Hq, D = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((S, Hq), dtype=torch.float32, device="cuda")
    total_pages = int(sum((int(L) + 15) // 16 for L in lay.context_lens))
    ws = torch.empty(pa.decode_workspace_size(S, lay.num_kv_heads, lay.gqa_ratio, D, total_pages, split_pages),
                     dtype=torch.uint8, device="cuda")
    pa.decode_fp8(out, q, kc, vc, ks, vs, bt, ctx, lay.context_lens, lay.scale, ws, lse_out=lse,
                  split_pages=split_pages)
    torch.cuda.synchronize()
    return out, lse


def oracle_fp8(lay, q, kc, ks, vc, vs, seqs=None):
    return of8.decode_fp8(q, kc, ks, vc, vs, lay.block_tables, lay.context_lens, lay.scale, lay.num_kv_heads,
                          lay.block_size, "bf16", seqs)


def fp8_layout(ctx, hq, hkv, seed):
    lay = decode_layout(ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, dtype="bf16", pool_factor=1.3,
                        seed=seed)
    lay.kv_dtype = "fp8"
    return lay


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (32, 8), (64, 8), (128, 8), (8, 2), (32, 2)])
def test_shapes_and_ragged_lengths(gpu_lib, hq, hkv):
    ctx = [1, 15, 16, 17, 63, 64, 65, 200, 1000, 2049]
    lay = fp8_layout(ctx, hq, hkv, seed=hq + hkv)
    say(f"case fp8 ragged hq={hq} hkv={hkv}")
    host = fp8_values_numpy(lay)
    dev = to_dev(*host)
    ro, rl = oracle_fp8(lay, *host)
    for sp in [0, 1, 3, 7]:
        out, lse = run_fp8(gpu_lib, lay, *dev, split_pages=sp)
        assert_close(lay, out_to_f64(out), ro, f"fp8 hq={hq} hkv={hkv} split_pages={sp}")
        assert np.abs(lse.cpu().numpy() - rl).max() < LSE_TOL


def test_llama8b_fp8_full(gpu_lib):
    lay = workload("llama8b_decode_fp8")
    say("case llama8b_decode_fp8 seed 0 (full)")
    host = fp8_values_numpy(lay)
    dev = to_dev(*host)
    out, lse = run_fp8(gpu_lib, lay, *dev)
    ro, rl = oracle_fp8(lay, *host)
    err, rel = assert_close(lay, out_to_f64(out), ro, "llama8b_decode_fp8")
    say(f"  max-abs {err:.2e} rel-L2 {rel:.2e}")
    assert np.abs(lse.cpu().numpy() - rl).max() < LSE_TOL
    assert torch.isfinite(out.float()).all()


# 8 and 16 q-heads (1 and 2 per kv-head) run on the vector stream kernel,
# 32 to 128 on the matrix-core kernel
@pytest.mark.parametrize("hq", [8, 16, 32, 64, 128])
def test_needle_gather_is_bit_exact(gpu_lib, hq):
    """One row per (sequence, kv-head) scores ~2500 above every other (code
    448, scale 1, against q = 64 on one column), so its weight is exactly 1
    and the output is that V row read back: code value times its scale.
    V scales are bf16 values, so the read-back row rounds to the same bf16
    bits on both sides.  Checks page lookup and the gather of codes and
    scales at first/last rows, page boundaries and random rows."""
    rng = np.random.default_rng(3)
    ctx = [1, 16, 17, 64, 65, 100, 255, 256, 257, 1000, 4096, 3000]
    lay = fp8_layout(ctx, hq, 8, seed=5)
    G = hq // 8
    say(f"case fp8 needle hq={hq}")
    q0, kc0, ks0, vc, vs = fp8_values_numpy(lay)
    valid = np.isfinite(vs)
    # V scales with 8 significant bits (exact in bf16)
    vs = np.where(valid, (2.0 ** -8) * (1 + rng.integers(0, 128, size=vs.shape) / 128), np.nan).astype(np.float32)
    for trial in range(3):
        kc = np.where(valid[..., None], np.uint8(0), kc0).astype(np.uint8)
        ks = np.where(valid, np.float32(1.0), ks0).astype(np.float32)
        qf = np.zeros((lay.num_seqs, hq, 128), dtype=np.float32)
        want = np.zeros((lay.num_seqs, hq, 128), dtype=np.uint16)
        for s, L in enumerate(ctx):
            for g in range(8):
                if trial == 0:
                    t = [0, L - 1][g % 2]
                elif trial == 1:
                    t = [min(15, L - 1), min(16, L - 1)][g % 2]
                else:
                    t = int(rng.integers(0, L))
                j = (s * 8 + g) % 128
                p = lay.block_tables[s, t // 16]
                kc[p, g, t % 16, j] = 0x7E
                qf[s, g * G:(g + 1) * G, j] = 64.0
                row = of8.dequantize(vc[p, g, t % 16], vs[p, g, t % 16])
                want[s, g * G:(g + 1) * G] = bf16_bits_from_f32(row.astype(np.float32))
        q = bf16_bits_from_f32(qf)
        ro, _ = oracle_fp8(lay, q, kc, ks, vc, vs)
        ref = bf16_bits_from_f32(ro.astype(np.float32))
        assert np.array_equal(ref, want), f"trial {trial}: oracle disagrees with the needle"
        out, _ = run_fp8(gpu_lib, lay, *to_dev(q, kc, ks, vc, vs), split_pages=[0, 1, 3][trial])
        got = out.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, ref), f"trial {trial}: gather mismatch against the oracle"


@pytest.mark.parametrize("hq", [32, 64, 128])
def test_power_of_two_scales_match_bf16_decode(gpu_lib, hq):
    """With power-of-two scales every read-back value is a bf16 value and
    every scaling is exact, so pa_decode_fp8 computes the same products as
    pa_decode on the read-back bf16 pools (whose parity is tested against
    the oracle on its own); only the float32 summation order of P.V differs
    (the two kernels give a lane 8 and 4 rows per load).  Outputs must agree
    to one bf16 rounding step, lse to 1e-5: far tighter than the oracle
    tolerance, so a mis-applied scale cannot hide in it."""
    rng = np.random.default_rng(8)
    ctx = [5, 33, 100, 640, 1500]
    lay = fp8_layout(ctx, hq, 8, seed=12)
    q, kc, _, vc, _ = fp8_values_numpy(lay)
    shape = kc.shape[:3]
    valid = np.isfinite(fp8_values_numpy(lay)[2])
    ks = np.where(valid, 2.0 ** rng.integers(-10, -4, size=shape), np.nan).astype(np.float32)
    vs = np.where(valid, 2.0 ** rng.integers(-10, -4, size=shape), np.nan).astype(np.float32)
    kb = bf16_bits_from_f32(np.nan_to_num(of8.dequantize(kc, ks)).astype(np.float32))
    vb = bf16_bits_from_f32(np.nan_to_num(of8.dequantize(vc, vs)).astype(np.float32))
    qd, kcd, ksd, vcd, vsd = to_dev(q, kc, ks, vc, vs)
    out8, lse8 = run_fp8(gpu_lib, lay, qd, kcd, ksd, vcd, vsd, split_pages=2)
    bt, ctxd = tables_to_device(lay)
    kbd = torch.from_numpy(kb.view(np.int16)).cuda().view(torch.bfloat16)
    vbd = torch.from_numpy(vb.view(np.int16)).cuda().view(torch.bfloat16)
    out16 = torch.empty_like(qd)
    lse16 = torch.empty_like(lse8)
    total_pages = int(sum((int(L) + 15) // 16 for L in ctx))
    ws = torch.empty(gpu_lib.decode_workspace_size(len(ctx), 8, hq // 8, 128, total_pages, 2), dtype=torch.uint8,
                     device="cuda")
    gpu_lib.decode(out16, qd, kbd, vbd, bt, ctxd, lay.context_lens, lay.scale, ws, lse_out=lse16, split_pages=2)
    torch.cuda.synchronize()
    a, b = out8.float(), out16.float()
    assert torch.all((a - b).abs() <= b.abs() * 2.0 ** -7 + 1e-6), float((a - b).abs().max())
    assert float((lse8 - lse16).abs().max()) <= 1e-5
