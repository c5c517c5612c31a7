"""Parity of pa_kv_append_fp8 (HIP, through the C ABI) against the oracle:
the codes and scales it writes must equal the oracle's bit for bit (the
quantised codes are integers decided in float32 on both sides); then decode
over the written cache must match the attention oracle."""

import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, out_to_f64, tables_to_device
from oracle import fp8 as of8
from workloads import bf16_bits_from_f32, decode_layout, mixed_layout

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def fp8_pools(lay, seed):
    rng = np.random.default_rng(seed)
    shape = (lay.num_pages, lay.num_kv_heads, 16, lay.head_dim)
    kc = rng.integers(0, 126, size=shape).astype(np.uint8)
    vc = rng.integers(0, 126, size=shape).astype(np.uint8)
    ks = rng.uniform(0.01, 0.02, size=shape[:3]).astype(np.float32)
    vs = rng.uniform(0.01, 0.02, size=shape[:3]).astype(np.float32)
    return kc, ks, vc, vs


def new_rows(lay, rng, dtype, spread=1.0):
    shape = (lay.num_tokens, lay.num_kv_heads, lay.head_dim)
    x = (rng.standard_normal(shape) * spread * np.exp(rng.uniform(-3, 3, size=shape[:2] + (1,)))).astype(np.float32)
    return (bf16_bits_from_f32(x), bf16_bits_from_f32(rng.standard_normal(shape).astype(np.float32))) \
        if dtype == "bf16" else (x, rng.standard_normal(shape).astype(np.float32))


def dev_rows(a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def run_append_fp8(pa, lay, pools, kn, vn, dtype):
    kc, ks, vc, vs = (torch.from_numpy(x).cuda() for x in pools)
    bt, ctx = tables_to_device(lay)
    cu = torch.from_numpy(lay.cu_q_lens.astype(np.int32)).cuda()
    pa.kv_append_fp8(kc, vc, ks, vs, dev_rows(kn, dtype), dev_rows(vn, dtype), bt, cu, lay.cu_q_lens, ctx,
                     lay.context_lens)
    torch.cuda.synchronize()
    return kc, ks, vc, vs


def check_pools(pa, lay, kn, vn, dtype, seed):
    pools = fp8_pools(lay, seed)
    want = of8.kv_append_fp8(*pools, kn, vn, lay.block_tables, lay.context_lens, lay.q_lens, 16, dtype)
    got = run_append_fp8(pa, lay, pools, kn, vn, dtype)
    for name, g, w in zip(("k codes", "k scales", "v codes", "v scales"), got, want):
        gh = g.cpu().numpy()
        assert np.array_equal(gh.view(np.uint8) if gh.dtype == np.uint8 else gh.view(np.uint32),
                              w.view(np.uint8) if w.dtype == np.uint8 else w.view(np.uint32)), name


@pytest.mark.parametrize("dtype,d,hkv", [("bf16", 128, 8), ("f32", 64, 2), ("bf16", 64, 4), ("f32", 128, 8)])
def test_whole_pools_bit_exact(gpu_lib, dtype, d, hkv):
    say(f"case append fp8 {dtype} D={d} Hkv={hkv}")
    lay = mixed_layout(chunk_prefixes=[0, 5, 33], chunk_len=20, decode_ctx=[1, 16, 17, 40, 100], num_q_heads=hkv * 2,
                       num_kv_heads=hkv, head_dim=d, dtype="bf16", name="append_fp8")
    rng = np.random.default_rng(d + hkv)
    kn, vn = new_rows(lay, rng, dtype)
    check_pools(gpu_lib, lay, kn, vn, dtype, seed=d)


def test_rounding_ties_subnormals_and_signs(gpu_lib):
    """Rows whose maximum is 448 * 2^k make the scale 2^k exactly, so every
    x / scale is exact and lands where the rounding rule alone decides:
    halfway between two codes (ties to even), in the subnormal range, on
    signed zeros and on +-448."""
    say("case append fp8 rounding stress")
    lay = mixed_layout(chunk_prefixes=[0], chunk_len=48, decode_ctx=[3, 20], num_q_heads=4, num_kv_heads=2,
                       head_dim=128, dtype="bf16", name="append_fp8_ties")
    vals = of8.E4M3_TABLE[np.array([c for c in range(127) if c != 0x7F])]  # non-negative finite codes
    mids = (vals[:-1] + vals[1:]) / 2  # exact halfway points
    pool = np.concatenate([vals, mids, vals / 4, mids / 2, [0.0, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -11]])
    rng = np.random.default_rng(1)
    T = lay.num_tokens
    kx = np.zeros((T, 2, 128), dtype=np.float32)
    for t in range(T):
        for g in range(2):
            row = rng.choice(pool, size=128) * rng.choice([-1.0, 1.0], size=128)
            row[0] = 448.0
            kx[t, g] = (row * 2.0 ** int(rng.integers(-12, 4))).astype(np.float32)
    kx[0, 0, 5] = -0.0
    kn = kx  # float32 rows: every value above is exact in float32
    vn = (-kx).astype(np.float32)
    check_pools(gpu_lib, lay, kn, vn, "f32", seed=7)


def test_append_then_fp8_decode(gpu_lib):
    """Write whole contexts with pa_kv_append_fp8 (every row new), then
    pa_decode_fp8 over the cache: against the oracle's append + decode."""
    say("case append fp8 then decode")
    ctx = [1, 17, 64, 100, 333, 1000]
    lay = decode_layout(ctx, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16", pool_factor=1.2, seed=3)
    lay.q_lens = lay.context_lens.copy()  # every row is new
    rng = np.random.default_rng(4)
    kn, vn = new_rows(lay, rng, "bf16", spread=0.5)
    pools = fp8_pools(lay, 11)
    kc, ks, vc, vs = of8.kv_append_fp8(*pools, kn, vn, lay.block_tables, lay.context_lens, lay.q_lens, 16, "bf16")
    got = run_append_fp8(gpu_lib, lay, pools, kn, vn, "bf16")
    q = bf16_bits_from_f32((rng.standard_normal((len(ctx), 32, 128)) * 0.5).astype(np.float32))
    qd = torch.from_numpy(q.view(np.int16)).cuda().view(torch.bfloat16)
    bt, ctxd = tables_to_device(lay)
    out = torch.empty_like(qd)
    lse = torch.empty((len(ctx), 32), dtype=torch.float32, device="cuda")
    total = int(sum((L + 15) // 16 for L in ctx))
    ws = torch.empty(gpu_lib.decode_workspace_size(len(ctx), 8, 4, 128, total, 0), dtype=torch.uint8, device="cuda")
    kcd, ksd, vcd, vsd = got
    gpu_lib.decode_fp8(out, qd, kcd, vcd, ksd, vsd, bt, ctxd, lay.context_lens, lay.scale, ws, lse_out=lse)
    torch.cuda.synchronize()
    ro, rl = of8.decode_fp8(q, kc, ks, vc, vs, lay.block_tables, lay.context_lens, lay.scale, 8, 16, "bf16")
    assert_close(lay, out_to_f64(out), ro, "append fp8 then decode")
    assert np.abs(lse.cpu().numpy() - rl).max() < 1e-3
