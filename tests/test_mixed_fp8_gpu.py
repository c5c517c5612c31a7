"""Parity of pa_mixed_chunk_fp8 (prefill chunks + decode tokens over an fp8
cache) against the fp64 oracle (oracle.mixed_chunk_fp8: token i of a
segment with L rows and n new tokens sees rows up to L - n + i, K and V read
back from e4m3fn codes and their scales), and of its decode rows against
pa_decode_fp8."""

import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_util import LSE_TOL, assert_close, oracle_full, out_to_f64
from workloads import bf16_bits_from_f32, fp8_values_numpy, fp8_values_torch, mixed_layout, workload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_device(q, kc, ks, vc, vs):
    d = torch.device("cuda")
    return (torch.from_numpy(q.view(np.int16)).to(d).view(torch.bfloat16), torch.from_numpy(kc).to(d),
            torch.from_numpy(ks).to(d), torch.from_numpy(vc).to(d), torch.from_numpy(vs).to(d))


def bits_to_f32(bits):
    """bf16 bit patterns -> their float32 values."""
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def run_mixed_fp8(pa, lay, q, kc, ks, vc, vs):
    T, Hq, D = q.shape
    dev = q.device
    bt = torch.from_numpy(lay.block_tables).to(dev)
    ctx = torch.from_numpy(lay.context_lens).to(dev)
    cu = torch.from_numpy(lay.cu_q_lens.astype(np.int32)).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    total = int(((lay.context_lens + 15) // 16).sum())
    # workspace poisoned with NaN bytes: nothing may be read before it is written
    ws = torch.full((pa.mixed_chunk_workspace_size(T, lay.num_seqs, lay.num_kv_heads, lay.gqa_ratio, D, total),),
                    0xFF, dtype=torch.uint8, device=dev)
    pa.mixed_chunk_fp8(out, q, kc, vc, ks, vs, bt, cu, lay.cu_q_lens, ctx, lay.context_lens, lay.scale, ws,
                       lse_out=lse)
    torch.cuda.synchronize()
    return out, lse


def run_decode_fp8(pa, q, kc, ks, vc, vs, bt, ctx_host, scale, hkv):
    S, Hq, D = q.shape
    ctx = torch.from_numpy(ctx_host).cuda()
    out = torch.empty_like(q)
    lse = torch.empty((S, Hq), dtype=torch.float32, device="cuda")
    total = int(((ctx_host + 15) // 16).sum())
    ws = torch.empty(pa.decode_workspace_size(S, hkv, Hq // hkv, D, total, 0), dtype=torch.uint8, device="cuda")
    pa.decode_fp8(out, q, kc, vc, ks, vs, bt, ctx, ctx_host, scale, ws, lse_out=lse)
    torch.cuda.synchronize()
    return out, lse


def oracle_mixed_fp8(lay, q, kc, ks, vc, vs):
    return oracle.mixed_chunk_fp8(q, kc, ks, vc, vs, lay.block_tables, lay.context_lens, lay.q_lens, lay.scale,
                                  lay.num_kv_heads, 16)


def fp8_mixed(prefixes, chunk, decode, hq, hkv, seed):
    lay = mixed_layout(chunk_prefixes=prefixes, chunk_len=chunk, decode_ctx=decode, num_q_heads=hq,
                       num_kv_heads=hkv, head_dim=128, seed=seed)
    lay.kv_dtype = "fp8"
    return lay


@pytest.mark.parametrize(
    "prefixes,chunk,decode,hq,hkv",
    [
        ([0, 37], 40, [5, 300, 17], 32, 8),         # prefix 0 (pure causal) and a ragged prefix
        ([100], 2, [1, 64], 32, 8),                 # the smallest chunk: two tokens
        ([0, 16, 1500], 70, [900], 32, 8),          # 280 rows: two row blocks; 1570 keys: two key splits
        ([64], 33, [40, 41], 8, 8),                 # G = 1: chunk tiles, then the vector stream kernel
        ([20, 2000], 19, [33], 64, 8),              # G = 8
        ([5], 24, [70, 3], 128, 8),                 # G = 16: 384 rows
        ([3000, 700], 128, [], 32, 8),              # chunks only, 512 rows, three key splits
        ([200], 9, [30, 2], 16, 8),                 # G = 2
    ],
)
def test_mixed_fp8_small(gpu_lib, prefixes, chunk, decode, hq, hkv):
    lay = fp8_mixed(prefixes, chunk, decode, hq, hkv, seed=len(prefixes) * 7 + chunk + 1)
    say(f"case mixed fp8 prefixes={prefixes} chunk={chunk} decode={decode} Hq={hq} Hkv={hkv}")
    host = fp8_values_numpy(lay)
    out, lse = run_mixed_fp8(gpu_lib, lay, *to_device(*host))
    assert torch.isfinite(out.float()).all()
    ro, rl = oracle_mixed_fp8(lay, *host)
    assert_close(lay, out_to_f64(out), ro, "mixed fp8")
    assert np.abs(lse.cpu().numpy() - rl).max() < LSE_TOL


def test_mixed_fp8_decode_only_equals_decode_fp8(gpu_lib):
    """No chunks: pa_decode_fp8's plan, bit for bit."""
    lay = fp8_mixed([], 2, [17, 500, 1000, 64, 3], 32, 8, seed=4)
    host = fp8_values_numpy(lay)
    q, kc, ks, vc, vs = to_device(*host)
    out, lse = run_mixed_fp8(gpu_lib, lay, q, kc, ks, vc, vs)
    bt = torch.from_numpy(lay.block_tables).cuda()
    dout, dlse = run_decode_fp8(gpu_lib, q, kc, ks, vc, vs, bt, lay.context_lens, lay.scale, 8)
    assert torch.equal(out.view(torch.int16), dout.view(torch.int16))
    assert torch.equal(lse, dlse)
    ro, _ = oracle_mixed_fp8(lay, *host)
    assert_close(lay, out_to_f64(out), ro, "decode-only mixed fp8")


def test_mixed_fp8_many_chunks(gpu_lib):
    """More chunks than one launch's chunk list holds (64): the chunk tiles
    and their merges run in several launches."""
    rng = np.random.default_rng(9)
    prefixes = [int(x) for x in rng.integers(0, 200, size=70)]
    lay = fp8_mixed(prefixes, 3, [50, 260], 32, 8, seed=9)
    host = fp8_values_numpy(lay)
    out, lse = run_mixed_fp8(gpu_lib, lay, *to_device(*host))
    ro, rl = oracle_mixed_fp8(lay, *host)
    assert_close(lay, out_to_f64(out), ro, "70 chunks, fp8")
    assert np.abs(lse.cpu().numpy() - rl).max() < LSE_TOL


def test_mixed_fp8_causal_needle(gpu_lib):
    """Chunk token i's q is a one-hot (64 at dim i); row L - n + k of the
    chunk holds the code of 64 (K scale 1) at dims 0 .. k and code 0
    elsewhere, every other row code 0.  Among the rows token i may see only
    its own row scores, so the output must be that row's V read back
    (code x a power-of-two scale: exact in bf16), bit for bit; attending to
    a later row would average several.  The decode token: one planted row
    per kv-head."""
    n = 100
    lay = fp8_mixed([45, 0], n, [77], 32, 8, seed=12)
    q, kc, ks, vc, vs = fp8_values_numpy(lay)
    c64 = torch.tensor([64.0]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()[0]
    kc = np.where(kc == 0x7F, kc, np.uint8(0)).astype(np.uint8)  # (0x7F: the rows no table names)
    rng = np.random.default_rng(3)
    qf = np.zeros((lay.num_tokens, 32, 128), dtype=np.float32)
    want = np.zeros((lay.num_tokens, 32, 128), dtype=np.float64)
    cu = lay.cu_q_lens

    def v_row(p, g, r):
        vs[p, g, r] = 2.0 ** int(rng.integers(-9, -5))
        return oracle.e4m3_to_f64(vc[p, g, r]) * float(vs[p, g, r])

    for s in range(2):
        L = int(lay.context_lens[s])
        for k_ in range(n):
            t = L - n + k_
            p = lay.block_tables[s, t // 16]
            kc[p, :, t % 16, : k_ + 1] = c64
            ks[p, :, t % 16] = 1.0
        for i in range(n):
            t = L - n + i
            p = lay.block_tables[s, t // 16]
            qf[cu[s] + i, :, i] = 64.0
            for g in range(8):
                want[cu[s] + i, g * 4:(g + 1) * 4] = v_row(p, g, t % 16)
    s = 2
    L = int(lay.context_lens[s])
    for g in range(8):
        t = (g * 11) % L
        p = lay.block_tables[s, t // 16]
        kc[p, g, t % 16, 127] = c64
        ks[p, g, t % 16] = 1.0
        qf[cu[s], g * 4:(g + 1) * 4, 127] = 64.0
        want[cu[s], g * 4:(g + 1) * 4] = v_row(p, g, t % 16)
    qq = bf16_bits_from_f32(qf)
    want_bits = bf16_bits_from_f32(want.astype(np.float32))
    assert np.array_equal(bits_to_f32(want_bits).astype(np.float64), want)  # the rows are exact in bf16
    ro, _ = oracle.mixed_chunk_fp8(qq, kc, ks, vc, vs, lay.block_tables, lay.context_lens, lay.q_lens, lay.scale, 8,
                                   16)
    # (compared as values: a zero of the row may come back as -0 where the
    # fp64 oracle adds negative terms far below bf16's range, or as +0)
    assert np.array_equal(bits_to_f32(bf16_bits_from_f32(ro.astype(np.float32))), bits_to_f32(want_bits)), \
        "the oracle misses the planted rows"
    out, _ = run_mixed_fp8(gpu_lib, lay, *to_device(qq, kc, ks, vc, vs))
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(bits_to_f32(got), bits_to_f32(want_bits)), "the kernel does not return the planted rows"


def test_chunked_piggyback_fp8_workload(gpu_lib):
    """The full mixed batch over an fp8 cache, in the launch configuration
    the benchmark times: every token against the oracle, the decode rows
    also against pa_decode_fp8 on the decode segments alone."""
    lay = workload("chunked_piggyback_fp8")
    say("case chunked_piggyback_fp8 seed 0 (every token)")
    q, kc, ks, vc, vs = fp8_values_torch(lay, "cuda")
    out, lse = run_mixed_fp8(gpu_lib, lay, q, kc, ks, vc, vs)
    assert torch.isfinite(out.float()).all()
    ro, rl = oracle_full(lay, q, kc, vc, k_scales=ks, v_scales=vs)
    err, rel = assert_close(lay, out_to_f64(out), ro, "chunked_piggyback_fp8, every token")
    say(f"  max-abs {err:.2e} rel-L2 {rel:.2e}")
    assert np.abs(lse.cpu().numpy() - rl).max() < LSE_TOL
    decs = [s for s in range(lay.num_seqs) if lay.q_lens[s] == 1]
    rows = torch.tensor([int(lay.cu_q_lens[s]) for s in decs], device="cuda")
    bt = torch.from_numpy(lay.block_tables[decs]).cuda()
    dout, dlse = run_decode_fp8(gpu_lib, q[rows].contiguous(), kc, ks, vc, vs, bt, lay.context_lens[decs].copy(),
                                lay.scale, 8)
    assert_close(lay, out_to_f64(out[rows]), out_to_f64(dout), "chunked_piggyback_fp8 decode rows vs pa_decode_fp8")
    assert (lse[rows] - dlse).abs().max().item() < LSE_TOL


def test_mixed_fp8_rejects_null_scales(gpu_lib):
    lay = fp8_mixed([10], 5, [20], 32, 8, seed=1)
    q, kc, ks, vc, vs = to_device(*fp8_values_numpy(lay))
    T, Hq, D = q.shape
    lib = gpu_lib.load()
    ch = lay.context_lens.astype(np.int32)
    cuh = lay.cu_q_lens.astype(np.int32)
    bt = torch.from_numpy(lay.block_tables).cuda()
    ctx = torch.from_numpy(ch).cuda()
    cu = torch.from_numpy(cuh).cuda()
    ws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    rc = lib.pa_mixed_chunk_fp8(out.data_ptr(), None, q.data_ptr(), kc.data_ptr(), vc.data_ptr(), ks.data_ptr(), None,
                                bt.data_ptr(), bt.shape[1], cu.data_ptr(), cuh.ctypes.data, ctx.data_ptr(),
                                ch.ctypes.data, lay.num_seqs, 8, 4, 128, 16, kc.shape[0], lay.scale, ws.data_ptr(),
                                ws.numel(), None)
    assert rc == gpu_lib.PA_EINVAL
