"""Parity of pa_mixed_chunk (prefill chunks + decode tokens in one call)
against the fp64 oracle, and of its decode rows against pa_decode."""

import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_util import LSE_TOL, assert_close, device_inputs, oracle_full, out_to_f64, to_device_values, to_host_values
from workloads import bf16_bits_from_f32, mixed_layout, values_numpy, workload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_mixed(pa, lay, q, k, v):
    T, Hq, D = q.shape
    dev = q.device
    bt = torch.from_numpy(lay.block_tables).to(dev)
    ctx = torch.from_numpy(lay.context_lens).to(dev)
    cu = torch.from_numpy(lay.cu_q_lens.astype(np.int32)).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)
    total = int(((lay.context_lens + 15) // 16).sum())
    ws = torch.empty(pa.mixed_chunk_workspace_size(T, lay.num_seqs, lay.num_kv_heads, lay.gqa_ratio, D, total),
                     dtype=torch.uint8, device=dev)
    pa.mixed_chunk(out, q, k, v, bt, cu, lay.cu_q_lens, ctx, lay.context_lens, lay.scale, ws, lse_out=lse)
    torch.cuda.synchronize()
    return out, lse


def run_decode(pa, q, k, v, bt, ctx_host, scale, hkv):
    S, Hq, D = q.shape
    ctx = torch.from_numpy(ctx_host).cuda()
    out = torch.empty_like(q)
    lse = torch.empty((S, Hq), dtype=torch.float32, device="cuda")
    total = int(((ctx_host + 15) // 16).sum())
    ws = torch.empty(pa.decode_workspace_size(S, hkv, Hq // hkv, D, total, 0), dtype=torch.uint8, device="cuda")
    pa.decode(out, q, k, v, bt, ctx, ctx_host, scale, ws, lse_out=lse)
    torch.cuda.synchronize()
    return out, lse


def oracle_mixed(lay, qh, kh, vh, seqs=None):
    return oracle.mixed_chunk(qh, kh, vh, lay.block_tables, lay.context_lens, lay.q_lens, lay.scale,
                              lay.num_kv_heads, 16, lay.dtype, seqs)


@pytest.mark.parametrize(
    "prefixes,chunk,decode,hq,hkv",
    [
        ([0, 37], 40, [5, 300, 17], 32, 8),         # prefix 0 (pure causal) and a ragged prefix
        ([100], 2, [1, 64], 32, 8),                 # the smallest chunk: two tokens
        ([0, 16, 1500], 70, [900], 32, 8),          # 280 rows: two row blocks; 1570 keys: two key splits
        ([64], 33, [40, 41], 8, 8),                 # G = 1
        ([20, 2000], 19, [33], 64, 8),              # G = 8
        ([5], 24, [70, 3], 128, 8),                 # G = 16: 384 rows
        ([3000, 700], 128, [], 32, 8),              # chunks only, 512 rows, three key splits
    ],
)
def test_mixed_small(gpu_lib, prefixes, chunk, decode, hq, hkv):
    lay = mixed_layout(chunk_prefixes=prefixes, chunk_len=chunk, decode_ctx=decode, num_q_heads=hq,
                       num_kv_heads=hkv, head_dim=128, seed=len(prefixes) * 7 + chunk)
    say(f"case mixed prefixes={prefixes} chunk={chunk} decode={decode} Hq={hq} Hkv={hkv}")
    (q, k, v), (qh, kh, vh) = device_inputs(lay)
    out, lse = run_mixed(gpu_lib, lay, q, k, v)
    ro, rl = oracle_mixed(lay, qh, kh, vh)
    assert_close(lay, out_to_f64(out), ro, "mixed")
    assert np.abs(lse.cpu().numpy() - rl).max() < LSE_TOL


def test_mixed_decode_only_equals_decode(gpu_lib):
    lay = mixed_layout(chunk_prefixes=[], chunk_len=2, decode_ctx=[17, 500, 1000, 64, 3], num_q_heads=32,
                       num_kv_heads=8, head_dim=128, seed=4)
    (q, k, v), (qh, kh, vh) = device_inputs(lay)
    out, lse = run_mixed(gpu_lib, lay, q, k, v)
    bt = torch.from_numpy(lay.block_tables).cuda()
    dout, dlse = run_decode(gpu_lib, q, k, v, bt, lay.context_lens, lay.scale, 8)
    assert torch.equal(out.view(torch.int16), dout.view(torch.int16))
    assert torch.equal(lse, dlse)
    ro, _ = oracle_mixed(lay, qh, kh, vh)
    assert_close(lay, out_to_f64(out), ro, "decode-only mixed")


def test_mixed_many_chunks(gpu_lib):
    """More chunks than one launch's chunk list holds (64): the chunk tiles
    and their merges run in several launches."""
    rng = np.random.default_rng(9)
    prefixes = [int(x) for x in rng.integers(0, 200, size=70)]
    lay = mixed_layout(chunk_prefixes=prefixes, chunk_len=3, decode_ctx=[50, 260], num_q_heads=32, num_kv_heads=8,
                       head_dim=128, seed=9)
    (q, k, v), (qh, kh, vh) = device_inputs(lay)
    out, lse = run_mixed(gpu_lib, lay, q, k, v)
    ro, rl = oracle_mixed(lay, qh, kh, vh)
    assert_close(lay, out_to_f64(out), ro, "70 chunks")
    assert np.abs(lse.cpu().numpy() - rl).max() < LSE_TOL


def test_chunked_piggyback_workload(gpu_lib):
    """The full mixed batch: 4 chunks of 512 tokens after prefixes of 0, 1024,
    4096 and 8192 rows, plus 256 decode tokens, in the launch configuration
    the benchmark times (chunks and decode tokens in one launch).  Every
    token against the oracle; the decode rows also against pa_decode on the
    decode segments alone (the one-launch kernel plans its own decode runs,
    so the split points and the rounding may differ)."""
    lay = workload("chunked_piggyback")
    say("case chunked_piggyback seed 0 (every token)")
    (q, k, v), _ = device_inputs(lay, host_values=False)
    out, lse = run_mixed(gpu_lib, lay, q, k, v)
    assert torch.isfinite(out.float()).all()
    cu = lay.cu_q_lens
    chunks = [s for s in range(lay.num_seqs) if lay.q_lens[s] > 1]
    decs = [s for s in range(lay.num_seqs) if lay.q_lens[s] == 1]
    assert len(chunks) == 4 and len(decs) == 256
    ro, rl = oracle_full(lay, q, k, v)
    err, rel = assert_close(lay, out_to_f64(out), ro, "chunked_piggyback, every token")
    say(f"  max-abs {err:.2e} rel-L2 {rel:.2e}")
    assert np.abs(lse.cpu().numpy() - rl).max() < LSE_TOL
    rows = torch.tensor([int(cu[s]) for s in decs], device="cuda")
    bt = torch.from_numpy(lay.block_tables[decs]).cuda()
    dout, dlse = run_decode(gpu_lib, q[rows].contiguous(), k, v, bt, lay.context_lens[decs].copy(), lay.scale, 8)
    assert_close(lay, out_to_f64(out[rows]), out_to_f64(dout), "chunked_piggyback decode rows vs pa_decode")
    assert (lse[rows] - dlse).abs().max().item() < LSE_TOL


def test_mixed_causal_needle(gpu_lib):
    """Chunk token i's q is a one-hot (64 at dim i) and rows L - n + k for
    k >= i of the chunk carry 64 at dim i: the token's own row and every
    later row of the chunk score alike, the rows before score 0.  Causal
    masking leaves exactly the token's own row, so the output must be that
    V row's bits; attending to a later row would average several."""
    n = 100
    lay = mixed_layout(chunk_prefixes=[45, 0], chunk_len=n, decode_ctx=[77], num_q_heads=32, num_kv_heads=8,
                       head_dim=128, seed=12)
    qh, kh, vh = values_numpy(lay)
    kk = np.where(np.isnan(oracle.stored_to_f64(kh, "bf16")), kh, np.uint16(0)).astype(np.uint16)
    big = bf16_bits_from_f32(np.array([64.0], dtype=np.float32))[0]
    qf = np.zeros((lay.num_tokens, 32, 128), dtype=np.float32)
    want = np.zeros((lay.num_tokens, 32, 128), dtype=np.uint16)
    cu = lay.cu_q_lens
    for s in range(2):
        L = int(lay.context_lens[s])
        for k_ in range(n):
            t = L - n + k_
            p = lay.block_tables[s, t // 16]
            kk[p, :, t % 16, : k_ + 1] = big  # row t: 64 at dims 0 .. k
        for i in range(n):
            t = L - n + i
            p = lay.block_tables[s, t // 16]
            qf[cu[s] + i, :, i] = 64.0
            want[cu[s] + i] = vh[p, np.arange(32) // 4, t % 16]
    s = 2  # the decode token: one row of its context dominates per kv-head
    L = int(lay.context_lens[s])
    for g in range(8):
        t = (g * 11) % L
        p = lay.block_tables[s, t // 16]
        kk[p, g, t % 16, 127] = big
        qf[cu[s], g * 4:(g + 1) * 4, 127] = 64.0
        want[cu[s], g * 4:(g + 1) * 4] = vh[p, g, t % 16]
    qq = bf16_bits_from_f32(qf)
    ro, _ = oracle_mixed(lay, qq, kk, vh)
    assert np.array_equal(bf16_bits_from_f32(ro.astype(np.float32)), want)
    qd, kd, vd = to_device_values(lay, qq, kk, vh)
    out, _ = run_mixed(gpu_lib, lay, qd, kd, vd)
    assert np.array_equal(to_host_values(lay, out), want)
