"""Parity of pa_prefix_cascade_fp8 (fp8 MFMA prefix tiles + fp8 suffix
stream + merge) against the fp64 oracle (oracle.prefix_cascade_fp8: decode
over each member's whole table, rows read back from e4m3fn codes and their
scales), and against pa_decode_fp8 on the same inputs."""

import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_util import LSE_TOL, assert_close, oracle_full, out_to_f64
from workloads import bf16_bits_from_f32, cascade_layout, fp8_values_numpy, fp8_values_torch, workload

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


def run_cascade_fp8(pa, lay, q, kc, ks, vc, vs):
    S, Hq, D = q.shape
    dev = q.device
    bt = torch.from_numpy(lay.block_tables).to(dev)
    ctx = torch.from_numpy(lay.context_lens).to(dev)
    go = torch.from_numpy(lay.group_seq_offsets).to(dev)
    pl = torch.from_numpy(lay.prefix_lens).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((S, Hq), dtype=torch.float32, device=dev)
    total = int(((lay.context_lens + 15) // 16).sum())
    ws = torch.full((pa.prefix_cascade_workspace_size(S, lay.num_kv_heads, lay.gqa_ratio, D, total),), 0xFF,
                    dtype=torch.uint8, device=dev)  # NaN bytes: nothing may be read before it is written
    pa.prefix_cascade_fp8(out, q, kc, vc, ks, vs, bt, ctx, lay.context_lens, go, lay.group_seq_offsets, pl,
                          lay.prefix_lens, lay.scale, ws, lse_out=lse)
    torch.cuda.synchronize()
    return out, lse


def run_decode_fp8(pa, lay, q, kc, ks, vc, vs):
    S, Hq, D = q.shape
    bt = torch.from_numpy(lay.block_tables).cuda()
    ctx = torch.from_numpy(lay.context_lens).cuda()
    out = torch.empty_like(q)
    lse = torch.empty((S, Hq), dtype=torch.float32, device="cuda")
    total = int(((lay.context_lens + 15) // 16).sum())
    ws = torch.empty(pa.decode_workspace_size(S, lay.num_kv_heads, lay.gqa_ratio, D, total, 0), dtype=torch.uint8,
                     device="cuda")
    pa.decode_fp8(out, q, kc, vc, ks, vs, bt, ctx, lay.context_lens, lay.scale, ws, lse_out=lse)
    torch.cuda.synchronize()
    return out, lse


def oracle_cascade_fp8(lay, q, kc, ks, vc, vs):
    return oracle.prefix_cascade_fp8(q, kc, ks, vc, vs, lay.block_tables, lay.context_lens, lay.scale,
                                     lay.num_kv_heads, 16, lay.group_seq_offsets, lay.prefix_lens)


def fp8_cascade(groups, per_group, prefix, suf_hi, hq, hkv, seed, prefix_lens=None):
    lay = cascade_layout(num_groups=groups, seqs_per_group=per_group, prefix_len=prefix, suffix_lo=1,
                         suffix_hi=suf_hi, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, seed=seed,
                         prefix_lens=prefix_lens)
    lay.kv_dtype = "fp8"
    return lay


@pytest.mark.parametrize(
    "groups,per_group,prefix,suf_hi,hq,hkv",
    [
        (3, 5, 64, 40, 32, 8),       # small groups, short suffixes
        (2, 70, 128, 300, 32, 8),    # 280 rows per kv-head: two row blocks
        (4, 8, 16, 17, 8, 8),        # G = 1 (suffix on the vector kernel), one-page prefix: a partial tile
        (2, 16, 80, 100, 64, 8),     # G = 8, prefix not a multiple of 64 keys
        (1, 33, 2048, 600, 32, 8),   # long prefix, several key splits
        (3, 4, 0, 90, 32, 8),        # no prefix at all
        (2, 12, 96, 70, 128, 8),     # G = 16
        (3, 10, 48, 60, 16, 8),      # G = 2 (suffix on the vector kernel)
    ],
)
def test_cascade_fp8_small(gpu_lib, groups, per_group, prefix, suf_hi, hq, hkv):
    lay = fp8_cascade(groups, per_group, prefix, suf_hi, hq, hkv, seed=groups + prefix + 7)
    say(f"case cascade fp8 groups={groups}x{per_group} prefix={prefix} suffix<= {suf_hi} Hq={hq} Hkv={hkv}")
    host = fp8_values_numpy(lay)
    dev = to_device(*host)
    out, lse = run_cascade_fp8(gpu_lib, lay, *dev)
    assert torch.isfinite(out.float()).all()
    ro, rl = oracle_cascade_fp8(lay, *host)
    assert_close(lay, out_to_f64(out), ro, "cascade fp8")
    assert np.abs(lse.cpu().numpy() - rl).max() < LSE_TOL
    dout, _ = run_decode_fp8(gpu_lib, lay, *dev)
    assert_close(lay, out_to_f64(out), out_to_f64(dout), "cascade fp8 vs decode fp8")


def test_cascade_fp8_mixed_prefix_lengths(gpu_lib):
    lay = fp8_cascade(4, 9, 0, 200, 32, 8, seed=11, prefix_lens=[0, 512, 32, 1040])
    host = fp8_values_numpy(lay)
    out, lse = run_cascade_fp8(gpu_lib, lay, *to_device(*host))
    ro, rl = oracle_cascade_fp8(lay, *host)
    assert_close(lay, out_to_f64(out), ro, "cascade fp8 mixed prefixes")
    assert np.abs(lse.cpu().numpy() - rl).max() < LSE_TOL


def test_cascade_fp8_needle_in_prefix_and_suffix(gpu_lib):
    """One key per (sequence, kv-head) dominates: in the shared prefix for
    even kv-heads, in the sequence's own suffix for odd ones.  That key's
    row holds code 64 at one position (K scale 1) and its V scale is a power
    of two, so the read-back V row is exact in bf16 and the output must be
    its bits."""
    lay = fp8_cascade(2, 6, 96, 70, 32, 8, seed=3)
    q, kc, ks, vc, vs = fp8_values_numpy(lay)
    c64 = torch.tensor([64.0]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()[0]
    qf = np.zeros((lay.num_seqs, 32, 128), dtype=np.float32)
    want = np.zeros((lay.num_seqs, 32, 128), dtype=np.float64)
    rng = np.random.default_rng(5)

    def plant(p, g, r, j):
        kc[p, g, r, :] = 0
        kc[p, g, r, j] = c64
        ks[p, g, r] = 1.0
        vs[p, g, r] = 2.0 ** int(rng.integers(-9, -5))
        return oracle.e4m3_to_f64(vc[p, g, r]) * float(vs[p, g, r])

    for gi in range(2):
        for g in range(0, 8, 2):
            t = int(rng.integers(0, 96))
            p = lay.block_tables[gi * 6, t // 16]
            j = g * 7 % 128
            row = plant(p, g, t % 16, j)
            for s in range(gi * 6, gi * 6 + 6):
                qf[s, g * 4:(g + 1) * 4, j] = 64.0
                want[s, g * 4:(g + 1) * 4] = row
    for s in range(lay.num_seqs):
        L = int(lay.context_lens[s])
        for g in range(1, 8, 2):
            t = int(rng.integers(96, L))
            p = lay.block_tables[s, t // 16]
            j = (s + g) % 128
            row = plant(p, g, t % 16, j)
            qf[s, g * 4:(g + 1) * 4, j] = 64.0
            want[s, g * 4:(g + 1) * 4] = row
    qq = bf16_bits_from_f32(qf)
    out, _ = run_cascade_fp8(gpu_lib, lay, *to_device(qq, kc, ks, vc, vs))
    want_bits = bf16_bits_from_f32(want.astype(np.float32))
    assert np.array_equal(bits_to_f32(want_bits).astype(np.float64), want)  # the rows are exact in bf16
    ro, _ = oracle_cascade_fp8(lay, qq, kc, ks, vc, vs)
    # (compared as values: a zero of the row may come back as -0 where the
    # fp64 oracle adds negative terms far below bf16's range, or as +0)
    assert np.array_equal(bits_to_f32(bf16_bits_from_f32(ro.astype(np.float32))), bits_to_f32(want_bits)), \
        "the oracle misses the planted rows"
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(bits_to_f32(got), bits_to_f32(want_bits)), "the kernel does not return the planted rows"


def test_shared_prefix_fp8_workload(gpu_lib):
    """The shared-prefix batch over an fp8 cache, in the launch
    configuration the benchmark times: every sequence against the oracle and
    against pa_decode_fp8."""
    lay = workload("shared_prefix_fp8")
    say("case shared_prefix_fp8 seed 0 (every sequence)")
    q, kc, ks, vc, vs = fp8_values_torch(lay, "cuda")
    out, lse = run_cascade_fp8(gpu_lib, lay, q, kc, ks, vc, vs)
    assert torch.isfinite(out.float()).all()
    ro, rl = oracle_full(lay, q, kc, vc, k_scales=ks, v_scales=vs)
    err, rel = assert_close(lay, out_to_f64(out), ro, "shared_prefix_fp8, every sequence")
    say(f"  max-abs {err:.2e} rel-L2 {rel:.2e}")
    assert np.abs(lse.cpu().numpy() - rl).max() < LSE_TOL
    dout, _ = run_decode_fp8(gpu_lib, lay, q, kc, ks, vc, vs)
    assert_close(lay, out_to_f64(out), out_to_f64(dout), "shared_prefix_fp8: cascade vs decode, all sequences")


def test_cascade_fp8_rejects_null_scales(gpu_lib):
    lay = fp8_cascade(2, 3, 32, 20, 32, 8, seed=1)
    q, kc, ks, vc, vs = to_device(*fp8_values_numpy(lay))
    S, Hq, D = q.shape
    lib = gpu_lib.load()
    ch = lay.context_lens.astype(np.int32)
    goh = lay.group_seq_offsets.astype(np.int32)
    plh = lay.prefix_lens.astype(np.int32)
    bt = torch.from_numpy(lay.block_tables).cuda()
    ctx = torch.from_numpy(lay.context_lens).cuda()
    go = torch.from_numpy(goh).cuda()
    pl = torch.from_numpy(plh).cuda()
    ws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    rc = lib.pa_prefix_cascade_fp8(out.data_ptr(), None, q.data_ptr(), kc.data_ptr(), vc.data_ptr(), None,
                                   vs.data_ptr(), bt.data_ptr(), bt.shape[1], ctx.data_ptr(), ch.ctypes.data, S,
                                   len(plh), go.data_ptr(), goh.ctypes.data, pl.data_ptr(), plh.ctypes.data, 8, 4,
                                   128, 16, kc.shape[0], lay.scale, ws.data_ptr(), ws.numel(), None)
    assert rc == gpu_lib.PA_EINVAL
