"""Parity of pa_prefix_cascade (MFMA prefix + suffix decode + merge) against
the fp64 oracle, and against pa_decode on the same inputs."""

import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (LSE_TOL, assert_close, device_inputs, oracle_full, out_to_f64, to_device_values,
                      to_host_values)
from workloads import bf16_bits_from_f32, cascade_layout, values_numpy, workload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_cascade(pa, lay, q, k, v):
    S, Hq, D = q.shape
    dev = q.device
    bt = torch.from_numpy(lay.block_tables).to(dev)
    ctx = torch.from_numpy(lay.context_lens).to(dev)
    go = torch.from_numpy(lay.group_seq_offsets).to(dev)
    pl = torch.from_numpy(lay.prefix_lens).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((S, Hq), dtype=torch.float32, device=dev)
    total = int(((lay.context_lens + 15) // 16).sum())
    ws = torch.empty(pa.prefix_cascade_workspace_size(S, lay.num_kv_heads, lay.gqa_ratio, D, total),
                     dtype=torch.uint8, device=dev)
    pa.prefix_cascade(out, q, k, v, bt, ctx, lay.context_lens, go, lay.group_seq_offsets, pl, lay.prefix_lens,
                      lay.scale, ws, lse_out=lse)
    torch.cuda.synchronize()
    return out, lse


def run_decode(pa, lay, q, k, v):
    S, Hq, D = q.shape
    bt = torch.from_numpy(lay.block_tables).cuda()
    ctx = torch.from_numpy(lay.context_lens).cuda()
    out = torch.empty_like(q)
    lse = torch.empty((S, Hq), dtype=torch.float32, device="cuda")
    total = int(((lay.context_lens + 15) // 16).sum())
    ws = torch.empty(pa.decode_workspace_size(S, lay.num_kv_heads, lay.gqa_ratio, D, total, 0), dtype=torch.uint8,
                     device="cuda")
    pa.decode(out, q, k, v, bt, ctx, lay.context_lens, lay.scale, ws, lse_out=lse)
    torch.cuda.synchronize()
    return out, lse


def oracle_cascade(lay, qh, kh, vh, seqs=None):
    return oracle.prefix_cascade(qh, kh, vh, lay.block_tables, lay.context_lens, lay.scale, lay.num_kv_heads, 16,
                                 "bf16", lay.group_seq_offsets, lay.prefix_lens, seqs)


@pytest.mark.parametrize(
    "groups,per_group,prefix,suf_hi,hq,hkv",
    [
        (3, 5, 64, 40, 32, 8),       # small groups, short suffixes
        (2, 70, 128, 300, 32, 8),    # 280 rows per kv-head: two row chunks
        (4, 8, 16, 17, 8, 8),        # G = 1, one-page prefix
        (2, 16, 80, 100, 64, 8),     # G = 8, prefix not a multiple of 64 keys
        (1, 33, 2048, 600, 32, 8),   # long prefix, several key splits
        (3, 4, 0, 90, 32, 8),        # no prefix at all
        (2, 12, 96, 70, 128, 8),     # G = 16: suffixes on the matrix-core stream kernel
        (3, 10, 48, 60, 16, 8),      # G = 2: suffixes on the vector stream kernel
    ],
)
def test_cascade_small(gpu_lib, groups, per_group, prefix, suf_hi, hq, hkv):
    lay = cascade_layout(num_groups=groups, seqs_per_group=per_group, prefix_len=prefix, suffix_lo=1,
                         suffix_hi=suf_hi, num_q_heads=hq, num_kv_heads=hkv, head_dim=128, seed=groups + prefix)
    say(f"case cascade groups={groups}x{per_group} prefix={prefix} suffix<= {suf_hi} Hq={hq} Hkv={hkv}")
    (q, k, v), (qh, kh, vh) = device_inputs(lay)
    out, lse = run_cascade(gpu_lib, lay, q, k, v)
    ro, rl = oracle_cascade(lay, qh, kh, vh)
    assert_close(lay, out_to_f64(out), ro, "cascade")
    assert np.abs(lse.cpu().numpy() - rl).max() < LSE_TOL
    dout, dlse = run_decode(gpu_lib, lay, q, k, v)
    assert_close(lay, out_to_f64(out), out_to_f64(dout).astype(np.float64), "cascade vs decode")


def test_cascade_mixed_prefix_lengths(gpu_lib):
    lay = cascade_layout(num_groups=4, seqs_per_group=9, prefix_len=0, suffix_lo=1, suffix_hi=200, num_q_heads=32,
                         num_kv_heads=8, head_dim=128, seed=11, prefix_lens=[0, 512, 32, 1040])
    (q, k, v), (qh, kh, vh) = device_inputs(lay)
    out, lse = run_cascade(gpu_lib, lay, q, k, v)
    ro, rl = oracle_cascade(lay, qh, kh, vh)
    assert_close(lay, out_to_f64(out), ro, "cascade mixed prefixes")
    assert np.abs(lse.cpu().numpy() - rl).max() < LSE_TOL


def test_shared_prefix_workload(gpu_lib):
    """The shared-prefix batch (16 groups x 64 sequences, 2048-token
    prefixes) in the launch configuration the benchmark times: every
    sequence against the oracle, and against pa_decode."""
    lay = workload("shared_prefix")
    say("case shared_prefix seed 0 (every sequence)")
    (q, k, v), _ = device_inputs(lay, host_values=False)
    out, lse = run_cascade(gpu_lib, lay, q, k, v)
    assert torch.isfinite(out.float()).all()
    ro, rl = oracle_full(lay, q, k, v)
    err, rel = assert_close(lay, out_to_f64(out), ro, "shared_prefix, every sequence")
    say(f"  max-abs {err:.2e} rel-L2 {rel:.2e}")
    assert np.abs(lse.cpu().numpy() - rl).max() < LSE_TOL
    dout, _ = run_decode(gpu_lib, lay, q, k, v)
    assert_close(lay, out_to_f64(out), out_to_f64(dout), "shared_prefix: cascade vs decode, all sequences")


def test_cascade_needle_in_prefix_and_suffix(gpu_lib):
    """One key per (sequence, kv-head) dominates: in the shared prefix for
    even kv-heads (the same prefix row for the whole group), in the
    sequence's own suffix for odd ones.  Outputs must be that V row's bits."""
    lay = cascade_layout(num_groups=2, seqs_per_group=6, prefix_len=96, suffix_lo=1, suffix_hi=70, num_q_heads=32,
                         num_kv_heads=8, head_dim=128, seed=3)
    qh, kh, vh = values_numpy(lay)
    kk = np.where(np.isnan(oracle.stored_to_f64(kh, "bf16")), kh, np.uint16(0)).astype(np.uint16)
    big = bf16_bits_from_f32(np.array([64.0], dtype=np.float32))[0]
    qf = np.zeros((lay.num_seqs, 32, 128), dtype=np.float32)
    want = np.zeros((lay.num_seqs, 32, 128), dtype=np.uint16)
    rng = np.random.default_rng(5)
    for gi in range(2):
        for g in range(8):
            if g % 2 == 0:
                t = int(rng.integers(0, 96))
                p = lay.block_tables[gi * 6, t // 16]
                j = g * 7 % 128
                kk[p, g, t % 16, j] = big
                for s in range(gi * 6, gi * 6 + 6):
                    qf[s, g * 4:(g + 1) * 4, j] = 64.0
                    want[s, g * 4:(g + 1) * 4] = vh[p, g, t % 16]
    for s in range(lay.num_seqs):
        L = int(lay.context_lens[s])
        for g in range(1, 8, 2):
            t = int(rng.integers(96, L))
            p = lay.block_tables[s, t // 16]
            j = (s + g) % 128
            kk[p, g, t % 16, j] = big
            qf[s, g * 4:(g + 1) * 4, j] = 64.0
            want[s, g * 4:(g + 1) * 4] = vh[p, g, t % 16]
    qq = bf16_bits_from_f32(qf)
    qd, kd, vd = to_device_values(lay, qq, kk, vh)
    out, _ = run_cascade(gpu_lib, lay, qd, kd, vd)
    got = to_host_values(lay, out)
    ro, _ = oracle_cascade(lay, qq, kk, vh)
    assert np.array_equal(bf16_bits_from_f32(ro.astype(np.float32)), want)
    assert np.array_equal(got, want)


def test_cascade_rejects_bad_groups(gpu_lib):
    lay = cascade_layout(num_groups=2, seqs_per_group=3, prefix_len=32, suffix_lo=1, suffix_hi=20, num_q_heads=32,
                         num_kv_heads=8, head_dim=128, seed=1)
    (q, k, v), _ = device_inputs(lay)
    bad = lay.prefix_lens.copy()
    bad[0] = 40  # not whole pages
    import dataclasses
    lay2 = dataclasses.replace(lay, prefix_lens=bad)
    with pytest.raises(gpu_lib.PAError) as e:
        run_cascade(gpu_lib, lay2, q, k, v)
    assert e.value.code == gpu_lib.PA_EINVAL
    bad = lay.prefix_lens.copy()
    bad[1] = int(lay.context_lens[3:].min()) // 16 * 16 + 16  # not shorter than a member
    lay3 = dataclasses.replace(lay, prefix_lens=bad)
    with pytest.raises(gpu_lib.PAError):
        run_cascade(gpu_lib, lay3, q, k, v)


def test_detected_groups_drive_the_cascade(gpu_lib):
    """End to end: a shared-prefix batch in shuffled order (no group
    structure given), groups found by pa_detect_prefix_groups, the batch
    taken in that order through pa_prefix_cascade, the outputs put back;
    they must match the oracle's plain decode of the shuffled batch."""
    import dataclasses

    base = cascade_layout(num_groups=5, seqs_per_group=12, prefix_len=256, suffix_lo=1, suffix_hi=200,
                          num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16", seed=21)
    perm = np.random.default_rng(8).permutation(base.num_seqs)
    qh, kh, vh = values_numpy(base)
    qh = qh[perm]
    bt, ctx = base.block_tables[perm], base.context_lens[perm]
    say("case cascade over detected groups, 5 x 12 shuffled")
    order, offs, pref = gpu_lib.detect_prefix_groups(bt, ctx)
    assert len(pref) == 5 and (pref == 256).all()
    lay = dataclasses.replace(base, block_tables=bt[order], context_lens=ctx[order], group_seq_offsets=offs,
                              prefix_lens=pref)
    q, k, v = to_device_values(lay, qh[order], kh, vh)
    out, lse = run_cascade(gpu_lib, lay, q, k, v)
    back = np.empty_like(order)
    back[order] = np.arange(len(order))
    got = out_to_f64(out)[back]
    ro, rl = oracle.decode(qh, kh, vh, bt, ctx, base.scale, base.num_kv_heads, 16, "bf16")
    assert_close(lay, got, ro, "cascade over detected groups")
    assert np.abs(lse.cpu().numpy()[back] - rl).max() < LSE_TOL
