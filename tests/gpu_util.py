"""Helpers for the GPU parity tests: move seeded inputs to the device, run
the library, bring inputs back for the oracle."""

import numpy as np
import torch

from workloads import Layout, values_numpy, values_torch


def to_device_values(lay: Layout, q, k, v):
    """numpy values (float32 or bf16 bit patterns) -> device tensors."""
    def conv(a):
        if lay.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()
    return conv(q), conv(k), conv(v)


def to_host_values(lay: Layout, t):
    """device tensor -> numpy in the oracle's stored form."""
    if lay.dtype == "bf16":
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.float().cpu().numpy()


def device_inputs(lay: Layout, host_values=True):
    """(q, k, v) on the device plus host copies (None when drawn on device)."""
    if host_values:
        qh, kh, vh = values_numpy(lay)
        return to_device_values(lay, qh, kh, vh), (qh, kh, vh)
    return values_torch(lay, "cuda"), None


def tables_to_device(lay: Layout):
    bt = torch.from_numpy(lay.block_tables).cuda()
    ctx = torch.from_numpy(lay.context_lens).cuda()
    return bt, ctx


def oracle_subset(lay: Layout, q_dev, k_dev, v_dev, seqs):
    """Host copies of just the pages the given sequences use, renumbered
    0..n-1 (a page relabelling, which leaves attention unchanged), with the
    matching q rows and table rows."""
    bs = lay.block_size
    cu = lay.cu_q_lens
    pages = []
    rows = []
    for s in seqs:
        n = (int(lay.context_lens[s]) + bs - 1) // bs
        pages.append(lay.block_tables[s, :n])
        rows.extend(range(cu[s], cu[s + 1]))
    uniq = np.unique(np.concatenate(pages))
    remap = {int(p): i for i, p in enumerate(uniq)}
    idx = torch.from_numpy(uniq.astype(np.int64)).cuda()
    k_sub = to_host_values(lay, k_dev.index_select(0, idx))
    v_sub = to_host_values(lay, v_dev.index_select(0, idx))
    q_sub = to_host_values(lay, q_dev[torch.tensor(rows, device=q_dev.device)])
    mb = max(len(p) for p in pages)
    bt = np.full((len(seqs), mb), -1, dtype=np.int32)
    for i, pl in enumerate(pages):
        bt[i, : len(pl)] = [remap[int(p)] for p in pl]
    ctx = lay.context_lens[list(seqs)].astype(np.int32)
    ql = lay.q_lens[list(seqs)].astype(np.int32)
    return q_sub, k_sub, v_sub, bt, ctx, ql


def assert_close(lay: Layout, got, ref, what=""):
    """The parity bar: max-abs 2e-3 (float32 inputs) or 2e-2 (bf16 inputs),
    plus a per-(token, head) relative L2 error of 1e-4 / 1e-2 so that a
    kernel returning near-zero rows for long, nearly-uniform contexts (where
    every |out| is small) cannot pass."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    tol, rel_tol = (2e-3, 1e-4) if lay.dtype == "f32" else (2e-2, 1e-2)
    err = np.abs(got - ref).max()
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)
    rel = (num / den).max()
    assert err <= tol, f"{what}: max-abs error {err:.3e} > {tol}"
    assert rel <= rel_tol, f"{what}: relative L2 error {rel:.3e} > {rel_tol}"
    return err, rel


def out_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


# Log-sum-exp bar for every kernel, 1e-3 absolute (natural log).  Every
# kernel forms lse = m + ln(sum_t p_t) from float32 probabilities p_t =
# 2^(x_t - m) (scores x_t in the log2 domain): no kernel sums the bf16-rounded
# p that P.V uses (rounding to nearest even moves a bf16 value by up to 2^-8
# of itself, so such a sum could be off by ln(1 + 2^-8) ~ 3.9e-3).  What is
# left, for contexts up to 32768 rows:
#  * each score is a float32 sum of D = 128 exact bf16 products:
#    |dx| <= 128 * 2^-24 * scale * sum_d |q_d k_d| -- 2e-5 for these inputs;
#  * each p carries the exp2 instruction's error (about 1 ulp, 2^-23 relative)
#    and every lazy or online rescale one more rounding;
#  * a lane adds at most L / 64 = 512 values, then a tree of 6 levels:
#    (512 + 6) * 2^-24 ~ 3e-5 relative on the sum;
#  * merges of partials add a float32 exp2 / log2 each (~1e-7).
# The sum of these stays below 1e-4, so 1e-3 holds with a wide margin.
LSE_TOL = 1.0e-3


def oracle_full(lay: Layout, q_dev, k_dev, v_dev, seqs=None, k_scales=None, v_scales=None):
    """The fp64 oracle over every token of the given sequences (default: the
    whole batch), computed unit by unit -- (sequence, kv-head) -- on the
    oracle's worker processes when they run (``oracle.parallel``), else in
    this process.  Each sequence's pages are copied from the device in table
    order (from the window's first page on for windowed layouts), so device-
    drawn pools of several GB never need a host copy.  fp8 pools: pass the
    scale tensors.  Returns out [T, Hq, D] and lse [T, Hq] in float64 (NaN
    for tokens of sequences not asked for)."""
    from oracle import parallel

    cu = lay.cu_q_lens
    T, Hq, D = q_dev.shape
    fp8 = k_scales is not None
    W = lay.window

    def fetch(s):
        L = int(lay.context_lens[s])
        lo = L - int(lay.q_lens[s]) + 1 - W if W is not None else 0  # the earliest row a token sees
        first = lo // 16 if lo > 0 else 0
        idx = torch.from_numpy(lay.block_tables[s, first:(L + 15) // 16].astype(np.int64)).to(k_dev.device)
        if fp8:
            kc = k_dev.index_select(0, idx).cpu().numpy()
            vc = v_dev.index_select(0, idx).cpu().numpy()
            return (to_host_values(lay, q_dev[int(cu[s]):int(cu[s + 1])]), kc, vc,
                    k_scales.index_select(0, idx).cpu().numpy(), v_scales.index_select(0, idx).cpu().numpy())
        return (to_host_values(lay, q_dev[int(cu[s]):int(cu[s + 1])]), to_host_values(lay, k_dev.index_select(0, idx)),
                to_host_values(lay, v_dev.index_select(0, idx)))

    out = np.full((T, Hq, D), np.nan)
    lse = np.full((T, Hq), np.nan)
    todo = range(lay.num_seqs) if seqs is None else seqs
    for s, o, l in parallel.batch_attention(fetch, todo, lay.context_lens, lay.q_lens, lay.num_kv_heads, lay.scale,
                                            lay.dtype, window=W, fp8_kv=fp8):
        out[int(cu[s]):int(cu[s + 1])] = o
        lse[int(cu[s]):int(cu[s + 1])] = l
    return out, lse
