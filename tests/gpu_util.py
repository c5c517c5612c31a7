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


# Log-sum-exp bound where MFMA tiles attend (shared prefixes, prefill
# chunks): their P.V contraction takes P rounded to bf16 on the bf16 MFMA,
# and the normaliser is summed from the same rounded P (so the weights of
# every output row sum to one).  Rounding to nearest even moves each p by at
# most 2^-9 of itself, so the sum, and exp(lse), by at most 2^-9 relative:
# lse within 2^-9 ~ 1.95e-3.  (The decode kernels sum the float32 p and
# meet 1e-3.)
LSE_TOL_MFMA_BF16 = 2.0e-3
