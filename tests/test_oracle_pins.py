"""Pins for the fp64 oracle: it is checked against closed forms, a library
routine, brute force and invariants -- never against itself.

Each ``pin_*`` helper returns a list of failure strings so that the planted-
mistake tests at the bottom can run every pin against a deliberately broken
oracle and require that some pin notices.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as opa
from workloads import bf16_bits_from_f32, cascade_layout, decode_layout, mixed_layout, values_numpy

# ---------------------------------------------------------------------------
# helpers that build paged inputs from dense per-sequence data (test-owned)
# ---------------------------------------------------------------------------


def scatter_dense(dense_k, dense_v, block_size, num_pages, rng):
    """Place dense per-sequence K/V ([L, Hkv, D] each) into a paged pool.

    Pure-Python loops; the physical page order is a random permutation, and
    every slot not written holds NaN.  Returns (k_pool, v_pool, tables).
    """
    hkv, d = dense_k[0].shape[1], dense_k[0].shape[2]
    kp = np.full((num_pages, hkv, block_size, d), np.nan, dtype=np.float32)
    vp = np.full_like(kp, np.nan)
    free = list(rng.permutation(num_pages))
    mb = max((len(k) + block_size - 1) // block_size for k in dense_k)
    tables = np.full((len(dense_k), mb), -1, dtype=np.int32)
    for s, (K, V) in enumerate(zip(dense_k, dense_v)):
        for t in range(len(K)):
            if t % block_size == 0:
                tables[s, t // block_size] = free.pop()
            page = tables[s, t // block_size]
            for g in range(hkv):
                for j in range(d):
                    kp[page, g, t % block_size, j] = K[t, g, j]
                    vp[page, g, t % block_size, j] = V[t, g, j]
    return kp, vp, tables


def brute_force(q, dense_k, dense_v, q_lens, scale, gqa):
    """Dense softmax attention with Python floats and math.exp.

    Query token i of a sequence with L rows and n new tokens sits at absolute
    position L - n + i and may see keys at positions <= its own.
    """
    outs, lses = [], []
    tok = 0
    for K, V, n in zip(dense_k, dense_v, q_lens):
        L = len(K)
        for i in range(n):
            pos = L - n + i
            for h in range(q.shape[1]):
                g = h // gqa
                xs = []
                for t in range(L):
                    if t <= pos:
                        acc = 0.0
                        for j in range(q.shape[2]):
                            acc += float(q[tok, h, j]) * float(K[t, g, j])
                        xs.append(float(np.float32(scale)) * acc)
                m = max(xs)
                ws = [math.exp(x - m) for x in xs]
                z = sum(ws)
                o = [sum(ws[t] * float(V[t, g, j]) for t in range(len(ws))) / z for j in range(q.shape[2])]
                outs.append(o)
                lses.append(m + math.log(z))
            tok += 1
    return np.array(outs), np.array(lses)


def random_dense_case(rng, n_seq, max_len, hkv, gqa, d, chunks=False):
    lens = [int(rng.integers(1, max_len + 1)) for _ in range(n_seq)]
    qls = [int(rng.integers(1, L + 1)) if chunks else 1 for L in lens]
    dk = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    dv = [rng.standard_normal((L, hkv, d)).astype(np.float32) for L in lens]
    q = rng.standard_normal((sum(qls), hkv * gqa, d)).astype(np.float32)
    return lens, qls, dk, dv, q


# ---------------------------------------------------------------------------
# pins, each returning failures
# ---------------------------------------------------------------------------


def pin_bruteforce(o=opa, seed=0, n_cases=6, chunks=False):
    fails = []
    rng = np.random.default_rng(seed)
    for c in range(n_cases):
        gqa = [1, 2, 4][c % 3]
        hkv = 2 if gqa < 4 else 1
        lens, qls, dk, dv, q = random_dense_case(rng, 3, 40, hkv, gqa, 8, chunks)
        bs = [1, 4, 16][c % 3]
        need = sum((L + bs - 1) // bs for L in lens)
        kp, vp, bt = scatter_dense(dk, dv, bs, need + 5, rng)
        scale = float(rng.uniform(0.2, 1.0))
        out, lse = o.paged_attention(q, kp, vp, bt, lens, qls, scale, hkv, bs, "f32")
        ro, rl = brute_force(q, dk, dv, qls, scale, gqa)
        err = max(np.abs(out.reshape(-1, 8) - ro).max(), np.abs(lse.reshape(-1) - rl).max())
        if not err < 1e-12:
            fails.append(f"bruteforce case {c}: err {err}")
    return fails


def _single(o, q_rows, K, V, scale, bs=16):
    """Run the oracle on one sequence / one kv-head from dense rows."""
    L, d = K.shape
    kp, vp, bt = scatter_dense([K[:, None, :]], [V[:, None, :]], bs, (L + bs - 1) // bs + 2, np.random.default_rng(1))
    n = q_rows.shape[0]
    out, lse = o.paged_attention(q_rows[:, None, :], kp, vp, bt, [L], [n], scale, 1, bs, "f32")
    return out[:, 0], lse[:, 0]


def pin_closed_forms(o=opa):
    fails = []
    # two keys, scores 0 and ln 3 -> weights 1/4, 3/4, lse = ln 4
    ln3 = np.float32(math.log(3.0))
    K = np.array([[0.0, 0.0], [1.0, 0.0]], dtype=np.float32)
    V = np.array([[4.0, 8.0], [8.0, 4.0]], dtype=np.float32)
    q = np.array([[1.0, 0.0]], dtype=np.float32)
    out, lse = _single(o, q, K, V, float(ln3))
    w1 = math.exp(float(ln3))  # 3, up to the float32 rounding of ln 3
    want = (np.array([4.0, 8.0]) + w1 * np.array([8.0, 4.0])) / (1.0 + w1)
    if not np.allclose(out[0], want, rtol=0, atol=1e-12):
        fails.append(f"two-key out {out[0]} != {want}")
    if not abs(lse[0] - math.log1p(w1)) < 1e-12:
        fails.append(f"two-key lse {lse[0]} != ln(1 + e^s)")
    if not np.allclose(out[0], [7.0, 5.0], rtol=0, atol=1e-6):
        fails.append(f"two-key out {out[0]} != (7, 5)")
    if not abs(lse[0] - math.log(4.0)) < 1e-6:
        fails.append(f"two-key lse {lse[0]} != ln 4")
    rng = np.random.default_rng(3)
    # one-row context returns its V row exactly
    K1 = rng.standard_normal((1, 8)).astype(np.float32)
    V1 = rng.standard_normal((1, 8)).astype(np.float32)
    out, lse = _single(o, rng.standard_normal((1, 8)).astype(np.float32), K1, V1, 0.5)
    if not np.array_equal(out[0], V1[0].astype(np.float64)):
        fails.append("one-row context does not return its V row")
    # constant V returns the constant
    Kc = rng.standard_normal((37, 8)).astype(np.float32)
    Vc = np.full((37, 8), 1.75, dtype=np.float32)
    out, _ = _single(o, 3 * rng.standard_normal((1, 8)).astype(np.float32), Kc, Vc, 0.7)
    if not np.allclose(out[0], 1.75, rtol=0, atol=1e-14):
        fails.append("constant V not returned")
    # q = 0: mean of the visible rows, lse = ln(rows); causal chunk of 5 tokens
    Vr = rng.standard_normal((29, 8)).astype(np.float32)
    out, lse = _single(o, np.zeros((5, 8), dtype=np.float32), Kc[:29], Vr, 0.9)
    for i in range(5):
        vis = 29 - 5 + i + 1
        if not np.allclose(out[i], Vr[:vis].astype(np.float64).mean(0), rtol=0, atol=1e-14):
            fails.append(f"q=0 row {i} is not the mean of {vis} rows")
        if not abs(lse[i] - math.log(vis)) < 1e-13:
            fails.append(f"q=0 row {i} lse {lse[i]} != ln {vis}")
    return fails


def pin_sdpa(o=opa, seed=5):
    """Prefix-free causal chunk against torch's SDPA in float64 on CPU."""
    fails = []
    rng = np.random.default_rng(seed)
    for hkv, gqa, L, bs in [(2, 4, 37, 16), (1, 1, 20, 4), (3, 2, 50, 8)]:
        d = 16
        K = rng.standard_normal((L, hkv, d)).astype(np.float32)
        V = rng.standard_normal((L, hkv, d)).astype(np.float32)
        q = rng.standard_normal((L, hkv * gqa, d)).astype(np.float32)
        kp, vp, bt = scatter_dense([K], [V], bs, (L + bs - 1) // bs + 3, rng)
        scale = 0.3
        out, lse = o.paged_attention(q, kp, vp, bt, [L], [L], scale, hkv, bs, "f32")
        tq = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)  # [H, L, d]
        tk = torch.from_numpy(K.astype(np.float64)).permute(1, 0, 2).repeat_interleave(gqa, dim=0)
        tv = torch.from_numpy(V.astype(np.float64)).permute(1, 0, 2).repeat_interleave(gqa, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, is_causal=True, scale=float(np.float32(scale))
        )
        err = np.abs(out - ref.permute(1, 0, 2).numpy()).max()
        if not err < 1e-12:
            fails.append(f"sdpa mismatch {err} (hkv={hkv}, G={gqa})")
    return fails


def _case(dtype="f32", seed=7, ctx=(1, 15, 16, 17, 40, 77), hq=8, hkv=2, d=16, pool_factor=1.5):
    lay = decode_layout(list(ctx), num_q_heads=hq, num_kv_heads=hkv, head_dim=d, dtype=dtype,
                        pool_factor=pool_factor, seed=seed, value_std=1.0)
    q, k, v = values_numpy(lay)
    return lay, q, k, v


def pin_permutation(o=opa):
    fails = []
    lay, q, k, v = _case()
    args = (lay.scale, lay.num_kv_heads, lay.block_size, lay.dtype)
    out, lse = o.decode(q, k, v, lay.block_tables, lay.context_lens, *args)
    pi = np.random.default_rng(11).permutation(lay.num_pages)
    k2 = np.empty_like(k)
    v2 = np.empty_like(v)
    k2[pi] = k
    v2[pi] = v
    bt2 = np.where(lay.block_tables >= 0, pi[np.maximum(lay.block_tables, 0)], -1).astype(np.int32)
    out2, lse2 = o.decode(q, k2, v2, bt2, lay.context_lens, *args)
    if not (np.array_equal(out, out2) and np.array_equal(lse, lse2)):
        fails.append("page relabelling changed the result")
    return fails


def pin_split_merge(o=opa, seed=13):
    fails = []
    rng = np.random.default_rng(seed)
    for L in [2, 17, 100, 333]:
        K = rng.standard_normal((L, 32))
        V = rng.standard_normal((L, 32))
        qv = 2.0 * rng.standard_normal(32)
        full = o.attend(qv, K, V, 0.4)
        cuts = sorted(set(rng.integers(0, L + 1, size=4).tolist()) | {0, L})
        parts = [o.attend(qv, K[a:b], V[a:b], 0.4) for a, b in zip(cuts[:-1], cuts[1:])]
        parts.append(o.attend(qv, K[:0], V[:0], 0.4))  # an empty split
        m = o.lse_merge(parts)
        if not (np.abs(m[0] - full[0]).max() < 1e-12 and abs(m[1] - full[1]) < 1e-12):
            fails.append(f"split/merge differs at L={L}")
        # a non-contiguous partition merges to the same result as well
        idx = rng.permutation(L)
        a, b = np.sort(idx[: L // 2]), np.sort(idx[L // 2 :])
        m2 = o.lse_merge([o.attend(qv, K[a], V[a], 0.4), o.attend(qv, K[b], V[b], 0.4)])
        if not (np.abs(m2[0] - full[0]).max() < 1e-12 and abs(m2[1] - full[1]) < 1e-12):
            fails.append(f"interleaved split/merge differs at L={L}")
    return fails


def pin_gqa_mapping(o=opa):
    """GQA (Hq=8, Hkv=2) equals MHA whose kv-head h is GQA kv-head h // 4."""
    fails = []
    lay, q, k, v = _case(hq=8, hkv=2)
    args = (lay.scale, 2, lay.block_size, lay.dtype)
    out, lse = o.decode(q, k, v, lay.block_tables, lay.context_lens, *args)
    k8 = np.repeat(k, 4, axis=1)
    v8 = np.repeat(v, 4, axis=1)
    out8, lse8 = o.decode(q, k8, v8, lay.block_tables, lay.context_lens, lay.scale, 8, lay.block_size, lay.dtype)
    if not (np.array_equal(out, out8) and np.array_equal(lse, lse8)):
        fails.append("GQA head mapping differs from the expanded MHA")
    return fails


def pin_mixed_vs_decode(o=opa):
    fails = []
    lay = mixed_layout(chunk_prefixes=[0, 19], chunk_len=9, decode_ctx=[5, 33, 16], num_q_heads=4,
                       num_kv_heads=2, head_dim=16, dtype="bf16", seed=3)
    q, k, v = values_numpy(lay)
    out, lse = o.mixed_chunk(q, k, v, lay.block_tables, lay.context_lens, lay.q_lens, lay.scale, 2, 16, "bf16")
    cu = lay.cu_q_lens
    dec_rows = [cu[s] for s in range(2, 5)]
    od, ld = o.decode(q[dec_rows], k, v, lay.block_tables[2:], lay.context_lens[2:], lay.scale, 2, 16, "bf16")
    if not (np.array_equal(out[dec_rows], od) and np.array_equal(lse[dec_rows], ld)):
        fails.append("decode rows of a mixed batch differ from decode")
    # the last token of each chunk sees the whole context: it equals decode
    for s in range(2):
        last = cu[s + 1] - 1
        o1, l1 = o.decode(q[[last]], k, v, lay.block_tables[[s]], lay.context_lens[[s]], lay.scale, 2, 16, "bf16")
        if not np.array_equal(out[[last]], o1):
            fails.append(f"last chunk token of segment {s} differs from decode")
    return fails


ALL_PINS = [pin_bruteforce, pin_closed_forms, pin_sdpa, pin_permutation, pin_split_merge,
            pin_gqa_mapping, pin_mixed_vs_decode]

# ---------------------------------------------------------------------------
# the tests
# ---------------------------------------------------------------------------


def test_bf16_widening_is_exact():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F7F, 0x8000], dtype=np.uint16)
    want = [1.0, -2.0, 1.0 + 2.0**-7, 2.0**-133, (2.0 - 2.0**-7) * 2.0**127, -0.0]
    got = opa.stored_to_f64(bits, "bf16")
    assert got.tolist() == want
    assert math.copysign(1.0, got[-1]) == -1.0


def test_generator_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        np.array([1 + 2.0**-8, 1 + 3 * 2.0**-8, -(1 + 2.0**-8), 3.0e38], dtype=np.float32),
    ])
    ours = bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert ours[-4] == 0x3F80 and ours[-3] == 0x3F82  # ties go to even


def test_bruteforce_decode():
    assert pin_bruteforce() == []


def test_bruteforce_chunks():
    assert pin_bruteforce(seed=1, chunks=True) == []


def test_closed_forms():
    assert pin_closed_forms() == []


def test_sdpa_causal_chunk():
    assert pin_sdpa() == []


def test_page_relabelling_invariance():
    assert pin_permutation() == []


def test_split_merge_equals_unsplit():
    assert pin_split_merge() == []


def test_gqa_mapping():
    assert pin_gqa_mapping() == []


def test_mixed_matches_decode():
    assert pin_mixed_vs_decode() == []


def test_cascade_equals_full_attention():
    lay = cascade_layout(num_groups=3, seqs_per_group=4, prefix_len=32, suffix_lo=1, suffix_hi=40,
                         num_q_heads=4, num_kv_heads=2, head_dim=16, seed=2)
    q, k, v = values_numpy(lay)
    args = (lay.scale, 2, 16, "bf16")
    oc, lc = oracle.prefix_cascade(q, k, v, lay.block_tables, lay.context_lens, *args,
                                   lay.group_seq_offsets, lay.prefix_lens)
    # the prefix/suffix merge identity, spelled out per (sequence, head)
    for s in [0, 5, 11]:
        L, P = int(lay.context_lens[s]), int(lay.prefix_lens[s // 4])
        for h in range(4):
            K = opa.gather_rows(k, lay.block_tables[s], h // 2, L, 16, "bf16")
            V = opa.gather_rows(v, lay.block_tables[s], h // 2, L, 16, "bf16")
            qv = opa.stored_to_f64(q[s, h], "bf16")
            m = opa.lse_merge([opa.attend(qv, K[:P], V[:P], lay.scale), opa.attend(qv, K[P:], V[P:], lay.scale)])
            assert np.abs(m[0] - oc[s, h]).max() < 1e-12 and abs(m[1] - lc[s, h]) < 1e-12
    # a member whose table does not share the prefix is rejected
    bad = lay.block_tables.copy()
    bad[5, 0], bad[5, 1] = bad[5, 1], bad[5, 0]
    with pytest.raises(ValueError):
        oracle.prefix_cascade(q, k, v, bad, lay.context_lens, *args, lay.group_seq_offsets, lay.prefix_lens)


def test_table_checker_flags_problems():
    lay = decode_layout([20, 33], num_q_heads=2, num_kv_heads=1, head_dim=8, dtype="f32", seed=1)
    assert oracle.check_block_tables(lay.block_tables, lay.context_lens, lay.num_pages, 16) == []
    bt = lay.block_tables.copy()
    bt[1, 0] = bt[0, 0]
    assert any("also used" in p for p in oracle.check_block_tables(bt, lay.context_lens, lay.num_pages, 16))
    bt = lay.block_tables.copy()
    bt[0, 1] = lay.num_pages
    assert any("out of range" in p for p in oracle.check_block_tables(bt, lay.context_lens, lay.num_pages, 16))


def test_nan_poison_never_reaches_the_oracle():
    lay, q, k, v = _case(dtype="bf16")
    assert np.isnan(opa.stored_to_f64(k, "bf16")).any()  # the pool is poisoned
    out, lse = oracle.decode(q, k, v, lay.block_tables, lay.context_lens, lay.scale, 2, 16, "bf16")
    assert np.isfinite(out).all() and np.isfinite(lse).all()


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin
# ---------------------------------------------------------------------------


def _run_pins_with(monkeypatch, name, fn):
    monkeypatch.setattr(opa, name, fn)
    fails = []
    for pin in ALL_PINS:
        try:
            fails += pin()
        except Exception as e:  # a crash also counts as caught
            fails.append(f"{pin.__name__} raised {e!r}")
    return fails


def _attend_no_scale(qvec, K, V, scale):
    return _orig_attend(qvec, K, V, 1.0)


def _attend_log2(qvec, K, V, scale):
    o, l = _orig_attend(qvec, K, V, scale)
    return o, l / math.log(2.0)


def _attend_drop_last(qvec, K, V, scale):
    n = K.shape[0]
    return _orig_attend(qvec, K[: max(n - 1, 1)], V[: max(n - 1, 1)], scale)


_orig_attend = opa.attend
_orig_gather = opa.gather_rows


def _gather_wrong_head(pool, table_row, kv_head, n_rows, block_size, dtype):
    return _orig_gather(pool, table_row, (kv_head + 1) % pool.shape[1], n_rows, block_size, dtype)


def _gather_slot_off_by_one(pool, table_row, kv_head, n_rows, block_size, dtype):
    t = np.arange(n_rows)
    pages = np.asarray(table_row)[t // block_size]
    slots = (t + 1) % block_size
    return opa.stored_to_f64(pool[pages, kv_head, slots, :], dtype)


@pytest.mark.parametrize(
    "name,fn",
    [
        ("attend", _attend_no_scale),
        ("attend", _attend_log2),
        ("attend", _attend_drop_last),
        ("gather_rows", _gather_wrong_head),
        ("gather_rows", _gather_slot_off_by_one),
    ],
)
def test_planted_mistake_is_caught(monkeypatch, name, fn):
    assert _run_pins_with(monkeypatch, name, fn), f"no pin noticed a broken {name}"
