"""Pins for the fp8 (e4m3fn) cache oracle: the code table and the quantiser
against torch's own float8_e4m3fn conversion (a library routine) and closed
forms; attention over an fp8 cache against the pinned bf16 attention oracle
and against brute force.

Each ``pin_*`` helper returns a list of failure strings, so the planted-
mistake tests at the bottom can run every pin against a broken oracle and
require that some pin notices.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as f8
from workloads import bf16_bits_from_f32, decode_layout

# ---------------------------------------------------------------------------
# helpers (test-owned)
# ---------------------------------------------------------------------------


def torch_code_values():
    """float32 value of each of the 256 codes, by torch's float8_e4m3fn."""
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def torch_quantize(x):
    """The token-group recipe written with torch ops: float32 scale, divide,
    clamp, float8_e4m3fn cast."""
    t = torch.from_numpy(np.asarray(x, dtype=np.float32))
    s = t.abs().amax(dim=-1).clamp_min(1e-10) / 448.0
    codes = (t / s[..., None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, s.numpy()


def finite_codes(rng, shape):
    """Random e4m3fn codes avoiding the two NaN codes."""
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    nan = (c & 0x7F) == 0x7F
    c[nan] = c[nan] ^ 0x01  # 0x7F -> 0x7E, 0xFF -> 0xFE
    return c


def fp8_cache(rng, ctx, hkv, d, block_size, pow2_scales):
    """A paged fp8 cache: every table a random run of free pages, unused
    pages and tail rows NaN (code 0x7F, scale NaN)."""
    lay = decode_layout(ctx, num_q_heads=hkv * 2, num_kv_heads=hkv, head_dim=d, dtype="bf16",
                        block_size=block_size, pool_factor=1.5, seed=int(rng.integers(1 << 30)))
    npg = lay.num_pages
    kc = np.full((npg, hkv, block_size, d), 0x7F, dtype=np.uint8)
    vc = kc.copy()
    ks = np.full((npg, hkv, block_size), np.nan, dtype=np.float32)
    vs = ks.copy()
    for s, L in enumerate(ctx):
        for t in range(L):
            p, r = lay.block_tables[s, t // block_size], t % block_size
            kc[p, :, r] = finite_codes(rng, (hkv, d))
            vc[p, :, r] = finite_codes(rng, (hkv, d))
            if pow2_scales:
                ks[p, :, r] = 2.0 ** rng.integers(-9, -3, size=hkv)
                vs[p, :, r] = 2.0 ** rng.integers(-9, -3, size=hkv)
            else:
                ks[p, :, r] = rng.uniform(0.5, 2.0, size=hkv).astype(np.float32) / 256
                vs[p, :, r] = rng.uniform(0.5, 2.0, size=hkv).astype(np.float32) / 256
    q = bf16_bits_from_f32(rng.standard_normal((len(ctx), hkv * 2, d)).astype(np.float32))
    return lay, q, kc, ks, vc, vs


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------


def pin_code_table():
    ref = torch_code_values()
    got = f8.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    return [f"code {c:#04x}: {got[c]} vs torch {ref[c]}" for c in np.nonzero(~same)[0][:5]]


def pin_closed_forms():
    fails = []
    v = f8.e4m3_to_f64
    want = {0x38: 1.0, 0x40: 2.0, 0x7E: 448.0, 0xFE: -448.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9,
            0x08: 2.0 ** -6, 0x30: 0.5, 0xB8: -1.0}
    for c, x in want.items():
        if v(np.uint8(c)) != x:
            fails.append(f"code {c:#04x} is {v(np.uint8(c))}, want {x}")
    if not (v(np.uint8(0)) == 0 and not np.signbit(v(np.uint8(0)))):
        fails.append("0x00 is not +0")
    if not (v(np.uint8(0x80)) == 0 and np.signbit(v(np.uint8(0x80)))):
        fails.append("0x80 is not -0")
    for c in (0x7F, 0xFF):
        if not math.isnan(v(np.uint8(c))):
            fails.append(f"code {c:#04x} is not NaN")
    return fails


def quantizer_rows():
    rng = np.random.default_rng(7)
    rows = [rng.standard_normal(128) * 0.5, rng.standard_normal(128) * 1e-3, rng.standard_normal(128) * 300,
            np.zeros(128), rng.uniform(-1, 1, 128) ** 9]
    ties = np.zeros(128)
    ties[0] = 448.0  # scale exactly 1: x / scale = x
    ties[1:8] = [1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -10, 104.0, 0.0]  # halfway cases
    rows.append(ties)
    return np.array(rows, dtype=np.float32)


def pin_quantizer_vs_torch():
    x = quantizer_rows()
    codes, scales = f8.quantize_rows(x)
    rc, rs = torch_quantize(x)
    fails = []
    if not np.array_equal(scales, rs):
        fails.append("scales differ from torch's recipe")
    bad = np.argwhere(codes != rc)
    fails += [f"row {r} col {c}: code {codes[r, c]:#04x} vs torch {rc[r, c]:#04x}" for r, c in bad[:5]]
    return fails


def pin_quantizer_properties():
    x = quantizer_rows()
    codes, scales = f8.quantize_rows(x)
    deq = f8.dequantize(codes, scales)
    fails = []
    for r in range(x.shape[0]):
        amax = float(np.max(np.abs(x[r])))
        if amax == 0:
            if np.any(codes[r] & 0x7F):
                fails.append(f"row {r}: zero row has nonzero codes")
            if scales[r] != np.float32(np.float32(1e-10) / np.float32(448)):
                fails.append(f"row {r}: zero-row scale {scales[r]}")
            continue
        j = int(np.argmax(np.abs(x[r])))
        if abs(f8.e4m3_to_f64(codes[r, j])) != 448.0:
            fails.append(f"row {r}: largest element does not map to +-448")
        # round to nearest: the error is at most half a code step at that
        # magnitude (step 2^(e-3) for normals, 2^-9 for subnormals), scaled
        y = np.abs(x[r].astype(np.float64) / float(scales[r]))
        e = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
        step = 2.0 ** (e - 3)
        # float32 division may round y itself: allow its half-ulp too
        bound = (step / 2 + y * 2.0 ** -24) * float(scales[r])
        if np.any(np.abs(deq[r] - x[r]) > bound * (1 + 1e-12)):
            fails.append(f"row {r}: read-back error above half a code step")
    neg_codes, _ = f8.quantize_rows(-x)
    nz = (codes & 0x7F) != 0
    if not np.array_equal(neg_codes[nz], codes[nz] ^ 0x80):
        fails.append("quantising -x does not flip the sign bit")
    return fails


def pin_attention_vs_bf16_oracle():
    """Power-of-two scales make every read-back value an exact bf16 value;
    attention over the fp8 cache then equals the bf16 oracle over those
    values, bit for bit (same float64 values, same arithmetic)."""
    rng = np.random.default_rng(11)
    ctx = [1, 15, 16, 17, 40]
    lay, q, kc, ks, vc, vs = fp8_cache(rng, ctx, hkv=2, d=16, block_size=16, pow2_scales=True)
    out, lse = f8.decode_fp8(q, kc, ks, vc, vs, lay.block_tables, lay.context_lens, 0.25, 2, 16)
    kd = f8.dequantize(kc, ks)
    vd = f8.dequantize(vc, vs)
    kb = bf16_bits_from_f32(np.nan_to_num(kd).astype(np.float32))
    vb = bf16_bits_from_f32(np.nan_to_num(vd).astype(np.float32))
    fails = []
    used = np.isfinite(kd)
    if not np.array_equal(oracle.stored_to_f64(kb, "bf16")[used], kd[used]):
        fails.append("power-of-two read-back values are not exact bf16 values")
    ro, rl = oracle.decode(q, kb, vb, lay.block_tables, lay.context_lens, 0.25, 2, 16, "bf16")
    if not (np.array_equal(out, ro) and np.array_equal(lse, rl)):
        fails.append(f"fp8 attention differs from bf16 attention: {np.nanmax(np.abs(out - ro)):.3e}")
    return fails


def pin_bruteforce():
    """Tiny inputs: codes read through torch's float8 conversion, dense K/V
    assembled with Python loops, softmax with math.exp."""
    rng = np.random.default_rng(5)
    ctx = [3, 18, 33]
    hkv, d, bs = 2, 8, 16
    lay, q, kc, ks, vc, vs = fp8_cache(rng, ctx, hkv=hkv, d=d, block_size=bs, pow2_scales=False)
    out, lse = f8.decode_fp8(q, kc, ks, vc, vs, lay.block_tables, lay.context_lens, 0.3, hkv, bs)
    cv = torch_code_values()
    qf = oracle.stored_to_f64(q, "bf16")
    sc = float(np.float32(0.3))
    fails = []
    for s, L in enumerate(ctx):
        for h in range(hkv * 2):
            g = h // 2
            xs, vrows = [], []
            for t in range(L):
                p, r = int(lay.block_tables[s, t // bs]), t % bs
                k = [cv[kc[p, g, r, j]] * float(ks[p, g, r]) for j in range(d)]
                vrows.append([cv[vc[p, g, r, j]] * float(vs[p, g, r]) for j in range(d)])
                xs.append(sc * sum(qf[s, h, j] * k[j] for j in range(d)))
            m = max(xs)
            w = [math.exp(x - m) for x in xs]
            z = sum(w)
            o = [sum(w[t] * vrows[t][j] for t in range(L)) / z for j in range(d)]
            if np.max(np.abs(np.array(o) - out[s, h])) > 1e-12 or abs(m + math.log(z) - lse[s, h]) > 1e-12:
                fails.append(f"seq {s} head {h} differs from brute force")
    return fails


def multi_q(rng, ctx, q_len, hq, d):
    return bf16_bits_from_f32(rng.standard_normal((len(ctx) * q_len, hq, d)).astype(np.float32))


def pin_multi_token_reductions():
    """q_len 1 is decode_fp8 bit for bit; with power-of-two scales the
    result equals the (pinned) chunk oracle over the read-back bf16 values,
    each sequence a segment of q_len tokens, bit for bit."""
    rng = np.random.default_rng(21)
    fails = []
    ctx = [3, 16, 17, 40, 70]
    lay, q1, kc, ks, vc, vs = fp8_cache(rng, ctx, hkv=2, d=16, block_size=16, pow2_scales=True)
    a = f8.decode_multi_fp8(q1, kc, ks, vc, vs, lay.block_tables, lay.context_lens, 1, 0.25, 2, 16)
    b = f8.decode_fp8(q1, kc, ks, vc, vs, lay.block_tables, lay.context_lens, 0.25, 2, 16)
    if not (np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])):
        fails.append("q_len 1 differs from decode_fp8")
    kb = bf16_bits_from_f32(np.nan_to_num(f8.dequantize(kc, ks)).astype(np.float32))
    vb = bf16_bits_from_f32(np.nan_to_num(f8.dequantize(vc, vs)).astype(np.float32))
    for n in (2, 3):
        q = multi_q(rng, ctx, n, 4, 16)
        out, lse = f8.decode_multi_fp8(q, kc, ks, vc, vs, lay.block_tables, lay.context_lens, n, 0.25, 2, 16)
        ro, rl = oracle.mixed_chunk(q, kb, vb, lay.block_tables, lay.context_lens, [n] * len(ctx), 0.25, 2, 16,
                                    "bf16")
        if not (np.array_equal(out, ro) and np.array_equal(lse, rl)):
            fails.append(f"q_len {n}: differs from the chunk oracle on read-back values")
    return fails


def pin_multi_token_bruteforce():
    """Tiny inputs, Python loops: token i sees rows 0 .. L - q_len + i."""
    rng = np.random.default_rng(9)
    ctx = [2, 17, 20]
    hkv, d, bs, n = 1, 4, 16, 2
    lay, _, kc, ks, vc, vs = fp8_cache(rng, ctx, hkv=hkv, d=d, block_size=bs, pow2_scales=False)
    q = multi_q(rng, ctx, n, 2, d)
    out, lse = f8.decode_multi_fp8(q, kc, ks, vc, vs, lay.block_tables, lay.context_lens, n, 0.5, hkv, bs)
    cv = torch_code_values()
    qf = oracle.stored_to_f64(q, "bf16")
    sc = float(np.float32(0.5))
    fails = []
    for s, L in enumerate(ctx):
        for i in range(n):
            for h in range(2):
                xs, vrows = [], []
                for t in range(L - n + i + 1):
                    p, r = int(lay.block_tables[s, t // bs]), t % bs
                    k = [cv[kc[p, 0, r, j]] * float(ks[p, 0, r]) for j in range(d)]
                    vrows.append([cv[vc[p, 0, r, j]] * float(vs[p, 0, r]) for j in range(d)])
                    xs.append(sc * sum(qf[s * n + i, h, j] * k[j] for j in range(d)))
                m = max(xs)
                w = [math.exp(x - m) for x in xs]
                z = sum(w)
                o = [sum(w[t] * vrows[t][j] for t in range(len(w))) / z for j in range(d)]
                if np.max(np.abs(np.array(o) - out[s * n + i, h])) > 1e-12 or \
                        abs(m + math.log(z) - lse[s * n + i, h]) > 1e-12:
                    fails.append(f"seq {s} token {i} head {h} differs from brute force")
    return fails


def pin_mixed_reductions():
    """A mixed batch (q_lens per segment): all ones is decode_fp8 and a
    uniform q_len is decode_multi_fp8, bit for bit; with power-of-two scales
    a ragged batch (decode tokens and chunks of 3 to 16 tokens) equals the
    (pinned) chunk oracle over the read-back bf16 values, bit for bit."""
    rng = np.random.default_rng(31)
    fails = []
    ctx = [3, 16, 17, 40, 70]
    lay, q1, kc, ks, vc, vs = fp8_cache(rng, ctx, hkv=2, d=16, block_size=16, pow2_scales=True)
    bt, cl = lay.block_tables, lay.context_lens
    a = f8.mixed_chunk_fp8(q1, kc, ks, vc, vs, bt, cl, [1] * len(ctx), 0.25, 2, 16)
    b = f8.decode_fp8(q1, kc, ks, vc, vs, bt, cl, 0.25, 2, 16)
    if not (np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])):
        fails.append("all-ones q_lens differ from decode_fp8")
    q3 = multi_q(rng, ctx, 3, 4, 16)
    a = f8.mixed_chunk_fp8(q3, kc, ks, vc, vs, bt, cl, [3] * len(ctx), 0.25, 2, 16)
    b = f8.decode_multi_fp8(q3, kc, ks, vc, vs, bt, cl, 3, 0.25, 2, 16)
    if not (np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])):
        fails.append("a uniform q_len differs from decode_multi_fp8")
    kb = bf16_bits_from_f32(np.nan_to_num(f8.dequantize(kc, ks)).astype(np.float32))
    vb = bf16_bits_from_f32(np.nan_to_num(f8.dequantize(vc, vs)).astype(np.float32))
    ql = [1, 3, 1, 16, 5]
    q = bf16_bits_from_f32(rng.standard_normal((sum(ql), 4, 16)).astype(np.float32))
    out, lse = f8.mixed_chunk_fp8(q, kc, ks, vc, vs, bt, cl, ql, 0.25, 2, 16)
    ro, rl = oracle.mixed_chunk(q, kb, vb, bt, cl, ql, 0.25, 2, 16, "bf16")
    if not (np.array_equal(out, ro) and np.array_equal(lse, rl)):
        fails.append("ragged q_lens: differs from the chunk oracle on read-back values")
    return fails


def pin_mixed_bruteforce():
    """Tiny ragged batch, Python loops: segment s's tokens follow those of
    the segments before it in q; token i sees rows 0 .. L - n + i."""
    rng = np.random.default_rng(12)
    ctx, ql = [2, 17, 20], [2, 1, 3]
    hkv, d, bs = 1, 4, 16
    lay, _, kc, ks, vc, vs = fp8_cache(rng, ctx, hkv=hkv, d=d, block_size=bs, pow2_scales=False)
    q = bf16_bits_from_f32(rng.standard_normal((sum(ql), 2, d)).astype(np.float32))
    out, lse = f8.mixed_chunk_fp8(q, kc, ks, vc, vs, lay.block_tables, lay.context_lens, ql, 0.5, hkv, bs)
    cv = torch_code_values()
    qf = oracle.stored_to_f64(q, "bf16")
    sc = float(np.float32(0.5))
    fails = []
    row = 0
    for s, L in enumerate(ctx):
        n = ql[s]
        for i in range(n):
            for h in range(2):
                xs, vrows = [], []
                for t in range(L - n + i + 1):
                    p, r = int(lay.block_tables[s, t // bs]), t % bs
                    k = [cv[kc[p, 0, r, j]] * float(ks[p, 0, r]) for j in range(d)]
                    vrows.append([cv[vc[p, 0, r, j]] * float(vs[p, 0, r]) for j in range(d)])
                    xs.append(sc * sum(qf[row, h, j] * k[j] for j in range(d)))
                m = max(xs)
                w = [math.exp(x - m) for x in xs]
                z = sum(w)
                o = [sum(w[t] * vrows[t][j] for t in range(len(w))) / z for j in range(d)]
                if np.max(np.abs(np.array(o) - out[row, h])) > 1e-12 or abs(m + math.log(z) - lse[row, h]) > 1e-12:
                    fails.append(f"segment {s} token {i} head {h} differs from brute force")
            row += 1
    return fails


ALL_PINS = [pin_code_table, pin_closed_forms, pin_quantizer_vs_torch, pin_quantizer_properties,
            pin_attention_vs_bf16_oracle, pin_bruteforce, pin_multi_token_reductions, pin_multi_token_bruteforce,
            pin_mixed_reductions, pin_mixed_bruteforce]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    fails = pin()
    assert not fails, fails


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin
# ---------------------------------------------------------------------------


def _fnuz_table():
    t = np.array([0.0] * 256)
    for c in range(256):
        e, m, sgn = (c >> 3) & 0xF, c & 7, -1.0 if c & 0x80 else 1.0
        t[c] = sgn * (m / 8 * 2.0 ** -7 if e == 0 else (1 + m / 8) * 2.0 ** (e - 8))
    t[0x80] = math.nan
    return t


def _ignore_scale(codes, scales):
    return f8.e4m3_to_f64(codes) * np.where(np.isnan(np.asarray(scales, dtype=np.float64)), np.nan, 1.0)[..., None]


def _round_ties_away(y):
    y = np.asarray(y, dtype=np.float64)
    codes = np.array([c for c in range(256) if not math.isnan(f8.E4M3_TABLE[c])])
    vals = f8.E4M3_TABLE[codes]
    flat = y.reshape(-1)
    d = np.abs(vals[None, :] - flat[:, None])
    cand = (d == d.min(axis=1, keepdims=True)) & (np.signbit(vals)[None, :] == np.signbit(flat)[:, None])
    mag = np.where(cand, np.abs(vals)[None, :], -1.0)
    return codes[np.argmax(mag, axis=1)].astype(np.uint8).reshape(y.shape)


PLANTED = {
    "fnuz_bias_8": ("E4M3_TABLE", _fnuz_table()),
    "scale_ignored": ("dequantize", _ignore_scale),
    "ties_away_from_zero": ("round_to_e4m3", _round_ties_away),
}


def _run_pins():
    """Names of the pins that fail (a pin that raises counts as failing)."""
    failed = []
    for p in ALL_PINS:
        try:
            bad = p()
        except (IndexError, ValueError) as e:
            bad = [f"raised {e!r}"]
        if bad:
            failed.append(p.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(PLANTED))
def test_planted_mistake_is_caught(monkeypatch, name):
    attr, bad = PLANTED[name]
    monkeypatch.setattr(f8, attr, bad)
    assert _run_pins(), f"no pin noticed {name}"


def test_planted_v_scale_swap_is_caught(monkeypatch):
    orig = f8.decode_fp8

    def swapped(q, kc, ks, vc, vs, *a, **kw):
        return orig(q, kc, ks, vc, ks, *a, **kw)

    monkeypatch.setattr(f8, "decode_fp8", swapped)
    assert _run_pins(), "no pin noticed the K scale used for V"


def test_kv_append_fp8_bruteforce_and_read_back():
    """Tiny mixed batch: every new row's codes and scale, found by a Python
    loop over tokens and kv-heads (torch's recipe for the codes), sit at its
    row of its page; every other row keeps its bits; reading the written
    rows back is within half a code step of the new values."""
    from workloads import mixed_layout

    lay = mixed_layout(chunk_prefixes=[0, 7], chunk_len=9, decode_ctx=[1, 16, 17, 40], num_q_heads=4,
                       num_kv_heads=2, head_dim=16, dtype="bf16", name="append_fp8")
    rng = np.random.default_rng(2)
    npg, hkv, bs, d = lay.num_pages, 2, 16, 16
    kc = rng.integers(0, 126, size=(npg, hkv, bs, d)).astype(np.uint8)
    vc = rng.integers(0, 126, size=(npg, hkv, bs, d)).astype(np.uint8)
    ks = rng.uniform(0.1, 1, size=(npg, hkv, bs)).astype(np.float32)
    vs = rng.uniform(0.1, 1, size=(npg, hkv, bs)).astype(np.float32)
    T = lay.num_tokens
    kn = bf16_bits_from_f32((rng.standard_normal((T, hkv, d)) * 3).astype(np.float32))
    vn = bf16_bits_from_f32((rng.standard_normal((T, hkv, d)) * 0.01).astype(np.float32))
    got = f8.kv_append_fp8(kc, ks, vc, vs, kn, vn, lay.block_tables, lay.context_lens, lay.q_lens, 16, "bf16")
    want = [kc.copy(), ks.copy(), vc.copy(), vs.copy()]
    touched = set()
    t = 0
    for s in range(lay.num_seqs):
        L, n = int(lay.context_lens[s]), int(lay.q_lens[s])
        for i in range(n):
            pos = L - n + i
            p, r = int(lay.block_tables[s, pos // 16]), pos % 16
            touched.add((p, r))
            for g in range(hkv):
                for new, ci, si in ((kn, 0, 1), (vn, 2, 3)):
                    row = oracle.stored_to_f64(new[t + i, g], "bf16").astype(np.float32)
                    codes, scale = torch_quantize(row[None, :])
                    want[ci][p, g, r] = codes[0]
                    want[si][p, g, r] = scale[0]
        t += n
    for a, b in zip(got, want):
        assert np.array_equal(a, b)
    # read-back of the written rows: within half a code step of the new value
    t = 0
    for s in range(lay.num_seqs):
        L, n = int(lay.context_lens[s]), int(lay.q_lens[s])
        for i in range(n):
            pos = L - n + i
            p, r = int(lay.block_tables[s, pos // 16]), pos % 16
            for g in range(hkv):
                for new, ci, si in ((kn, 0, 1), (vn, 2, 3)):
                    x = oracle.stored_to_f64(new[t + i, g], "bf16")
                    sc = float(got[si][p, g, r])
                    back = f8.dequantize(got[ci][p, g, r][None], got[si][p, g, r][None])[0]
                    y = np.abs(x) / sc
                    step = 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 3)
                    assert np.all(np.abs(back - x) <= (step / 2 + y * 2.0 ** -24) * sc * (1 + 1e-12))
        t += n


@pytest.mark.parametrize("name,bad", [("sees one row more", lambda L, n, i: L - n + i + 2),
                                      ("sees one row less", lambda L, n, i: L - n + i),
                                      ("tokens reversed", lambda L, n, i: L - i)])
def test_planted_multi_token_mistake_is_caught(monkeypatch, name, bad):
    monkeypatch.setattr(f8, "_visible", bad)
    assert _run_pins(), f"no pin noticed: {name}"


def test_planted_segment_offsets_are_caught(monkeypatch):
    """Segments read from q at the offsets the q_lens would have in ascending
    order (every row index stays in range, so a pin must notice the values)."""
    monkeypatch.setattr(f8, "_segment_starts",
                        lambda ql: np.concatenate([[0], np.cumsum(np.sort(np.asarray(ql, dtype=np.int64)))]))
    assert _run_pins(), "no pin noticed segments read at the wrong offsets"


# ---------------------------------------------------------------------------
# shared-prefix (cascade) decode over an fp8 cache
# ---------------------------------------------------------------------------


def _cascade_case(seed=11):
    from workloads import cascade_layout, fp8_values_numpy

    lay = cascade_layout(num_groups=3, seqs_per_group=3, prefix_len=48, suffix_lo=1, suffix_hi=40, num_q_heads=8,
                         num_kv_heads=2, head_dim=32, seed=seed, prefix_lens=[48, 16, 64])
    lay.kv_dtype = "fp8"
    return lay, fp8_values_numpy(lay)


def pin_cascade_is_prefix_merge_suffix():
    """Attention over prefix + suffix equals the log-sum-exp merge of the
    fp8 attention over the shared prefix rows alone (table cut at the
    prefix) and over each member's suffix rows alone (table shifted past the
    prefix, which ends on a page boundary), within fp64 rounding."""
    lay, (q, kc, ks, vc, vs) = _cascade_case()
    out, lse = oracle.prefix_cascade_fp8(q, kc, ks, vc, vs, lay.block_tables, lay.context_lens, lay.scale,
                                         lay.num_kv_heads, 16, lay.group_seq_offsets, lay.prefix_lens)
    per_seq_prefix = np.repeat(lay.prefix_lens, np.diff(lay.group_seq_offsets))
    fails = []
    for s in range(lay.num_seqs):
        P, L = int(per_seq_prefix[s]), int(lay.context_lens[s])
        parts = []
        if P > 0:
            po, pl = f8.decode_fp8(q[s:s + 1], kc, ks, vc, vs, lay.block_tables[s:s + 1], np.array([P]), lay.scale,
                                   lay.num_kv_heads, 16)
            parts.append((po[0], pl[0]))
        bt = np.full_like(lay.block_tables[s:s + 1], -1)
        n = (L + 15) // 16 - P // 16
        bt[0, :n] = lay.block_tables[s, P // 16:(L + 15) // 16]
        so, sl = f8.decode_fp8(q[s:s + 1], kc, ks, vc, vs, bt, np.array([L - P]), lay.scale, lay.num_kv_heads, 16)
        parts.append((so[0], sl[0]))
        for h in range(lay.num_q_heads):
            mo, ml = oracle.lse_merge([(o[h], l[h]) for o, l in parts])
            if not (np.max(np.abs(mo - out[s, h])) <= 1e-12 and abs(ml - lse[s, h]) <= 1e-12):
                fails.append(f"seq {s} head {h}: cascade != prefix (+) suffix")
    return fails


def pin_cascade_checks_groups():
    """A member whose prefix entries differ from its group's is rejected."""
    lay, (q, kc, ks, vc, vs) = _cascade_case(seed=12)
    bt = lay.block_tables.copy()
    bt[1, 0] = bt[lay.group_seq_offsets[1], 0]  # member 1 of group 0 names group 1's first prefix page
    try:
        oracle.prefix_cascade_fp8(q, kc, ks, vc, vs, bt, lay.context_lens, lay.scale, lay.num_kv_heads, 16,
                                  lay.group_seq_offsets, lay.prefix_lens)
    except ValueError:
        return []
    return ["an unshared prefix was accepted"]


CASCADE_PINS = [pin_cascade_is_prefix_merge_suffix, pin_cascade_checks_groups]


@pytest.mark.parametrize("pin", CASCADE_PINS, ids=lambda p: p.__name__)
def test_cascade_pin(pin):
    fails = pin()
    assert not fails, fails[:5]


def _cascade_prefix_only(q, kc, ks, vc, vs, bt, ctx, scale, hkv, bs, go, pl, q_dtype="bf16", seqs=None):
    per = np.repeat(np.asarray(pl), np.diff(np.asarray(go)))
    return f8.decode_fp8(q, kc, ks, vc, vs, bt, np.maximum(per, 1), scale, hkv, bs, q_dtype, seqs)


def _cascade_no_check(q, kc, ks, vc, vs, bt, ctx, scale, hkv, bs, go, pl, q_dtype="bf16", seqs=None):
    return f8.decode_fp8(q, kc, ks, vc, vs, bt, ctx, scale, hkv, bs, q_dtype, seqs)


def _cascade_prefix_twice(q, kc, ks, vc, vs, bt, ctx, scale, hkv, bs, go, pl, q_dtype="bf16", seqs=None):
    per = np.repeat(np.asarray(pl), np.diff(np.asarray(go)))
    out, lse = f8.decode_fp8(q, kc, ks, vc, vs, bt, ctx, scale, hkv, bs, q_dtype, seqs)
    po, plse = f8.decode_fp8(q, kc, ks, vc, vs, bt, np.maximum(per, 1), scale, hkv, bs, q_dtype, seqs)
    m = np.maximum(lse, plse)
    a, b = np.exp(lse - m), np.exp(plse - m)
    return (a[..., None] * out + b[..., None] * po) / (a + b)[..., None], m + np.log(a + b)


@pytest.mark.parametrize("name,bad", [("prefix rows only", _cascade_prefix_only),
                                      ("group structure unchecked", _cascade_no_check),
                                      ("prefix counted twice", _cascade_prefix_twice)])
def test_planted_cascade_mistake_is_caught(monkeypatch, name, bad):
    monkeypatch.setattr(oracle, "prefix_cascade_fp8", bad)
    assert any(p() for p in CASCADE_PINS), f"no pin noticed: {name}"
