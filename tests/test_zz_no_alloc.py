"""pa_decode_noalloc (fixed per-GPU scratch, no workspace) against pa_decode
(caller workspace) through the C ABI: two calls in a row, the second on a
smaller batch, each bit-identical to pa_decode's output and lse (same
kernels, same plan), and within the oracle's tolerance; a batch whose plan
needs more than the scratch maximum is rejected before anything runs."""

import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_util import LSE_TOL, assert_close, device_inputs, out_to_f64, tables_to_device
from workloads import decode_layout, workload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_both(pa, lay, q, k, v, split_pages=0):
    bt, ctx = tables_to_device(lay)
    S, Hq, D = q.shape
    total = int(((lay.context_lens + 15) // 16).sum())
    ws = torch.empty(pa.decode_workspace_size(S, lay.num_kv_heads, lay.gqa_ratio, D, total, split_pages),
                     dtype=torch.uint8, device="cuda")
    out_a = torch.empty_like(q)
    lse_a = torch.empty((S, Hq), dtype=torch.float32, device="cuda")
    pa.decode(out_a, q, k, v, bt, ctx, lay.context_lens, lay.scale, ws, lse_out=lse_a, split_pages=split_pages)
    out_b = torch.full_like(q, float("nan"))
    lse_b = torch.full((S, Hq), float("nan"), dtype=torch.float32, device="cuda")
    pa.decode_noalloc(out_b, q, k, v, bt, ctx, lay.context_lens, lay.scale, lse_out=lse_b, split_pages=split_pages)
    torch.cuda.synchronize()
    return out_a, lse_a, out_b, lse_b


def check(lay, out_a, lse_a, out_b, lse_b, what):
    view = torch.int16 if out_a.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(out_a.view(view), out_b.view(view)), f"{what}: output differs from pa_decode"
    assert torch.equal(lse_a, lse_b), f"{what}: lse differs from pa_decode"


@pytest.mark.parametrize("second", ["bf16-g4", "bf16-g2", "f32-g4"])
def test_two_calls_in_a_row_match_pa_decode(gpu_lib, second):
    # first call: the Llama-shaped batch (shared sequences, partials in the scratch)
    lay = workload("llama8b_decode", seed=1)
    say(f"case no-alloc llama8b_decode seed 1, then {second}")
    (q, k, v), (qh, kh, vh) = device_inputs(lay)
    out_a, lse_a, out_b, lse_b = run_both(gpu_lib, lay, q, k, v)
    check(lay, out_a, lse_a, out_b, lse_b, "llama8b_decode")
    ro, rl = oracle.decode(qh, kh, vh, lay.block_tables, lay.context_lens, lay.scale, lay.num_kv_heads, 16, "bf16")
    assert_close(lay, out_to_f64(out_b), ro, "no-alloc llama8b_decode")
    assert np.abs(lse_b.cpu().numpy() - rl).max() < LSE_TOL
    # second call: a smaller batch over the scratch the first call left
    dtype, g = second.split("-")
    hkv = 2
    hq = hkv * int(g[1:])
    lay2 = decode_layout([1, 17, 300, 64, 1000, 33, 2], num_q_heads=hq, num_kv_heads=hkv,
                         head_dim=64 if dtype == "f32" else 128, dtype=dtype, pool_factor=1.2, seed=3,
                         value_std=1.0 if dtype == "f32" else 0.5)
    (q2, k2, v2), (qh2, kh2, vh2) = device_inputs(lay2)
    for sp in (0, 2):
        out_a, lse_a, out_b, lse_b = run_both(gpu_lib, lay2, q2, k2, v2, split_pages=sp)
        check(lay2, out_a, lse_a, out_b, lse_b, f"{second} split {sp}")
        ro, rl = oracle.decode(qh2, kh2, vh2, lay2.block_tables, lay2.context_lens, lay2.scale, hkv, 16, dtype)
        assert_close(lay2, out_to_f64(out_b), ro, f"no-alloc {second} split {sp}")
        assert np.abs(lse_b.cpu().numpy() - rl).max() < (1e-4 if dtype == "f32" else LSE_TOL)


def test_plan_beyond_the_scratch_is_rejected(gpu_lib):
    lay = workload("llama8b_decode", seed=2)
    (q, k, v), _ = device_inputs(lay)
    bt, ctx = tables_to_device(lay)
    out = torch.full_like(q, 7.0)
    # one page per wave: thousands of waves, far more partials than 32 MiB hold
    with pytest.raises(gpu_lib.PAError) as e:
        gpu_lib.decode_noalloc(out, q, k, v, bt, ctx, lay.context_lens, lay.scale, split_pages=1)
    assert e.value.code == gpu_lib.PA_EWORKSPACE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
