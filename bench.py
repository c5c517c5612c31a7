"""Benchmark: paged decode attention at the Llama-3-8B shape on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one library call over the whole batch (pa_decode for decode
batches, pa_prefix_cascade for shared-prefix groups, pa_mixed_chunk for
prefill chunks + decode tokens, their fp8 forms over fp8 pools), with inputs
resident in HBM.  Each timed step follows a 1 GiB read sweep of a scratch
buffer on the same stream (outside the step's own event pair), so no input
is still in the last-level cache.  Prints ONE JSON line: value =
algorithmic bytes per step / median cold step time (GB/s), with the minimum
and a warm-cache (back-to-back) figure under "timing"; decode tokens/s for
a 32-layer model (attention only); a roofline object for the dominant
kernel timed with HIP events on its own stream (in a second pass of the
same cold steps, so that those events stay out of the timed steps); and the
fp64 CPU oracle timed on a bounded sample of the same workload over the
host cores (oracle.parallel).  Profile runs pass --no-cpu-baseline, so that
no worker process is started under the profiler.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama8b_decode")
    ap.add_argument("--op", choices=["attention", "append"], default="attention",
                    help="attention (the call the workload names) or the KV append of its new tokens")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--split-pages", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget for the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush", choices=["read", "fill", "none"], default="read",
                    help="before each timed step: read a 1 GiB buffer (default), fill it, or nothing")
    ap.add_argument("--via-mixed", action="store_true",
                    help="multi-token batches (every sequence the same q_len > 1) through pa_mixed_chunk "
                         "instead of pa_decode_multi")
    ap.add_argument("--hbm-probe", action="store_true",
                    help="only run the HBM load-path probe (random 4 KB tiles of two pools, LDS DMA against "
                         "loads into registers, a sweep of waves per CU)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES (calibrates HBM traffic counters)")
    return ap.parse_args()


KERNEL_SOURCES = ["paged_kv_decode_02_amd/csrc/pa_decode.hip", "paged_kv_decode_02_amd/csrc/pa_stream.h",
                  "paged_kv_decode_02_amd/csrc/pa_common.h"]
APPEND_SOURCES = ["paged_kv_decode_02_amd/csrc/pa_append.hip", "paged_kv_decode_02_amd/csrc/pa_common.h"]
TILE_SOURCES = ["paged_kv_decode_02_amd/csrc/pa_tiles.hip", "paged_kv_decode_02_amd/csrc/pa_stream.h",
                "paged_kv_decode_02_amd/csrc/pa_common.h"]


def source_digest(sources) -> str:
    import hashlib

    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, sources=KERNEL_SOURCES):
    """HBM bytes per launch of the dominant kernel, from the PMC summary
    committed under profiles/ -- or None when there is none for this
    workload or the kernel source changed since the counters were taken."""
    import glob
    import re

    digest = source_digest(sources)
    for path in glob.glob(os.path.join(ROOT, "profiles", "*.md")):
        for m in re.finditer(r"<!-- traffic: (.*?) -->", open(path).read()):
            kv = dict(x.split("=", 1) for x in m.group(1).split())
            if kv.get("workload") == workload and kv.get("source_sha256") == digest:
                return int(float(kv["fetch_kib"]) * float(kv["fetch_scale"]) * 1024 +
                           float(kv["write_kib"]) * float(kv["write_scale"]) * 1024)
    return None


def copy_probe(nbytes: int) -> None:
    """A plain copy of known size: under rocprofv3 --pmc its FETCH_SIZE and
    WRITE_SIZE give the counters' scale (KiB per byte moved)."""
    import torch

    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "copies": 3}), flush=True)


def hbm_probe() -> None:
    """The decode kernels' access pattern without their math: every tile of
    two pools of 150,000 random 4 KB tiles (614 MB each) read once per launch
    in a random order, 2 or 4 tiles of each pool per batch, the next batch
    in flight while one is consumed, by LDS DMA (mode 0) or by loads into
    registers (mode 1), at 1 to 16 waves per CU; then the same number of
    reads over a few distinct tiles (L2- and MALL-resident).  One JSON line
    per point."""
    import ctypes

    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_decode_02_amd", "libpa_probe.so"))
    lib.hbm_probe_run.restype = ctypes.c_float
    lib.hbm_probe_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    n = 150_000
    torch.manual_seed(0)
    kp = torch.randint(0, 255, (n * 4096,), dtype=torch.uint8, device="cuda")
    vp = torch.randint(0, 255, (n * 4096,), dtype=torch.uint8, device="cuda")
    ids = torch.randperm(n, device="cuda").to(torch.int32)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    st = torch.cuda.current_stream().cuda_stream
    nbytes = 2 * n * 4096
    for mode in (0, 1):
        for tpb in (2, 4):
            for wpc in (1, 2, 3, 4, 5, 6, 8, 12, 16):
                ms = lib.hbm_probe_run(mode, tpb, kp.data_ptr(), vp.data_ptr(), ids.data_ptr(), n, wpc * cus, 5, st)
                if ms <= 0:
                    raise RuntimeError(f"hbm probe failed ({ms})")
                print(json.dumps({"probe": "hbm", "load_path": ["lds_dma", "registers"][mode], "tiles_per_batch": tpb,
                                  "waves_per_cu": wpc, "bytes": nbytes, "ms": round(ms, 5),
                                  "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1)}), flush=True)
    # The same reads over ids that name only `distinct` tiles of each pool:
    # 256 (1 MB per pool) stay in the L2s, 2,048 (8 MB) spill to the MALL,
    # 16,384 (64 MB) live in the MALL.
    for distinct in (256, 2048, 16384):
        ids_d = (torch.randperm(n, device="cuda") % distinct).to(torch.int32)
        for mode in (0, 1):
            ms = lib.hbm_probe_run(mode, 2, kp.data_ptr(), vp.data_ptr(), ids_d.data_ptr(), n, 4 * cus, 5, st)
            if ms <= 0:
                raise RuntimeError(f"hbm probe failed ({ms})")
            print(json.dumps({"probe": "reuse", "distinct_tiles": distinct, "load_path": ["lds_dma", "registers"][mode],
                              "tiles_per_batch": 2, "waves_per_cu": 4, "bytes": nbytes, "ms": round(ms, 5),
                              "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1)}), flush=True)


def visible_pairs(lay, segs):
    """(token, key) pairs the given segments' queries see (per q-head)."""
    tot = 0
    for s in segs:
        L, n = int(lay.context_lens[s]), int(lay.q_lens[s])
        if lay.window is not None:
            tot += sum(min(L - n + i + 1, lay.window) for i in range(n))  # each token over its own window
        else:
            tot += n * (L - n) + n * (n + 1) // 2
    return tot


def cpu_baseline(lay, q, k, v, total_bytes, budget_s, k_scales=None, v_scales=None):
    """Time the fp64 oracle, as it stands, on the host cores: whole sequences
    of the same batch in random order, split into (sequence, kv-head) units
    over the oracle's worker processes (one BLAS thread each), fed until
    about budget_s seconds of wall time have passed; the wall time of that
    sample is scaled to the whole batch by the (token, key) pairs attended,
    and the batch's algorithmic bytes over that time are reported."""
    import torch

    from oracle import parallel

    def host(t):
        if t.dtype == torch.bfloat16:
            return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return t.float().cpu().numpy()

    cu = lay.cu_q_lens
    fp8 = k_scales is not None
    W = lay.window
    order = [int(x) for x in np.random.default_rng(123).permutation(lay.num_seqs)]
    fed = []
    t0 = time.perf_counter()

    def seqs():
        for s in order:
            if time.perf_counter() - t0 > budget_s:
                return
            fed.append(s)
            yield s

    def fetch(s):
        L = int(lay.context_lens[s])
        lo = L - int(lay.q_lens[s]) + 1 - W if W is not None else 0  # the earliest row a token sees
        first = lo // 16 if lo > 0 else 0
        idx = torch.from_numpy(lay.block_tables[s, first:(L + 15) // 16].astype(np.int64)).to(k.device)
        qs = host(q[int(cu[s]) : int(cu[s + 1])])
        if fp8:
            return (qs, k.index_select(0, idx).cpu().numpy(), v.index_select(0, idx).cpu().numpy(),
                    k_scales.index_select(0, idx).cpu().numpy(), v_scales.index_select(0, idx).cpu().numpy())
        return qs, host(k.index_select(0, idx)), host(v.index_select(0, idx))

    done = [s for s, _, _ in parallel.batch_attention(fetch, seqs(), lay.context_lens, lay.q_lens,
                                                          lay.num_kv_heads, lay.scale, lay.dtype, window=W,
                                                          fp8_kv=fp8)]
    spent = time.perf_counter() - t0
    frac = visible_pairs(lay, done) / visible_pairs(lay, range(lay.num_seqs))
    est = spent / frac
    cores = max(1, parallel.pool_size())
    return {
        "value": round(total_bytes / est / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{len(done)} of {lay.num_seqs} sequences ({100 * frac:.1f}% of the batch's (token, key) pairs) "
                  f"in {spent:.1f} s wall on {cores} worker processes (fp64 numpy, one BLAS thread each, units of "
                  f"(sequence, kv-head)), pages copied from the device per sequence; whole-batch time scaled by pairs",
    }


def bench_append(args):
    """pa_kv_append alone: every new token of the workload's batch (q_lens
    rows per segment) written into the pools through the block tables.
    Bytes: each new K and V row read once and written once, plus cu_q_lens,
    context_lens and one table entry per token."""
    import torch

    from paged_kv_decode_02_amd import pa, roofline
    from workloads import fp8_values_torch, new_rows_torch, values_torch, workload

    lay = workload(args.workload, seed=args.seed)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fp8 = lay.kv_dtype == "fp8"
    if fp8:
        _, k, ks, v, vs = fp8_values_torch(lay, dev)
    else:
        _, k, v = values_torch(lay, dev)
    kn, vn = new_rows_torch(lay, dev)
    bt = torch.from_numpy(lay.block_tables).to(dev)
    ctx = torch.from_numpy(lay.context_lens).to(dev)
    cu = torch.from_numpy(lay.cu_q_lens.astype(np.int32)).to(dev)
    stream = torch.cuda.current_stream()
    T = lay.num_tokens

    def step():
        if fp8:
            pa.kv_append_fp8(k, v, ks, vs, kn, vn, bt, cu, lay.cu_q_lens, ctx, lay.context_lens, stream=stream)
        else:
            pa.kv_append(k, v, kn, vn, bt, cu, lay.cu_q_lens, ctx, lay.context_lens, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    pa.profile_enable(args.steps)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kern = float(np.mean(pa.profile_collect(args.steps)))
    pa.profile_enable(0)
    # new K and V rows read once and written once (fp8: codes plus a float32
    # scale per row written)
    rows = 2 * T * lay.num_kv_heads * lay.head_dim * lay.elem_bytes
    rows += 2 * T * lay.num_kv_heads * (lay.head_dim + 4) if fp8 else rows
    nbytes = rows + 4 * (lay.num_seqs + 1) + 4 * lay.num_seqs + 4 * T
    achieved = nbytes / (kern * 1e-3) / 1e9
    print(json.dumps({
        "metric": "paged KV append GB/s (new K/V rows into the pool)", "value": round(nbytes / (ms * 1e-3) / 1e9, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"{lay.dtype} rows -> fp8 e4m3fn cache" if fp8 else lay.dtype, "data": "synthetic",
        "config": {"workload": args.workload, "op": "append", "new_tokens": int(T), "kv_heads": lay.num_kv_heads,
                   "head_dim": lay.head_dim, "block_size": 16, "seed": args.seed},
        "algorithmic_bytes_per_step": int(nbytes),
        "roofline": {"bound": "hbm", "kernel": "kv_append_fp8_kernel" if fp8 else "kv_append_kernel",
                     "achieved": round(achieved, 1),
                     "peak": roofline.HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / roofline.HBM_PEAK_GBS, 4),
                     "kernel_ms": round(kern, 5),
                     "traffic": measured_traffic("append:" + args.workload, APPEND_SOURCES)},
    }), flush=True)


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.hbm_probe:
        hbm_probe()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); this path does not shard across GPUs.",
              file=sys.stderr)
        sys.exit(2)
    if args.op == "append":
        bench_append(args)
        return
    if not args.no_cpu_baseline:
        # the oracle's worker processes start before this process touches
        # the GPU (they are fresh interpreters that never do)
        from oracle import parallel

        parallel.start_pool()
    import torch

    from paged_kv_decode_02_amd import pa, roofline
    from workloads import fp8_values_torch, values_torch, workload

    lay = workload(args.workload, seed=args.seed)
    cascade = lay.group_seq_offsets is not None
    mixed = lay.q_lens.max() > 1
    # every sequence the same number of new tokens (> 1): a multi-token
    # decode step, through pa_decode_multi unless asked otherwise
    multi = bool(mixed and (lay.q_lens == lay.q_lens[0]).all() and not args.via_mixed)
    if multi:
        mixed = False
        n_tok = int(lay.q_lens[0])
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] workload {args.workload} seed {args.seed}: drawing inputs on the device", file=sys.stderr,
          flush=True)
    fp8 = lay.kv_dtype == "fp8"
    if fp8:
        q, k, ks, v, vs = fp8_values_torch(lay, dev)
    else:
        q, k, v = values_torch(lay, dev)
    bt = torch.from_numpy(lay.block_tables).to(dev)
    ctx = torch.from_numpy(lay.context_lens).to(dev)
    out = torch.empty_like(q)
    T, Hq, D = q.shape
    S = lay.num_seqs
    total_pages = int(((lay.context_lens + 15) // 16).sum())
    stream = torch.cuda.current_stream()
    if cascade:
        go = torch.from_numpy(lay.group_seq_offsets).to(dev)
        pl = torch.from_numpy(lay.prefix_lens).to(dev)
        ws = torch.empty(pa.prefix_cascade_workspace_size(S, lay.num_kv_heads, lay.gqa_ratio, D, total_pages),
                         dtype=torch.uint8, device=dev)

        if fp8:
            def step():
                pa.prefix_cascade_fp8(out, q, k, v, ks, vs, bt, ctx, lay.context_lens, go, lay.group_seq_offsets, pl,
                                      lay.prefix_lens, lay.scale, ws, stream=stream)
        else:
            def step():
                pa.prefix_cascade(out, q, k, v, bt, ctx, lay.context_lens, go, lay.group_seq_offsets, pl,
                                  lay.prefix_lens, lay.scale, ws, stream=stream)
    elif mixed or multi:
        cu = torch.from_numpy(lay.cu_q_lens.astype(np.int32)).to(dev)
        mws = torch.empty(pa.mixed_chunk_workspace_size(T, S, lay.num_kv_heads, lay.gqa_ratio, D, total_pages),
                          dtype=torch.uint8, device=dev)

        def mixed_step():
            if fp8:
                pa.mixed_chunk_fp8(out, q, k, v, ks, vs, bt, cu, lay.cu_q_lens, ctx, lay.context_lens, lay.scale, mws,
                                   stream=stream)
            else:
                pa.mixed_chunk(out, q, k, v, bt, cu, lay.cu_q_lens, ctx, lay.context_lens, lay.scale, mws,
                               stream=stream)

        step = mixed_step
        if multi:
            ws = torch.empty(pa.decode_multi_workspace_size(S, n_tok, lay.num_kv_heads, lay.gqa_ratio, D, total_pages,
                                                            args.split_pages), dtype=torch.uint8, device=dev)

            def step():
                if fp8:
                    pa.decode_multi_fp8(out, q, k, v, ks, vs, bt, ctx, lay.context_lens, lay.scale, n_tok, ws,
                                        split_pages=args.split_pages, stream=stream)
                elif lay.window is not None:
                    pa.decode_multi_window(out, q, k, v, bt, ctx, lay.context_lens, lay.scale, n_tok, lay.window,
                                           ws, split_pages=args.split_pages, stream=stream)
                else:
                    pa.decode_multi(out, q, k, v, bt, ctx, lay.context_lens, lay.scale, n_tok, ws,
                                    split_pages=args.split_pages, stream=stream)
    else:
        ws = torch.empty(pa.decode_workspace_size(S, lay.num_kv_heads, lay.gqa_ratio, D, total_pages,
                                                  args.split_pages), dtype=torch.uint8, device=dev)

        def step():
            if fp8:
                pa.decode_fp8(out, q, k, v, ks, vs, bt, ctx, lay.context_lens, lay.scale, ws,
                              split_pages=args.split_pages, stream=stream)
            elif lay.window is not None:
                pa.decode_window(out, q, k, v, bt, ctx, lay.context_lens, lay.scale, lay.window, ws,
                                 split_pages=args.split_pages, stream=stream)
            else:
                pa.decode(out, q, k, v, bt, ctx, lay.context_lens, lay.scale, ws, split_pages=args.split_pages,
                          stream=stream)

    def timed(fn, n):
        """Warm-cache mean: n steps back to back between two events."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # Cold cache: before each timed step 1 GiB passes through the caches on
    # the same stream, outside the step's event pair, which evicts the step's
    # inputs from the 256 MB last-level cache (MALL) and the L2s.  The
    # default sweep reads the buffer (a sum): a fill would leave up to 256 MB
    # of dirty lines whose write-back to HBM then lands inside the timed
    # step (measured: 186 against 116 us on the Llama-shaped batch).
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    flush_out = torch.empty((), dtype=torch.float32, device=dev)

    def flush():
        if args.flush == "read":
            torch.sum(flush_buf, dim=0, out=flush_out)
        elif args.flush == "fill":
            flush_buf.zero_()

    def cold(fn, n, pairs=0):
        """Per-step times (ms) of n steps, each after a cache flush and
        timed by its own event pair; with pairs > 0 the library's events
        around its dominant kernel(s) are collected as well."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        if pairs:
            pa.profile_enable(n * pairs)
        torch.cuda.synchronize()
        for a, b in ev:
            flush()
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        kern = None
        if pairs:
            # (as many pairs per step as the library recorded: a mixed batch
            # with chunks and decode tokens in one launch records one)
            kern = np.array(pa.profile_collect(n * pairs)).reshape(n, -1)
            pa.profile_enable(0)
        return np.array([a.elapsed_time(b) for a, b in ev]), kern

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps", file=sys.stderr, flush=True)

    # Dominant kernel(s) of a step: HIP events the library records around
    # them on the same stream (decode: the stream kernel; cascade: the prefix
    # kernel; mixed: the chunk kernel, then the decode stream kernel).
    has_dec = bool((lay.q_lens == 1).any())
    pairs = 2 if mixed and has_dec else 1
    if multi:
        # folded passes: one stream kernel each
        fold = max(1, min(n_tok, 16 // lay.gqa_ratio))
        pairs = -(-n_tok // fold)
    # The timed steps run without the library's event pairs (each pair adds
    # its own event records to the step: about 8 us on the Llama-shaped
    # decode); the dominant kernels are timed in a second pass of the same
    # cold steps.
    t0 = time.perf_counter()
    step_ms, _ = cold(step, args.steps)
    wall = time.perf_counter() - t0
    ms_per_step = float(np.median(step_ms))
    ms_min = float(step_ms.min())
    _, kern_ms = cold(step, args.steps, pairs)
    kern_avg = [float(x) for x in kern_ms.mean(axis=0)]
    warm_ms = timed(step, args.steps)

    def hbm_roof(kernel, nbytes, ms, traffic):
        achieved = nbytes / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1), "peak": roofline.HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / roofline.HBM_PEAK_GBS, 4), "kernel_ms": round(ms, 5),
                "traffic": traffic}

    def mfma_roof(kernel, flops, ms, traffic=None):
        tflops = flops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "kernel": kernel, "achieved": round(tflops, 1),
                "peak": roofline.MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / roofline.MFMA_BF16_PEAK_TFLOPS, 4), "kernel_ms": round(ms, 5),
                "traffic": traffic}

    def stream_kernel(rows):
        # waves of 4 or more bf16 query rows (bf16 or fp8 pools) run on the
        # matrix-core kernel
        return "stream_mfma_kernel" if lay.dtype == "bf16" and rows >= 4 else "stream_decode_kernel"

    extra = {}
    if cascade:
        nb = roofline.cascade_bytes(lay.context_lens, lay.group_seq_offsets, lay.prefix_lens, lay.num_q_heads,
                                    lay.num_kv_heads, D, 2 if fp8 else lay.elem_bytes, kv_fp8=fp8)
        flops = roofline.prefix_flops(lay.group_seq_offsets, lay.prefix_lens, lay.num_q_heads, D)
        roof = mfma_roof("tile_kernel (shared prefix, fp8 pools)" if fp8 else "tile_kernel (shared prefix)", flops,
                         kern_avg[0], measured_traffic("tile:" + args.workload, TILE_SOURCES))
        # the same batch through plain decode, for the cascade's speed-up
        dws = torch.empty(pa.decode_workspace_size(S, lay.num_kv_heads, lay.gqa_ratio, D, total_pages, 0),
                          dtype=torch.uint8, device=dev)
        dout = torch.empty_like(q)
        if fp8:
            def dec_step():
                pa.decode_fp8(dout, q, k, v, ks, vs, bt, ctx, lay.context_lens, lay.scale, dws, stream=stream)
        else:
            def dec_step():
                pa.decode(dout, q, k, v, bt, ctx, lay.context_lens, lay.scale, dws, stream=stream)
        dec_ms = float(np.median(cold(dec_step, args.steps)[0]))
        extra = {"prefix_gflop": round(flops / 1e9, 3), "decode_same_batch_ms": round(dec_ms, 5),
                 "cascade_speedup_vs_decode": round(dec_ms / ms_per_step, 3)}
    elif multi:
        if fp8:
            nb = roofline.decode_fp8_bytes(lay.context_lens, lay.num_q_heads, lay.num_kv_heads, D, q_len=n_tok)
        elif lay.window is not None:
            # the rows any of a sequence's tokens sees: its last window + n - 1
            nb = roofline.mixed_bytes(np.minimum(lay.context_lens, lay.window + n_tok - 1), lay.q_lens,
                                      lay.num_q_heads, lay.num_kv_heads, D, lay.elem_bytes)
        else:
            nb = roofline.mixed_bytes(lay.context_lens, lay.q_lens, lay.num_q_heads, lay.num_kv_heads, D,
                                      lay.elem_bytes)
        rows = 2
        while rows < lay.gqa_ratio * fold:
            rows *= 2
        label = f"{stream_kernel(rows)} ({n_tok} tokens folded" + (
            f", {lay.window}-token window)" if lay.window is not None else ")")
        roof = hbm_roof(label, nb["total"], float(sum(kern_avg)), measured_traffic(args.workload))
        extra = {"tokens_per_step": int(T), "fold_passes": pairs}
        if lay.window is None:  # (the chunk path takes no window)
            extra["mixed_chunk_same_batch_ms"] = round(float(np.median(cold(mixed_step, args.steps)[0])), 5)
    elif mixed:
        nb = roofline.mixed_bytes(lay.context_lens, lay.q_lens, lay.num_q_heads, lay.num_kv_heads, D,
                                  2 if fp8 else lay.elem_bytes, kv_fp8=fp8)
        flops = roofline.chunk_flops(lay.context_lens, lay.q_lens, lay.num_q_heads, D)
        pools = " (fp8 pools)" if fp8 else ""
        chunk_roof = mfma_roof("tile_kernel (prefill chunks)" + pools, flops, kern_avg[0])
        extra = {"chunk_gflop": round(flops / 1e9, 3), "tokens_per_step": int(T)}
        roof = chunk_roof
        if has_dec and len(kern_avg) == 1:
            # chunks and decode tokens in one launch (mixed_kernel): its HBM
            # view (all K/V bytes of the step) and its matrix view (the chunk
            # flops) over the same kernel time
            traffic = measured_traffic("mixed:" + args.workload, TILE_SOURCES)
            roof = hbm_roof("mixed_kernel (prefill chunks + decode tokens, one launch)" + pools, nb["total"],
                            kern_avg[0], traffic)
            extra["mixed_kernel_mfma"] = mfma_roof("mixed_kernel (chunk flops)" + pools, flops, kern_avg[0], traffic)
        elif has_dec:
            dec = lay.q_lens == 1
            if fp8:
                dbytes = roofline.decode_fp8_bytes(lay.context_lens[dec], lay.num_q_heads, lay.num_kv_heads,
                                                   D)["total"]
            else:
                dbytes = roofline.decode_bytes(lay.context_lens[dec], lay.num_q_heads, lay.num_kv_heads, D,
                                               lay.elem_bytes)["total"]
            dec_roof = hbm_roof(f"{stream_kernel(lay.gqa_ratio)} (decode tokens)" + pools, dbytes, kern_avg[1], None)
            # the dominant kernel is the one that takes longer
            roof, other = (chunk_roof, dec_roof) if kern_avg[0] >= kern_avg[1] else (dec_roof, chunk_roof)
            extra["other_kernel_roofline"] = other
        else:
            # no single-token segments: the chunk kernel is the whole step;
            # its K/V traffic, for the HBM view of the same launch
            extra["chunk_kernel_hbm"] = hbm_roof("tile_kernel (prefill chunks)" + pools, nb["total"], kern_avg[0],
                                                 None)
    elif lay.window is not None:
        # the rows each query sees: the last min(L, window) of its sequence
        nb = roofline.decode_bytes(np.minimum(lay.context_lens, lay.window), lay.num_q_heads, lay.num_kv_heads, D,
                                   lay.elem_bytes)
        roof = hbm_roof(f"{stream_kernel(lay.gqa_ratio)} (sliding window)", nb["total"], kern_avg[0],
                        measured_traffic(args.workload))
    elif fp8:
        nb = roofline.decode_fp8_bytes(lay.context_lens, lay.num_q_heads, lay.num_kv_heads, D)
        roof = hbm_roof(f"{stream_kernel(lay.gqa_ratio)} (fp8 pools)", nb["total"], kern_avg[0],
                        measured_traffic(args.workload))
    else:
        nb = roofline.decode_bytes(lay.context_lens, lay.num_q_heads, lay.num_kv_heads, D, lay.elem_bytes)
        roof = hbm_roof(stream_kernel(lay.gqa_ratio), nb["total"], kern_avg[0], measured_traffic(args.workload))
    gbs = nb["total"] / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": "paged decode attn KV GB/s (% of HBM peak) + decode tokens/s, Llama-8B shape",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 q/out, fp8 e4m3fn K/V" if fp8 else lay.dtype,
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "num_seqs": int(S),
            "num_tokens": int(T),
            "q_heads": lay.num_q_heads,
            "kv_heads": lay.num_kv_heads,
            "head_dim": int(D),
            "block_size": 16,
            "kv_tokens": int(np.minimum(lay.context_lens, lay.window).sum() if lay.window else lay.context_lens.sum()),
            **({"window": int(lay.window)} if lay.window else {}),
            "seed": args.seed,
            "parallelism": "single GPU",
        },
        "hbm_frac": round(gbs / roofline.HBM_PEAK_GBS, 4),
        "timing": {"cache": {"read": "cold: a 1 GiB read sweep before each step, outside its event pair",
                             "fill": "cold: a 1 GiB fill before each step, outside its event pair",
                             "none": "warm: no flush between steps"}[args.flush],
                   "median_ms": round(ms_per_step, 5), "min_ms": round(ms_min, 5),
                   "mean_ms": round(float(step_ms.mean()), 5),
                   "min_step_GBps": round(nb["total"] / (ms_min * 1e-3) / 1e9, 1),
                   "warm_cache_mean_ms": round(warm_ms, 5),
                   "warm_cache_GBps": round(nb["total"] / (warm_ms * 1e-3) / 1e9, 1)},
        # (a multi-token decode step decodes every one of its tokens)
        "decode_tokens_per_s_32_layers": round(int(T if multi else (lay.q_lens == 1).sum()) /
                                               (roofline.LLAMA8B_LAYERS * ms_per_step * 1e-3), 1),
        "algorithmic_bytes_per_step": nb["total"],
        "wall_s": round(wall, 3),
        "roofline": roof,
    }
    result.update(extra)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(lay, q, k, v, nb["total"], args.cpu_seconds,
                                              ks if fp8 else None, vs if fp8 else None)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
