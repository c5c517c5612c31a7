"""Run the fp64 oracle over a whole batch on every host core.

TEST INFRASTRUCTURE ONLY (see the package docstring): the GPU parity tests
and the benchmark's CPU-baseline leg use it to compare or time full-size
batches.

The work is split into units of (sequence, kv-head): attention of one
kv-head's G q-heads (and all of the sequence's query tokens) over that
sequence's rows, which is independent of every other unit (q-head h reads
kv-head h // G only).  Each unit is computed by the oracle's own functions
(``attention.paged_attention``, ``attention.decode_window``,
``attention.decode_multi_window``, ``fp8.decode_multi_fp8``) on a one-kv-head copy of the sequence's pages with
its table relabelled 0..n-1 -- a page relabelling, which the oracle's pins
show leaves the result bit-identical.  Nothing here computes attention
itself.

Worker processes are started with the "spawn" method: fresh interpreters
that import numpy and this package only, never a GPU runtime.  Start them
with :func:`start_pool` before the calling process initialises a GPU; each
worker limits its BLAS to one thread, so N workers use N cores.  Without a
pool the units run in the calling process, one after another.
"""

from __future__ import annotations

import multiprocessing as mp
import os
from collections import deque
from typing import Callable, Iterable, Optional

import numpy as np

_POOL = None
_POOL_N = 0


def host_cores(cap: int = 16) -> int:
    """Cores this process may run on, at most ``cap``."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, cap))


def _init_worker():
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
        os.environ[var] = "1"
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(1)
    except ImportError:  # pragma: no cover
        pass


def start_pool(workers: Optional[int] = None) -> int:
    """Start (once) ``workers`` spawned worker processes (default: the host
    cores, at most 16); returns the pool size."""
    global _POOL, _POOL_N
    if _POOL is None:
        n = host_cores() if workers is None else max(1, int(workers))
        # the children must not inherit a BLAS thread count from the parent
        # environment before _init_worker runs
        _POOL = mp.get_context("spawn").Pool(n, initializer=_init_worker)
        _POOL_N = n
    return _POOL_N


def stop_pool() -> None:
    global _POOL, _POOL_N
    if _POOL is not None:
        _POOL.terminate()
        _POOL.join()
        _POOL, _POOL_N = None, 0


def pool_size() -> int:
    return _POOL_N


def _unit(task):
    """One (sequence, kv-head) unit; returns (key, out [n, G, D], lse [n, G])."""
    from . import attention, fp8

    key, kind = task["key"], task["kind"]
    L, n = int(task["L"]), int(task["q_len"])
    P = task["k"].shape[0]
    bt = np.arange(P, dtype=np.int32)[None, :]
    if kind == "window":
        # entries before the (earliest token's) window's first page are
        # never read; name page 0
        first = task["first_page"]
        bt = np.concatenate([np.zeros(first, np.int32), np.arange(P, dtype=np.int32)])[None, :]
        if n == 1:
            out, lse = attention.decode_window(task["q"], task["k"], task["v"], bt, np.array([L]), task["window"],
                                               task["scale"], 1, 16, task["dtype"])
        else:
            out, lse = attention.decode_multi_window(task["q"], task["k"], task["v"], bt, np.array([L]), n,
                                                     task["window"], task["scale"], 1, 16, task["dtype"])
    elif kind == "fp8":
        out, lse = fp8.decode_multi_fp8(task["q"], task["k"], task["ks"], task["v"], task["vs"], bt, np.array([L]),
                                        n, task["scale"], 1, 16, task["dtype"])
    else:
        out, lse = attention.paged_attention(task["q"], task["k"], task["v"], bt, np.array([L]), np.array([n]),
                                             task["scale"], 1, 16, task["dtype"])
    return key, out, lse


def run_units(tasks: Iterable[dict], inflight: Optional[int] = None):
    """Compute units, yielding (key, out, lse) as they finish (any order).
    At most ``inflight`` tasks (default 2 per worker) are queued at once, so
    the caller's generator produces inputs only as fast as they are used."""
    if _POOL is None:
        for t in tasks:
            yield _unit(t)
        return
    cap = inflight or 2 * _POOL_N
    pending = deque()
    it = iter(tasks)
    exhausted = False
    while True:
        while not exhausted and len(pending) < cap:
            try:
                t = next(it)
            except StopIteration:
                exhausted = True
                break
            pending.append(_POOL.apply_async(_unit, (t,)))
        if not pending:
            return
        yield pending.popleft().get()


def batch_attention(fetch: Callable, seqs, context_lens, q_lens, num_kv_heads: int, scale: float, dtype: str,
                    window: Optional[int] = None, fp8_kv: bool = False, inflight: Optional[int] = None):
    """The oracle over the given sequences of a batch, unit by unit.

    ``fetch(s)`` returns sequence s's stored inputs as numpy arrays:
    ``(q [n, Hq, D], k [P, Hkv, 16, D], v [P, Hkv, 16, D])`` -- plus
    ``(k_scales [P, Hkv, 16], v_scales [P, Hkv, 16])`` when ``fp8_kv`` --
    where the P pages are the ones its table names, in table order (from
    the first page of the earliest token's window on when ``window`` is
    given), and n =
    ``q_lens[s]`` tokens.  Yields (s, out [n, Hq, D], lse [n, Hq]) in
    float64 as sequences complete.
    """
    ctx = np.asarray(context_lens, dtype=np.int64)
    ql = np.asarray(q_lens, dtype=np.int64)
    parts = {}

    def tasks():
        for s in seqs:
            got = fetch(s)
            q, k, v = got[0], got[1], got[2]
            n, Hq, D = q.shape
            G = Hq // num_kv_heads
            L = int(ctx[s])
            for g in range(num_kv_heads):
                t = {"key": (int(s), g), "kind": "attn", "L": L, "q_len": int(ql[s]), "scale": float(scale),
                     "dtype": dtype, "q": np.ascontiguousarray(q[:, g * G:(g + 1) * G]),
                     "k": np.ascontiguousarray(k[:, g:g + 1]), "v": np.ascontiguousarray(v[:, g:g + 1])}
                if window is not None:
                    lo = L - int(ql[s]) + 1 - int(window)  # the earliest row a token sees
                    t.update(kind="window", window=int(window), first_page=lo // 16 if lo > 0 else 0)
                if fp8_kv:
                    t.update(kind="fp8", ks=np.ascontiguousarray(got[3][:, g:g + 1]),
                             vs=np.ascontiguousarray(got[4][:, g:g + 1]))
                yield t

    for (s, g), out, lse in run_units(tasks(), inflight):
        d = parts.setdefault(s, {})
        d[g] = (out, lse)
        if len(d) == num_kv_heads:
            del parts[s]
            yield s, np.concatenate([d[i][0] for i in range(num_kv_heads)], axis=1), \
                np.concatenate([d[i][1] for i in range(num_kv_heads)], axis=1)
