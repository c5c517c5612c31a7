"""ctypes binding for libpa.so (the HIP paged-attention library).

Argument marshalling only: this module checks that tensor shapes agree with
each other (so the sizes handed to the C ABI describe the buffers passed),
converts tensors to raw pointers and forwards to the library.  Every step of
the computation runs in the library's kernels; there is no fallback path.
If the built library is missing, :func:`load` raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# PA_LIB names another build of the same C ABI (the host-only sanitizer
# build in the CPU tests); by default the in-tree libpa.so.
LIB_PATH = os.environ.get("PA_LIB") or os.path.join(HERE, "libpa.so")

PA_F32 = 0
PA_BF16 = 1
PA_OK = 0
PA_EINVAL = -1
PA_EUNSUPPORTED = -2
PA_EWORKSPACE = -3
PA_EHIP = -4

# every symbol include/pa.h declares
EXPORTS = (
    "pa_decode_workspace_size",
    "pa_decode",
    "pa_decode_noalloc",
    "pa_decode_fp8",
    "pa_decode_window",
    "pa_decode_multi_workspace_size",
    "pa_decode_multi",
    "pa_decode_multi_window",
    "pa_decode_multi_fp8",
    "pa_prefix_cascade_workspace_size",
    "pa_prefix_cascade",
    "pa_prefix_cascade_fp8",
    "pa_mixed_chunk_workspace_size",
    "pa_mixed_chunk",
    "pa_mixed_chunk_fp8",
    "pa_kv_append",
    "pa_kv_append_fp8",
    "pa_check_block_tables",
    "pa_detect_prefix_groups",
    "pa_last_error",
    "pa_profile_enable",
    "pa_profile_collect",
)

_lib = None

c_i32 = ctypes.c_int32
c_i64 = ctypes.c_int64
c_vp = ctypes.c_void_p
c_sz = ctypes.c_size_t


class PAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libpa error {code}: {msg}")
        self.code = code


def load(path: Optional[str] = None):
    """Load libpa.so (built in-tree by ``paged_kv_decode_02_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m paged_kv_decode_02_amd.build`")
    lib = ctypes.CDLL(p)
    lib.pa_decode_workspace_size.restype = c_sz
    lib.pa_decode_workspace_size.argtypes = [c_i32, c_i32, c_i32, c_i32, c_i64, c_i32]
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                              c_i32, c_i64, ctypes.c_float, ctypes.c_int, c_i32, c_vp, c_sz, c_vp]
    lib.pa_decode_window.restype = ctypes.c_int
    lib.pa_decode_noalloc.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32,
                                      c_i32, c_i32, c_i64, ctypes.c_float, c_i32, c_i32, c_vp]
    lib.pa_decode_noalloc.restype = c_i32
    lib.pa_decode_window.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32,
                                     c_i32, c_i32, c_i64, ctypes.c_float, ctypes.c_int, c_i32, c_i32, c_vp, c_sz,
                                     c_vp]
    lib.pa_decode_multi_workspace_size.restype = c_sz
    lib.pa_decode_multi_workspace_size.argtypes = [c_i32, c_i32, c_i32, c_i32, c_i32, c_i64, c_i32]
    lib.pa_decode_multi.restype = ctypes.c_int
    lib.pa_decode_multi.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32,
                                    c_i32, c_i32, c_i64, ctypes.c_float, ctypes.c_int, c_i32, c_vp, c_sz, c_vp]
    lib.pa_decode_multi_window.restype = ctypes.c_int
    lib.pa_decode_multi_window.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32, c_i32,
                                           c_i32, c_i32, c_i32, c_i32, c_i32, c_i64, ctypes.c_float, ctypes.c_int,
                                           c_i32, c_vp, c_sz, c_vp]
    lib.pa_decode_multi_fp8.restype = ctypes.c_int
    lib.pa_decode_multi_fp8.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32,
                                        c_i32, c_i32, c_i32, c_i32, c_i32, c_i64, ctypes.c_float, c_i32, c_vp, c_sz,
                                        c_vp]
    lib.pa_decode_fp8.restype = ctypes.c_int
    lib.pa_decode_fp8.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32, c_i32,
                                  c_i32, c_i32, c_i32, c_i64, ctypes.c_float, c_i32, c_vp, c_sz, c_vp]
    lib.pa_prefix_cascade_workspace_size.restype = c_sz
    lib.pa_prefix_cascade_workspace_size.argtypes = [c_i32, c_i32, c_i32, c_i32, c_i64]
    lib.pa_prefix_cascade.restype = ctypes.c_int
    lib.pa_prefix_cascade.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_vp, c_vp,
                                      c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i64, ctypes.c_float, ctypes.c_int,
                                      c_vp, c_sz, c_vp]
    lib.pa_prefix_cascade_fp8.restype = ctypes.c_int
    lib.pa_prefix_cascade_fp8.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32,
                                          c_i32, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_i64,
                                          ctypes.c_float, c_vp, c_sz, c_vp]
    lib.pa_mixed_chunk_workspace_size.restype = c_sz
    lib.pa_mixed_chunk_workspace_size.argtypes = [c_i32, c_i32, c_i32, c_i32, c_i32, c_i64]
    lib.pa_mixed_chunk.restype = ctypes.c_int
    lib.pa_mixed_chunk.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32,
                                   c_i32, c_i32, c_i32, c_i64, ctypes.c_float, ctypes.c_int, c_vp, c_sz, c_vp]
    lib.pa_mixed_chunk_fp8.restype = ctypes.c_int
    lib.pa_mixed_chunk_fp8.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp,
                                       c_i32, c_i32, c_i32, c_i32, c_i32, c_i64, ctypes.c_float, c_vp, c_sz, c_vp]
    lib.pa_kv_append.restype = ctypes.c_int
    lib.pa_kv_append.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32,
                                 c_i32, c_i64, ctypes.c_int, c_vp]
    lib.pa_detect_prefix_groups.restype = ctypes.c_int
    lib.pa_detect_prefix_groups.argtypes = [c_vp, c_i32, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp]
    lib.pa_kv_append_fp8.restype = ctypes.c_int
    lib.pa_kv_append_fp8.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp, c_i32,
                                     c_i32, c_i32, c_i32, c_i64, ctypes.c_int, c_vp]
    lib.pa_check_block_tables.restype = ctypes.c_int
    lib.pa_check_block_tables.argtypes = [c_vp, c_i32, c_vp, c_i32, c_i32, c_i64, c_i32, c_vp, c_vp]
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_last_error.argtypes = []
    lib.pa_profile_enable.restype = ctypes.c_int
    lib.pa_profile_enable.argtypes = [c_i32]
    lib.pa_profile_collect.restype = ctypes.c_int
    lib.pa_profile_collect.argtypes = [ctypes.POINTER(ctypes.c_float), c_i32]
    if path is None:
        _lib = lib
    return lib


def last_error() -> str:
    return load().pa_last_error().decode()


def _check(rc: int) -> int:
    if rc < 0:
        raise PAError(rc, last_error())
    return rc


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _host_i32(a, name):
    arr = np.ascontiguousarray(a.numpy() if hasattr(a, "numpy") else a, dtype=np.int32)
    return arr


def _stream_ptr(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def decode_workspace_size(max_num_seqs, num_kv_heads, gqa_ratio, head_dim, max_total_pages, split_pages=0) -> int:
    return int(load().pa_decode_workspace_size(max_num_seqs, num_kv_heads, gqa_ratio, head_dim, max_total_pages,
                                               split_pages))


def decode_window(out, q, k_pool, v_pool, block_tables, context_lens, context_lens_host, scale, window, workspace,
                  lse_out=None, split_pages=0, stream=None):
    """pa_decode_window on torch tensors: as :func:`decode`, each query
    seeing only the last ``window`` rows of its sequence."""
    import torch

    S, Hq, D = q.shape
    NP, Hkv, BS, D2 = k_pool.shape
    if tuple(out.shape) != (S, Hq, D) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if tuple(v_pool.shape) != tuple(k_pool.shape) or k_pool.dtype != q.dtype or v_pool.dtype != q.dtype:
        raise ValueError("k_pool and v_pool must match each other and q's dtype")
    if D2 != D or Hq % Hkv:
        raise ValueError("head_dim mismatch or q heads not a multiple of kv heads")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    ch = _host_i32(context_lens_host, "context_lens_host")
    if ch.size != S:
        raise ValueError("context_lens_host must have one entry per sequence")
    if lse_out is not None and tuple(lse_out.shape) != (S, Hq):
        raise ValueError("lse_out must be [S, Hq]")
    rc = load().pa_decode_window(
        _dev(out, "out"),
        _dev(lse_out, "lse_out", torch.float32) if lse_out is not None else None,
        _dev(q, "q"),
        _dev(k_pool, "k_pool"),
        _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32),
        ch.ctypes.data,
        S, Hkv, Hq // Hkv, D, BS, NP, float(scale), _dtype_code(q), int(window), int(split_pages),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream_ptr(stream),
    )
    return _check(rc)


def decode_multi_workspace_size(max_num_seqs, q_len, num_kv_heads, gqa_ratio, head_dim, max_total_pages,
                                split_pages=0) -> int:
    return int(load().pa_decode_multi_workspace_size(max_num_seqs, q_len, num_kv_heads, gqa_ratio, head_dim,
                                                     max_total_pages, split_pages))


def decode_multi(out, q, k_pool, v_pool, block_tables, context_lens, context_lens_host, scale, q_len, workspace,
                 lse_out=None, split_pages=0, stream=None):
    """pa_decode_multi on torch tensors: ``q_len`` new tokens per sequence,
    q / out ``[S * q_len, Hq, D]`` (token i of sequence s at row
    s * q_len + i), causal among the new tokens."""
    return _decode_multi(None, out, q, k_pool, v_pool, block_tables, context_lens, context_lens_host, scale, q_len,
                         workspace, lse_out, split_pages, stream)


def decode_multi_window(out, q, k_pool, v_pool, block_tables, context_lens, context_lens_host, scale, q_len, window,
                        workspace, lse_out=None, split_pages=0, stream=None):
    """pa_decode_multi_window on torch tensors: pa_decode_multi's tokens,
    each seeing only the ``window`` rows up to its own position."""
    return _decode_multi(int(window), out, q, k_pool, v_pool, block_tables, context_lens, context_lens_host, scale,
                         q_len, workspace, lse_out, split_pages, stream)


def _decode_multi(window, out, q, k_pool, v_pool, block_tables, context_lens, context_lens_host, scale, q_len,
                  workspace, lse_out, split_pages, stream):
    import torch

    T, Hq, D = q.shape
    NP, Hkv, BS, D2 = k_pool.shape
    q_len = int(q_len)
    if q_len < 1 or T % q_len:
        raise ValueError("q rows must be num_seqs * q_len")
    S = T // q_len
    if tuple(out.shape) != (T, Hq, D) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if tuple(v_pool.shape) != tuple(k_pool.shape) or k_pool.dtype != q.dtype or v_pool.dtype != q.dtype:
        raise ValueError("k_pool and v_pool must match each other and q's dtype")
    if D2 != D or Hq % Hkv:
        raise ValueError("head_dim mismatch or q heads not a multiple of kv heads")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    ch = _host_i32(context_lens_host, "context_lens_host")
    if ch.size != S:
        raise ValueError("context_lens_host must have one entry per sequence")
    if lse_out is not None and tuple(lse_out.shape) != (T, Hq):
        raise ValueError("lse_out must be [S * q_len, Hq]")
    head = (
        _dev(out, "out"),
        _dev(lse_out, "lse_out", torch.float32) if lse_out is not None else None,
        _dev(q, "q"),
        _dev(k_pool, "k_pool"),
        _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32),
        ch.ctypes.data,
        S, q_len,
    )
    tail = (Hkv, Hq // Hkv, D, BS, NP, float(scale), _dtype_code(q), int(split_pages),
            _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream_ptr(stream))
    if window is None:
        rc = load().pa_decode_multi(*head, *tail)
    else:
        rc = load().pa_decode_multi_window(*head, int(window), *tail)
    return _check(rc)


def decode_fp8(out, q, k_pool, v_pool, k_scales, v_scales, block_tables, context_lens, context_lens_host, scale,
               workspace, lse_out=None, split_pages=0, stream=None):
    """pa_decode_fp8 on torch tensors.

    q, out: [S, Hq, D] bfloat16; k_pool, v_pool: [NP, Hkv, 16, D] uint8
    e4m3fn codes (or torch.float8_e4m3fn); k_scales, v_scales: [NP, Hkv, 16]
    float32; the rest as :func:`decode`.
    """
    import torch

    S, Hq, D = q.shape
    NP, Hkv, BS, D2 = k_pool.shape
    if q.dtype != torch.bfloat16 or tuple(out.shape) != (S, Hq, D) or out.dtype != torch.bfloat16:
        raise ValueError("q and out must be bfloat16 [S, Hq, D]")
    codes = (torch.uint8, torch.float8_e4m3fn)
    if tuple(v_pool.shape) != tuple(k_pool.shape) or k_pool.dtype not in codes or v_pool.dtype not in codes:
        raise ValueError("k_pool and v_pool must be [NP, Hkv, BS, D] uint8 / float8_e4m3fn")
    for t, nm in ((k_scales, "k_scales"), (v_scales, "v_scales")):
        if tuple(t.shape) != (NP, Hkv, BS) or t.dtype != torch.float32:
            raise ValueError(f"{nm} must be float32 [NP, Hkv, BS]")
    if D2 != D or Hq % Hkv:
        raise ValueError("head_dim mismatch or q heads not a multiple of kv heads")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    ch = _host_i32(context_lens_host, "context_lens_host")
    if ch.size != S:
        raise ValueError("context_lens_host must have one entry per sequence")
    if lse_out is not None and tuple(lse_out.shape) != (S, Hq):
        raise ValueError("lse_out must be [S, Hq]")
    rc = load().pa_decode_fp8(
        _dev(out, "out"),
        _dev(lse_out, "lse_out", torch.float32) if lse_out is not None else None,
        _dev(q, "q"),
        _dev(k_pool, "k_pool"),
        _dev(v_pool, "v_pool"),
        _dev(k_scales, "k_scales", torch.float32),
        _dev(v_scales, "v_scales", torch.float32),
        _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32),
        ch.ctypes.data,
        S, Hkv, Hq // Hkv, D, BS, NP, float(scale), int(split_pages),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream_ptr(stream),
    )
    return _check(rc)


def decode_multi_fp8(out, q, k_pool, v_pool, k_scales, v_scales, block_tables, context_lens, context_lens_host,
                     scale, q_len, workspace, lse_out=None, split_pages=0, stream=None):
    """pa_decode_multi_fp8 on torch tensors: :func:`decode_multi`'s tokens
    (q / out ``[S * q_len, Hq, D]`` bfloat16) over :func:`decode_fp8`'s
    pools and scales."""
    import torch

    T, Hq, D = q.shape
    NP, Hkv, BS, D2 = k_pool.shape
    q_len = int(q_len)
    if q_len < 1 or T % q_len:
        raise ValueError("q rows must be num_seqs * q_len")
    S = T // q_len
    if q.dtype != torch.bfloat16 or tuple(out.shape) != (T, Hq, D) or out.dtype != torch.bfloat16:
        raise ValueError("q and out must be bfloat16 [S * q_len, Hq, D]")
    codes = (torch.uint8, torch.float8_e4m3fn)
    if tuple(v_pool.shape) != tuple(k_pool.shape) or k_pool.dtype not in codes or v_pool.dtype not in codes:
        raise ValueError("k_pool and v_pool must be [NP, Hkv, BS, D] uint8 / float8_e4m3fn")
    for t, nm in ((k_scales, "k_scales"), (v_scales, "v_scales")):
        if tuple(t.shape) != (NP, Hkv, BS) or t.dtype != torch.float32:
            raise ValueError(f"{nm} must be float32 [NP, Hkv, BS]")
    if D2 != D or Hq % Hkv:
        raise ValueError("head_dim mismatch or q heads not a multiple of kv heads")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    ch = _host_i32(context_lens_host, "context_lens_host")
    if ch.size != S:
        raise ValueError("context_lens_host must have one entry per sequence")
    if lse_out is not None and tuple(lse_out.shape) != (T, Hq):
        raise ValueError("lse_out must be [S * q_len, Hq]")
    rc = load().pa_decode_multi_fp8(
        _dev(out, "out"),
        _dev(lse_out, "lse_out", torch.float32) if lse_out is not None else None,
        _dev(q, "q"),
        _dev(k_pool, "k_pool"),
        _dev(v_pool, "v_pool"),
        _dev(k_scales, "k_scales", torch.float32),
        _dev(v_scales, "v_scales", torch.float32),
        _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32),
        ch.ctypes.data,
        S, q_len, Hkv, Hq // Hkv, D, BS, NP, float(scale), int(split_pages),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream_ptr(stream),
    )
    return _check(rc)


def decode(out, q, k_pool, v_pool, block_tables, context_lens, context_lens_host, scale, workspace,
           lse_out=None, split_pages=0, stream=None):
    """pa_decode on torch tensors.

    q, out: [S, Hq, D]; k_pool, v_pool: [NP, Hkv, 16, D]; block_tables
    [S, MB] int32; context_lens [S] int32 (device) and context_lens_host
    (numpy or CPU tensor, same values); workspace: uint8 device tensor.
    """
    import torch

    S, Hq, D = q.shape
    NP, Hkv, BS, D2 = k_pool.shape
    if tuple(out.shape) != (S, Hq, D) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if tuple(v_pool.shape) != tuple(k_pool.shape) or k_pool.dtype != q.dtype or v_pool.dtype != q.dtype:
        raise ValueError("k_pool and v_pool must match each other and q's dtype")
    if D2 != D or Hq % Hkv:
        raise ValueError("head_dim mismatch or q heads not a multiple of kv heads")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    ch = _host_i32(context_lens_host, "context_lens_host")
    if ch.size != S:
        raise ValueError("context_lens_host must have one entry per sequence")
    if lse_out is not None and tuple(lse_out.shape) != (S, Hq):
        raise ValueError("lse_out must be [S, Hq]")
    rc = load().pa_decode(
        _dev(out, "out"),
        _dev(lse_out, "lse_out", torch.float32) if lse_out is not None else None,
        _dev(q, "q"),
        _dev(k_pool, "k_pool"),
        _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32),
        ch.ctypes.data,
        S, Hkv, Hq // Hkv, D, BS, NP, float(scale), _dtype_code(q), int(split_pages),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream_ptr(stream),
    )
    return _check(rc)


def decode_noalloc(out, q, k_pool, v_pool, block_tables, context_lens, context_lens_host, scale, lse_out=None,
                   split_pages=0, stream=None):
    """pa_decode_noalloc on torch tensors: pa_decode's arguments without a
    workspace (the library's fixed per-GPU scratch is used; calls that
    overlap on one GPU race)."""
    import torch

    S, Hq, D = q.shape
    NP, Hkv, BS, D2 = k_pool.shape
    if tuple(out.shape) != (S, Hq, D) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if tuple(v_pool.shape) != tuple(k_pool.shape) or k_pool.dtype != q.dtype or v_pool.dtype != q.dtype:
        raise ValueError("k_pool and v_pool must match each other and q's dtype")
    if D2 != D or Hq % Hkv:
        raise ValueError("head_dim mismatch or q heads not a multiple of kv heads")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    ch = _host_i32(context_lens_host, "context_lens_host")
    if ch.size != S:
        raise ValueError("context_lens_host must have one entry per sequence")
    if lse_out is not None and tuple(lse_out.shape) != (S, Hq):
        raise ValueError("lse_out must be [S, Hq]")
    rc = load().pa_decode_noalloc(
        _dev(out, "out"),
        _dev(lse_out, "lse_out", torch.float32) if lse_out is not None else None,
        _dev(q, "q"),
        _dev(k_pool, "k_pool"),
        _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32),
        block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32),
        ch.ctypes.data,
        S, Hkv, Hq // Hkv, D, BS, NP, float(scale), _dtype_code(q), int(split_pages), _stream_ptr(stream),
    )
    return _check(rc)


def prefix_cascade_workspace_size(max_num_seqs, num_kv_heads, gqa_ratio, head_dim, max_total_pages) -> int:
    return int(load().pa_prefix_cascade_workspace_size(max_num_seqs, num_kv_heads, gqa_ratio, head_dim,
                                                       max_total_pages))


def prefix_cascade(out, q, k_pool, v_pool, block_tables, context_lens, context_lens_host, group_seq_offsets,
                   group_seq_offsets_host, prefix_lens, prefix_lens_host, scale, workspace, lse_out=None,
                   stream=None):
    """pa_prefix_cascade on torch tensors (shapes as :func:`decode`);
    group_seq_offsets [NG+1] / prefix_lens [NG] int32 on the device plus
    host twins with the same values."""
    import torch

    S, Hq, D = q.shape
    NP, Hkv, BS, D2 = k_pool.shape
    if tuple(out.shape) != (S, Hq, D) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if tuple(v_pool.shape) != tuple(k_pool.shape) or k_pool.dtype != q.dtype or v_pool.dtype != q.dtype:
        raise ValueError("k_pool and v_pool must match each other and q's dtype")
    if D2 != D or Hq % Hkv:
        raise ValueError("head_dim mismatch or q heads not a multiple of kv heads")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    ch = _host_i32(context_lens_host, "context_lens_host")
    goh = _host_i32(group_seq_offsets_host, "group_seq_offsets_host")
    plh = _host_i32(prefix_lens_host, "prefix_lens_host")
    NG = plh.size
    if ch.size != S or goh.size != NG + 1 or group_seq_offsets.numel() != NG + 1 or prefix_lens.numel() != NG:
        raise ValueError("group arrays must be [NG+1] offsets and [NG] prefix lengths")
    if lse_out is not None and tuple(lse_out.shape) != (S, Hq):
        raise ValueError("lse_out must be [S, Hq]")
    rc = load().pa_prefix_cascade(
        _dev(out, "out"),
        _dev(lse_out, "lse_out", torch.float32) if lse_out is not None else None,
        _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), ch.ctypes.data, S, NG,
        _dev(group_seq_offsets, "group_seq_offsets", torch.int32), goh.ctypes.data,
        _dev(prefix_lens, "prefix_lens", torch.int32), plh.ctypes.data,
        Hkv, Hq // Hkv, D, BS, NP, float(scale), _dtype_code(q),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream_ptr(stream),
    )
    return _check(rc)


def prefix_cascade_fp8(out, q, k_pool, v_pool, k_scales, v_scales, block_tables, context_lens, context_lens_host,
                       group_seq_offsets, group_seq_offsets_host, prefix_lens, prefix_lens_host, scale, workspace,
                       lse_out=None, stream=None):
    """pa_prefix_cascade_fp8 on torch tensors: the groups of
    :func:`prefix_cascade`, the pools and scales of :func:`decode_fp8`."""
    import torch

    S, Hq, D = q.shape
    NP, Hkv, BS, D2 = k_pool.shape
    if q.dtype != torch.bfloat16 or tuple(out.shape) != (S, Hq, D) or out.dtype != torch.bfloat16:
        raise ValueError("q and out must be bfloat16 [S, Hq, D]")
    codes = (torch.uint8, torch.float8_e4m3fn)
    if tuple(v_pool.shape) != tuple(k_pool.shape) or k_pool.dtype not in codes or v_pool.dtype not in codes:
        raise ValueError("k_pool and v_pool must be [NP, Hkv, BS, D] uint8 / float8_e4m3fn")
    for t, nm in ((k_scales, "k_scales"), (v_scales, "v_scales")):
        if tuple(t.shape) != (NP, Hkv, BS) or t.dtype != torch.float32:
            raise ValueError(f"{nm} must be float32 [NP, Hkv, BS]")
    if D2 != D or Hq % Hkv:
        raise ValueError("head_dim mismatch or q heads not a multiple of kv heads")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables / context_lens must have one row per sequence")
    ch = _host_i32(context_lens_host, "context_lens_host")
    goh = _host_i32(group_seq_offsets_host, "group_seq_offsets_host")
    plh = _host_i32(prefix_lens_host, "prefix_lens_host")
    NG = plh.size
    if ch.size != S or goh.size != NG + 1 or group_seq_offsets.numel() != NG + 1 or prefix_lens.numel() != NG:
        raise ValueError("group arrays must be [NG+1] offsets and [NG] prefix lengths")
    if lse_out is not None and tuple(lse_out.shape) != (S, Hq):
        raise ValueError("lse_out must be [S, Hq]")
    rc = load().pa_prefix_cascade_fp8(
        _dev(out, "out"),
        _dev(lse_out, "lse_out", torch.float32) if lse_out is not None else None,
        _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(k_scales, "k_scales", torch.float32), _dev(v_scales, "v_scales", torch.float32),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), ch.ctypes.data, S, NG,
        _dev(group_seq_offsets, "group_seq_offsets", torch.int32), goh.ctypes.data,
        _dev(prefix_lens, "prefix_lens", torch.int32), plh.ctypes.data,
        Hkv, Hq // Hkv, D, BS, NP, float(scale),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream_ptr(stream),
    )
    return _check(rc)


def mixed_chunk_workspace_size(max_num_tokens, max_num_segments, num_kv_heads, gqa_ratio, head_dim,
                               max_total_pages) -> int:
    return int(load().pa_mixed_chunk_workspace_size(max_num_tokens, max_num_segments, num_kv_heads, gqa_ratio,
                                                    head_dim, max_total_pages))


def mixed_chunk(out, q, k_pool, v_pool, block_tables, cu_q_lens, cu_q_lens_host, context_lens, context_lens_host,
                scale, workspace, lse_out=None, stream=None):
    """pa_mixed_chunk on torch tensors.

    q, out: [T, Hq, D] (T = cu_q_lens[-1]); k_pool, v_pool: [NP, Hkv, 16, D];
    block_tables [S, MB] int32; cu_q_lens [S+1] / context_lens [S] int32 on
    the device plus host twins with the same values.
    """
    import torch

    T, Hq, D = q.shape
    NP, Hkv, BS, D2 = k_pool.shape
    if tuple(out.shape) != (T, Hq, D) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if tuple(v_pool.shape) != tuple(k_pool.shape) or k_pool.dtype != q.dtype or v_pool.dtype != q.dtype:
        raise ValueError("k_pool and v_pool must match each other and q's dtype")
    if D2 != D or Hq % Hkv:
        raise ValueError("head_dim mismatch or q heads not a multiple of kv heads")
    cq = _host_i32(cu_q_lens_host, "cu_q_lens_host")
    ch = _host_i32(context_lens_host, "context_lens_host")
    S = ch.size
    if cq.size != S + 1 or cu_q_lens.numel() != S + 1 or context_lens.numel() != S:
        raise ValueError("cu_q_lens must have one entry more than context_lens")
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must have one row per segment")
    if S and int(cq[-1]) != T:
        raise ValueError("q must have cu_q_lens[-1] rows")
    if lse_out is not None and tuple(lse_out.shape) != (T, Hq):
        raise ValueError("lse_out must be [T, Hq]")
    rc = load().pa_mixed_chunk(
        _dev(out, "out"),
        _dev(lse_out, "lse_out", torch.float32) if lse_out is not None else None,
        _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(cu_q_lens, "cu_q_lens", torch.int32), cq.ctypes.data,
        _dev(context_lens, "context_lens", torch.int32), ch.ctypes.data,
        S, Hkv, Hq // Hkv, D, BS, NP, float(scale), _dtype_code(q),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream_ptr(stream),
    )
    return _check(rc)


def mixed_chunk_fp8(out, q, k_pool, v_pool, k_scales, v_scales, block_tables, cu_q_lens, cu_q_lens_host,
                    context_lens, context_lens_host, scale, workspace, lse_out=None, stream=None):
    """pa_mixed_chunk_fp8 on torch tensors: the segments of
    :func:`mixed_chunk`, the pools and scales of :func:`decode_fp8`."""
    import torch

    T, Hq, D = q.shape
    NP, Hkv, BS, D2 = k_pool.shape
    if q.dtype != torch.bfloat16 or tuple(out.shape) != (T, Hq, D) or out.dtype != torch.bfloat16:
        raise ValueError("q and out must be bfloat16 [T, Hq, D]")
    codes = (torch.uint8, torch.float8_e4m3fn)
    if tuple(v_pool.shape) != tuple(k_pool.shape) or k_pool.dtype not in codes or v_pool.dtype not in codes:
        raise ValueError("k_pool and v_pool must be [NP, Hkv, BS, D] uint8 / float8_e4m3fn")
    for t, nm in ((k_scales, "k_scales"), (v_scales, "v_scales")):
        if tuple(t.shape) != (NP, Hkv, BS) or t.dtype != torch.float32:
            raise ValueError(f"{nm} must be float32 [NP, Hkv, BS]")
    if D2 != D or Hq % Hkv:
        raise ValueError("head_dim mismatch or q heads not a multiple of kv heads")
    cq = _host_i32(cu_q_lens_host, "cu_q_lens_host")
    ch = _host_i32(context_lens_host, "context_lens_host")
    S = ch.size
    if cq.size != S + 1 or cu_q_lens.numel() != S + 1 or context_lens.numel() != S:
        raise ValueError("cu_q_lens must have one entry more than context_lens")
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must have one row per segment")
    if S and int(cq[-1]) != T:
        raise ValueError("q must have cu_q_lens[-1] rows")
    if lse_out is not None and tuple(lse_out.shape) != (T, Hq):
        raise ValueError("lse_out must be [T, Hq]")
    rc = load().pa_mixed_chunk_fp8(
        _dev(out, "out"),
        _dev(lse_out, "lse_out", torch.float32) if lse_out is not None else None,
        _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(k_scales, "k_scales", torch.float32), _dev(v_scales, "v_scales", torch.float32),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(cu_q_lens, "cu_q_lens", torch.int32), cq.ctypes.data,
        _dev(context_lens, "context_lens", torch.int32), ch.ctypes.data,
        S, Hkv, Hq // Hkv, D, BS, NP, float(scale),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream_ptr(stream),
    )
    return _check(rc)


def kv_append(k_pool, v_pool, k_new, v_new, block_tables, cu_q_lens, cu_q_lens_host, context_lens,
              context_lens_host, stream=None):
    """pa_kv_append on torch tensors: the new rows into the pools, in place.

    k_pool, v_pool: [NP, Hkv, 16, D]; k_new, v_new: [T, Hkv, D] of the same
    dtype (T = cu_q_lens[-1]); block_tables [S, MB] int32; cu_q_lens [S+1] /
    context_lens [S] int32 on the device plus host twins with the same values.
    """
    import torch

    NP, Hkv, BS, D = k_pool.shape
    T = k_new.shape[0]
    if tuple(v_pool.shape) != tuple(k_pool.shape) or v_pool.dtype != k_pool.dtype:
        raise ValueError("k_pool and v_pool must match")
    if tuple(k_new.shape) != (T, Hkv, D) or tuple(v_new.shape) != (T, Hkv, D):
        raise ValueError("k_new and v_new must be [T, Hkv, D] with the pools' Hkv and D")
    if k_new.dtype != k_pool.dtype or v_new.dtype != k_pool.dtype:
        raise ValueError("new rows must have the pools' dtype")
    cq = _host_i32(cu_q_lens_host, "cu_q_lens_host")
    ch = _host_i32(context_lens_host, "context_lens_host")
    S = ch.size
    if cq.size != S + 1 or cu_q_lens.numel() != S + 1 or context_lens.numel() != S:
        raise ValueError("cu_q_lens must have one entry more than context_lens")
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must have one row per segment")
    if S and int(cq[-1]) != T:
        raise ValueError("k_new must have cu_q_lens[-1] rows")
    rc = load().pa_kv_append(
        _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(cu_q_lens, "cu_q_lens", torch.int32), cq.ctypes.data,
        _dev(context_lens, "context_lens", torch.int32), ch.ctypes.data,
        S, Hkv, D, BS, NP, _dtype_code(k_pool), _stream_ptr(stream),
    )
    return _check(rc)


def check_block_tables(block_tables, context_lens, num_pages, block_size=16, group_seq_offsets=None,
                       prefix_lens=None) -> int:
    bt = _host_i32(block_tables, "block_tables")
    ctx = _host_i32(context_lens, "context_lens")
    ng = 0
    go = pl = None
    if group_seq_offsets is not None:
        go = _host_i32(group_seq_offsets, "group_seq_offsets")
        pl = _host_i32(prefix_lens, "prefix_lens")
        ng = go.size - 1
    rc = load().pa_check_block_tables(
        bt.ctypes.data, bt.shape[1] if bt.ndim == 2 else 0, ctx.ctypes.data, ctx.size, block_size, num_pages, ng,
        go.ctypes.data if go is not None else None, pl.ctypes.data if pl is not None else None)
    return _check(rc)


def profile_enable(num_pairs: int) -> None:
    _check(load().pa_profile_enable(num_pairs))


def profile_collect(cap: int = 1 << 16):
    buf = (ctypes.c_float * cap)()
    n = _check(load().pa_profile_collect(buf, cap))
    return [buf[i] for i in range(n)]


def detect_prefix_groups(block_tables, context_lens, block_size=16, min_group=2, min_prefix_pages=1):
    """pa_detect_prefix_groups on host arrays (numpy, or CPU tensors).

    Returns (order [S], group_offsets [NG+1], prefix_lens [NG]) int32 numpy
    arrays: take sequences in ``order`` (tables, lengths, q rows) to call
    pa_prefix_cascade with these groups; its output rows then follow
    ``order`` too.
    """
    bt = _host_i32(block_tables, "block_tables")
    ctx = _host_i32(context_lens, "context_lens")
    if bt.ndim != 2 or bt.shape[0] != ctx.size:
        raise ValueError("block_tables must be [S, max_blocks] with one row per context length")
    S = ctx.size
    order = np.zeros(S, dtype=np.int32)
    offs = np.zeros(S + 1, dtype=np.int32)
    pref = np.zeros(max(S, 1), dtype=np.int32)
    ng = ctypes.c_int32(0)
    rc = load().pa_detect_prefix_groups(bt.ctypes.data, bt.shape[1], ctx.ctypes.data, S, int(block_size),
                                        int(min_group), int(min_prefix_pages), order.ctypes.data, offs.ctypes.data,
                                        pref.ctypes.data, ctypes.byref(ng))
    _check(rc)
    n = ng.value
    return order, offs[: n + 1].copy(), pref[:n].copy()


def kv_append_fp8(k_pool, v_pool, k_scales, v_scales, k_new, v_new, block_tables, cu_q_lens, cu_q_lens_host,
                  context_lens, context_lens_host, stream=None):
    """pa_kv_append_fp8 on torch tensors: the new rows quantised into an fp8
    cache, in place.

    k_pool, v_pool: [NP, Hkv, 16, D] uint8 (or float8_e4m3fn); k_scales,
    v_scales: [NP, Hkv, 16] float32; k_new, v_new: [T, Hkv, D] bfloat16 or
    float32; the rest as :func:`kv_append`.
    """
    import torch

    NP, Hkv, BS, D = k_pool.shape
    T = k_new.shape[0]
    codes = (torch.uint8, torch.float8_e4m3fn)
    if tuple(v_pool.shape) != tuple(k_pool.shape) or k_pool.dtype not in codes or v_pool.dtype not in codes:
        raise ValueError("k_pool and v_pool must be [NP, Hkv, BS, D] uint8 / float8_e4m3fn")
    for t, nm in ((k_scales, "k_scales"), (v_scales, "v_scales")):
        if tuple(t.shape) != (NP, Hkv, BS) or t.dtype != torch.float32:
            raise ValueError(f"{nm} must be float32 [NP, Hkv, BS]")
    if tuple(k_new.shape) != (T, Hkv, D) or tuple(v_new.shape) != (T, Hkv, D) or k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must be [T, Hkv, D] of one dtype")
    if k_new.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("new rows must be bfloat16 or float32")
    cq = _host_i32(cu_q_lens_host, "cu_q_lens_host")
    ch = _host_i32(context_lens_host, "context_lens_host")
    S = ch.size
    if cq.size != S + 1 or cu_q_lens.numel() != S + 1 or context_lens.numel() != S:
        raise ValueError("cu_q_lens must have one entry more than context_lens")
    if block_tables.dim() != 2 or block_tables.shape[0] != S:
        raise ValueError("block_tables must have one row per segment")
    if S and int(cq[-1]) != T:
        raise ValueError("k_new must have cu_q_lens[-1] rows")
    rc = load().pa_kv_append_fp8(
        _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), _dev(k_scales, "k_scales", torch.float32),
        _dev(v_scales, "v_scales", torch.float32), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(cu_q_lens, "cu_q_lens", torch.int32), cq.ctypes.data, _dev(context_lens, "context_lens", torch.int32),
        ch.ctypes.data, S, Hkv, D, BS, NP, _dtype_code(k_new), _stream_ptr(stream),
    )
    return _check(rc)
