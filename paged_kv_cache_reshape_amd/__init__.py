"""Python binding of libpagedattn (paged KV write, decode and prefill attention).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libpagedattn.so``.  PyTorch supplies device memory and the
current stream.  If the library has not been built, importing works but every
call raises -- there is no fallback path.

Functions (names follow the C ABI in ``include/pagedattn.h``):
  reshape_and_cache(key, value, k_cache, v_cache, slot_mapping)
  paged_attention_decode(q, k_cache, v_cache, block_tables, context_lens,
                         scale, partition_size=0, out=None, workspace=None)
  decode_step(q, key, value, k_cache, v_cache, block_tables, context_lens,
              scale, ...)   the write of each sequence's new token fused in
  decode_step_noalloc(q, key, value, k_cache, v_cache, block_tables,
                      context_lens, scale, out, partition_size=0)
                    the same with the library's own device buffer: no allocation
  paged_attention_prefill(q, k_cache, v_cache, block_tables, context_lens,
                          query_start, scale, max_query_len=None, out=None)
  copy_blocks(k_cache, v_cache, block_pairs)
  decode_partition_size(...), decode_workspace_bytes(...)
  debug_gather_kv(k_cache, v_cache, block_tables, context_lens)
  reload_options()   re-read the PAGEDATTN_* overrides (tests, tuning)
"""
from __future__ import annotations

import contextlib
import ctypes
import functools
import os
import threading

import torch

__all__ = [
    "LIB_PATH", "load_library", "PagedAttnError", "reshape_and_cache",
    "paged_attention_decode", "decode_step", "paged_attention_prefill", "copy_blocks",
    "decode_partition_size", "decode_workspace_bytes", "debug_gather_kv", "workspace_for",
    "counters_for", "reload_options", "decode_step_noalloc",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so")

PA_DTYPE_F32 = 0
PA_DTYPE_BF16 = 1
_DTYPES = {torch.float32: PA_DTYPE_F32, torch.bfloat16: PA_DTYPE_BF16}

_lib = None
_lock = threading.Lock()


class PagedAttnError(RuntimeError):
    """A libpagedattn call returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load (once) and return the C library; raises if it is not built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = path or LIB_PATH
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with "
                "`python -m paged_kv_cache_reshape_amd.build` (no fallback exists)")
        lib = ctypes.CDLL(path)
        vp, i32, i64, sz, f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                 ctypes.c_size_t, ctypes.c_float)
        lib.pa_version.restype = i32
        lib.pa_version.argtypes = []
        lib.pa_status_string.restype = ctypes.c_char_p
        lib.pa_status_string.argtypes = [i32]
        lib.pa_last_error_message.restype = ctypes.c_char_p
        lib.pa_last_error_message.argtypes = []
        lib.pa_reload_options.restype = None
        lib.pa_reload_options.argtypes = []
        lib.pa_reshape_and_cache.restype = i32
        lib.pa_reshape_and_cache.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                             i32, i32, vp]
        lib.pa_decode_partition_size.restype = i32
        lib.pa_decode_partition_size.argtypes = [i32] * 7
        lib.pa_decode_workspace_bytes.restype = sz
        lib.pa_decode_workspace_bytes.argtypes = [i32] * 7
        lib.pa_paged_attention_decode.restype = i32
        lib.pa_paged_attention_decode.argtypes = [
            vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32,
            vp, sz, vp, i64, i32, vp]
        lib.pa_decode_step.restype = i32
        lib.pa_decode_step.argtypes = [
            vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32,
            vp, sz, vp, i64, i32, vp]
        lib.pa_decode_step_noalloc.restype = i32
        lib.pa_decode_step_noalloc.argtypes = [
            vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32,
            i32, vp]
        lib.pa_paged_attention_prefill.restype = i32
        lib.pa_paged_attention_prefill.argtypes = [
            vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, f32,
            i32, vp]
        lib.pa_copy_blocks.restype = i32
        lib.pa_copy_blocks.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
        lib.pa_debug_gather_kv.restype = i32
        lib.pa_debug_gather_kv.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                           i32, i32, i32, vp]
        _lib = lib
        return lib


def reload_options() -> None:
    """Make the library re-read its PAGEDATTN_* environment overrides (it
    reads them once otherwise); the workspace sizes cached here follow."""
    load_library().pa_reload_options()
    decode_workspace_bytes.cache_clear()


def _check(status: int, what: str) -> None:
    if status != 0:
        lib = load_library()
        msg = lib.pa_last_error_message().decode()
        raise PagedAttnError(status, f"{what}: {lib.pa_status_string(status).decode()}"
                                     f" ({msg})")


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"dtype {t.dtype} not supported (float32 or bfloat16)") from None


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _on(device: torch.device):
    """Make `device` current for the call (a no-op context when it already
    is: entering torch.cuda.device costs more than a launch on small batches)."""
    if device.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(device)


def _same_device(*ts: torch.Tensor) -> torch.device:
    dev = ts[0].device
    _need(dev.type == "cuda", "tensors must be on a GPU")
    for t in ts:
        _need(t.device == dev, "all tensors must be on the same GPU")
        _need(t.is_contiguous(), "tensors must be contiguous")
    return dev


def reshape_and_cache(key: torch.Tensor, value: torch.Tensor, k_cache: torch.Tensor,
                      v_cache: torch.Tensor, slot_mapping: torch.Tensor) -> None:
    """Write new K/V rows ``[N, Hkv, D]`` into the paged caches at ``slot_mapping``."""
    lib = load_library()
    dev = _same_device(key, value, k_cache, v_cache, slot_mapping)
    _need(k_cache.dim() == 4 and v_cache.shape == k_cache.shape,
          "caches must be [num_blocks, block_size, Hkv, D] and alike")
    nb, bs, hkv, d = k_cache.shape
    _need(key.dim() == 3 and key.shape[1:] == (hkv, d) and value.shape == key.shape,
          "key/value must be [N, Hkv, D] matching the cache")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.shape == (key.shape[0],),
          "slot_mapping must be int64 [N]")
    dt = _dtype_code(k_cache)
    _need(key.dtype == value.dtype == v_cache.dtype == k_cache.dtype, "dtype mismatch")
    with _on(dev):
        st = lib.pa_reshape_and_cache(
            key.data_ptr(), value.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            slot_mapping.data_ptr(), key.shape[0], hkv, d, nb, bs, dt, _stream(dev))
    _check(st, "pa_reshape_and_cache")


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor,
                block_pairs: torch.Tensor) -> None:
    """Copy-on-write of shared blocks: for each row (src, dst) of the int64
    ``[n, 2]`` device tensor ``block_pairs``, block dst of both caches becomes
    a copy of block src."""
    lib = load_library()
    dev = _same_device(k_cache, v_cache, block_pairs)
    _need(k_cache.dim() == 4 and v_cache.shape == k_cache.shape,
          "caches must be [num_blocks, block_size, Hkv, D] and alike")
    _need(block_pairs.dtype == torch.int64 and block_pairs.dim() == 2
          and block_pairs.shape[1] == 2 and block_pairs.is_contiguous(),
          "block_pairs must be a contiguous int64 [n, 2] tensor")
    nb, bs, hkv, d = k_cache.shape
    dt = _dtype_code(k_cache)
    _need(v_cache.dtype == k_cache.dtype, "dtype mismatch")
    with _on(dev):
        st = lib.pa_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(), block_pairs.data_ptr(),
                                block_pairs.shape[0], hkv, d, nb, bs, dt, _stream(dev))
    _check(st, "pa_copy_blocks")


def decode_partition_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                          max_blocks_per_seq, block_size, requested=0) -> int:
    return int(load_library().pa_decode_partition_size(
        num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size,
        requested))


@functools.lru_cache(maxsize=256)
def decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                           max_blocks_per_seq, block_size, partition_size=0) -> int:
    return int(load_library().pa_decode_workspace_bytes(
        num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size,
        partition_size))


_workspaces: dict = {}
_counters: dict = {}


def workspace_for(device: torch.device, nbytes: int,
                  stream: int | None = None) -> torch.Tensor | None:
    """A zero-initialised workspace of >= nbytes for this device and current
    stream (cached).  Every decode call leaves the workspace it used at zero,
    so it is reused by later calls on the same stream, whatever their sizes,
    and replaced by a larger one when needed.
    """
    if nbytes == 0:
        return None
    key = (device.index, _stream(device) if stream is None else stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def counters_for(device: torch.device, count: int, stream: int | None = None) -> torch.Tensor:
    """Zero-initialised int32 arrival counters (>= count) for this device and
    current stream.  Every decode call leaves the counters it used at zero, so
    one array serves all later calls on the stream, whatever their sizes."""
    key = (device.index, _stream(device) if stream is None else stream)
    c = _counters.get(key)
    if c is None or c.numel() < count:
        c = torch.zeros(max(count, 1024), dtype=torch.int32, device=device)
        _counters[key] = c
    return c


def _decode_call(q, k_cache, v_cache, block_tables, context_lens, scale, partition_size,
                 out, workspace, counters, step, noalloc=False):
    """Checks and buffers shared by the decode entry points; `step` is None or
    the (key, value) rows to write; `noalloc` calls pa_decode_step_noalloc
    (no workspace, no counters, `out` given)."""
    lib = load_library()
    extra = step if step is not None else ()
    dev = _same_device(q, k_cache, v_cache, block_tables, context_lens, *extra)
    _need(q.dim() == 3, "q must be [B, Hq, D]")
    B, hq, d = q.shape
    _need(k_cache.dim() == 4 and v_cache.shape == k_cache.shape,
          "caches must be [num_blocks, block_size, Hkv, D] and alike")
    nb, bs, hkv, d2 = k_cache.shape
    _need(d2 == d, "head_dim of q and cache differ")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == B, "block_tables must be int32 [B, max_blocks]")
    _need(context_lens.dtype == torch.int32 and context_lens.shape == (B,),
          "context_lens must be int32 [B]")
    dt = _dtype_code(q)
    _need(k_cache.dtype == v_cache.dtype == q.dtype, "dtype mismatch")
    if step is not None:
        key, value = step
        _need(key.shape == (B, hkv, d) and value.shape == key.shape,
              "key/value must be [B, Hkv, D] matching q and the cache")
        _need(key.dtype == value.dtype == q.dtype, "dtype mismatch")
    max_blocks = block_tables.shape[1]
    if out is None:
        out = torch.empty_like(q)
    else:
        _same_device(out)
        _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    stream = _stream(dev)
    if noalloc:
        with _on(dev):
            st = lib.pa_decode_step_noalloc(
                out.data_ptr(), q.data_ptr(), key.data_ptr(), value.data_ptr(),
                k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
                context_lens.data_ptr(), B, hq, hkv, d, nb, bs, max_blocks, float(scale),
                partition_size, dt, stream)
        _check(st, "pa_decode_step_noalloc")
        return out
    need = decode_workspace_bytes(B, hq, hkv, d, max_blocks, bs, partition_size)
    if workspace is None:
        workspace = workspace_for(dev, need, stream)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if need and counters is None:
        counters = counters_for(dev, B * hkv, stream)
    if counters is not None:
        _need(counters.dtype == torch.int32 and counters.device == dev
              and counters.is_contiguous(), "counters must be contiguous int32 on the GPU")
    c_ptr = counters.data_ptr() if counters is not None else None
    c_len = counters.numel() if counters is not None else 0
    tail = (block_tables.data_ptr(), context_lens.data_ptr(), B, hq, hkv, d, nb, bs,
            max_blocks, float(scale), partition_size, ws_ptr, ws_len, c_ptr, c_len, dt,
            stream)
    with _on(dev):
        if step is None:
            st = lib.pa_paged_attention_decode(out.data_ptr(), q.data_ptr(), k_cache.data_ptr(),
                                               v_cache.data_ptr(), *tail)
            what = "pa_paged_attention_decode"
        else:
            st = lib.pa_decode_step(out.data_ptr(), q.data_ptr(), key.data_ptr(),
                                    value.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                    *tail)
            what = "pa_decode_step"
    _check(st, what)
    return out


def paged_attention_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           block_tables: torch.Tensor, context_lens: torch.Tensor,
                           scale: float, partition_size: int = 0,
                           out: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None,
                           counters: torch.Tensor | None = None) -> torch.Tensor:
    """Decode attention ``out[B, Hq, D]`` over the paged caches.

    ``workspace`` (uint8) and ``counters`` (int32), both all zero before
    first use and kept zero by every call, default to per-stream buffers
    managed here.
    """
    return _decode_call(q, k_cache, v_cache, block_tables, context_lens, scale, partition_size,
                        out, workspace, counters, None)


def decode_step(q: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                context_lens: torch.Tensor, scale: float, partition_size: int = 0,
                out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                counters: torch.Tensor | None = None) -> torch.Tensor:
    """One decode step in one launch: each sequence's new rows ``key[b]`` /
    ``value[b]`` (``[B, Hkv, D]``) are written at its position
    ``context_lens[b] - 1``, then ``out[B, Hq, D]`` is computed as by
    :func:`paged_attention_decode`."""
    return _decode_call(q, k_cache, v_cache, block_tables, context_lens, scale, partition_size,
                        out, workspace, counters, (key, value))


def decode_step_noalloc(q: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                        k_cache: torch.Tensor, v_cache: torch.Tensor,
                        block_tables: torch.Tensor, context_lens: torch.Tensor,
                        scale: float, out: torch.Tensor,
                        partition_size: int = 0) -> torch.Tensor:
    """:func:`decode_step` through ``pa_decode_step_noalloc``: no workspace or
    counters are allocated (the library's static device buffer serves, one
    per GPU, shared by every call on it), and ``out`` is the caller's."""
    _need(out is not None, "decode_step_noalloc writes into the caller's out")
    return _decode_call(q, k_cache, v_cache, block_tables, context_lens, scale, partition_size,
                        out, None, None, (key, value), noalloc=True)


def paged_attention_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            block_tables: torch.Tensor, context_lens: torch.Tensor,
                            query_start: torch.Tensor, scale: float,
                            max_query_len: int | None = None,
                            out: torch.Tensor | None = None) -> torch.Tensor:
    """Causal prefill attention ``out[T, Hq, D]`` over the paged caches.

    Sequence b's new tokens are rows ``query_start[b] : query_start[b+1]`` of
    ``q``, the last ones of its ``context_lens[b]`` positions (their K/V rows
    already written).  ``max_query_len`` bounds the rows per sequence; if not
    given it is read from ``query_start`` (a device-to-host copy).
    """
    lib = load_library()
    dev = _same_device(q, k_cache, v_cache, block_tables, context_lens, query_start)
    _need(q.dim() == 3, "q must be [T, Hq, D]")
    T, hq, d = q.shape
    _need(k_cache.dim() == 4 and v_cache.shape == k_cache.shape,
          "caches must be [num_blocks, block_size, Hkv, D] and alike")
    nb, bs, hkv, d2 = k_cache.shape
    _need(d2 == d, "head_dim of q and cache differ")
    B = context_lens.shape[0]
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == B, "block_tables must be int32 [B, max_blocks]")
    _need(context_lens.dtype == torch.int32 and context_lens.dim() == 1,
          "context_lens must be int32 [B]")
    _need(query_start.dtype == torch.int32 and query_start.shape == (B + 1,),
          "query_start must be int32 [B + 1]")
    dt = _dtype_code(q)
    _need(k_cache.dtype == v_cache.dtype == q.dtype, "dtype mismatch")
    if max_query_len is None:
        qs = query_start.cpu()
        max_query_len = int((qs[1:] - qs[:-1]).max()) if B else 0
    if out is None:
        out = torch.empty_like(q)
    else:
        _same_device(out)
        _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    with _on(dev):
        st = lib.pa_paged_attention_prefill(
            out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            block_tables.data_ptr(), context_lens.data_ptr(), query_start.data_ptr(), B, T,
            hq, hkv, d, nb, bs, block_tables.shape[1], int(max_query_len), float(scale), dt,
            _stream(dev))
    _check(st, "pa_paged_attention_prefill")
    return out


def debug_gather_kv(k_cache: torch.Tensor, v_cache: torch.Tensor,
                    block_tables: torch.Tensor, context_lens: torch.Tensor):
    """Dense ``[B, max_blocks * block_size, Hkv, D]`` copies of each sequence's rows."""
    lib = load_library()
    dev = _same_device(k_cache, v_cache, block_tables, context_lens)
    nb, bs, hkv, d = k_cache.shape
    B, max_blocks = block_tables.shape
    _need(block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32,
          "block_tables and context_lens must be int32")
    dt = _dtype_code(k_cache)
    kd = torch.empty((B, max_blocks * bs, hkv, d), dtype=k_cache.dtype, device=dev)
    vd = torch.empty_like(kd)
    with _on(dev):
        st = lib.pa_debug_gather_kv(
            kd.data_ptr(), vd.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            block_tables.data_ptr(), context_lens.data_ptr(), B, hkv, d, nb, bs,
            max_blocks, dt, _stream(dev))
    _check(st, "pa_debug_gather_kv")
    return kd, vd
