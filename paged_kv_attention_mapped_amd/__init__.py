"""Paged KV-cache attention for AMD Instinct MI355X (gfx950).

A thin ctypes binding over the C ABI of ``libpkv.so`` (declared in
``include/pkv.h``).  It only marshals arguments: every step of the path runs
in the HIP kernels of that library.  Torch provides device memory (tensors)
and the stream (the current torch stream); bf16 data may be passed as
``torch.bfloat16`` or as its 16-bit patterns in ``torch.int16``/``uint16``.

The library is loaded after torch so that both use torch's HIP runtime.
If it has not been built (``python -m paged_kv_attention_mapped_amd.build``),
every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "PkvError",
    "StepGraph",
    "append",
    "append_mapped",
    "capture_graph",
    "decode",
    "decode_append",
    "decode_combine",
    "decode_method",
    "decode_noalloc",
    "decode_plan",
    "decode_split",
    "decode_stream",
    "decode_stream_merge",
    "decode_stream_waves",
    "decode_workspace_bytes",
    "exported_symbols",
    "lib",
    "lib_path",
    "page_alloc",
    "page_free",
    "prefill_varlen",
    "slot_mapping",
    "stream_read",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpkv.so")

EXPORTS = (
    "pkv_status_string",
    "pkv_device_info",
    "pkv_stream_read",
    "pkv_slot_mapping",
    "pkv_append",
    "pkv_append_mapped",
    "pkv_page_alloc",
    "pkv_page_free",
    "pkv_decode_plan",
    "pkv_decode_method",
    "pkv_decode_workspace_bytes",
    "pkv_decode",
    "pkv_decode_append",
    "pkv_decode_noalloc",
    "pkv_decode_split",
    "pkv_decode_combine",
    "pkv_decode_stream_waves",
    "pkv_decode_stream_workspace_bytes",
    "pkv_decode_stream",
    "pkv_decode_stream_merge",
    "pkv_prefill_varlen",
    "pkv_prefill_split_workspace_bytes",
    "pkv_prefill_varlen_split",
    "pkv_graph_begin",
    "pkv_graph_end",
    "pkv_graph_launch",
    "pkv_graph_nodes",
    "pkv_graph_destroy",
)


class PkvError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status} ({msg})")
        self.status = status


_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t
_SIGS = {
    "pkv_status_string": ([_I32], ctypes.c_char_p),
    "pkv_device_info": ([_P, _P], _I32),
    "pkv_stream_read": ([_P, _SZ, _I32, _P, _P], _I32),
    "pkv_slot_mapping": ([_P, _I32, _P, _P, _I32, _I32, _I32, _I32, _P, _P], _I32),
    "pkv_append": ([_P, _P, _P, _I32, _I32, _I32, _P, _P, _I64, _P], _I32),
    "pkv_append_mapped": ([_P, _P, _P, _I32, _P, _P] + [_I32] * 7 + [_P, _P, _P, _P], _I32),
    "pkv_page_alloc": ([_P, _P, _I32, _P, _I32, _I32, _P, _P, _I32, _P, _P], _I32),
    "pkv_page_free": ([_P, _P, _I32, _P, _I32, _I32, _P, _P, _I32, _P, _P], _I32),
    "pkv_decode_plan": ([_I32, _I32, _I32, _I32, _I32, _I32, _P, _P], _I32),
    "pkv_decode_method": ([_I32] * 8 + [_P, _P], _I32),
    "pkv_decode_workspace_bytes": ([_I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32], _SZ),
    "pkv_decode": ([_P, _P, _P, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                    _F, _I32, _I32, _P, _SZ, _P, _P], _I32),
    "pkv_decode_append": ([_P, _P, _P, _P, _P, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                           _I32, _F, _I32, _I32, _P, _SZ, _P, _P], _I32),
    "pkv_decode_noalloc": ([_P, _P, _P, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                            _F, _I32, _I32, _P, _P], _I32),
    "pkv_decode_split": ([_P, _P, _P, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                          _F, _I32, _I32, _I32, _P, _P, _P, _P], _I32),
    "pkv_decode_combine": ([_P, _P, _P, _I32, _I32, _I32, _I32, _P, _P], _I32),
    "pkv_decode_stream_waves": ([_I32, _I32, _I32, _I32, _I32, _I32, _I32, _P], _I32),
    "pkv_decode_stream_workspace_bytes": ([_I32, _I32, _I32, _I32], _SZ),
    "pkv_decode_stream": ([_P, _P, _P, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32, _I32, _F,
                           _I32, _I32, _P, _SZ, _P, _P], _I32),
    "pkv_decode_stream_merge": ([_P, _SZ, _I32, _I32, _I32, _I32, _P, _P], _I32),
    "pkv_prefill_varlen": ([_P, _P, _P, _P, _I32, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                            _I32, _I32, _I32, _F, _I32, _P, _P], _I32),
    "pkv_prefill_split_workspace_bytes": ([_I32, _I32, _I32, _I32], _SZ),
    "pkv_prefill_varlen_split": ([_P, _P, _P, _P, _I32, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                  _I32, _I32, _I32, _I32, _F, _I32, _I32, _P, _SZ, _P, _P], _I32),
    "pkv_graph_begin": ([_P], _I32),
    "pkv_graph_end": ([_P, _P], _I32),
    "pkv_graph_launch": ([_P, _P], _I32),
    "pkv_graph_nodes": ([_P, _P, _P], _I32),
    "pkv_graph_destroy": ([_P], _I32),
}


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded ``libpkv.so`` (loaded on first use; raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(
                f"{_LIB_PATH} is missing: build it with "
                "`python -m paged_kv_attention_mapped_amd.build` (there is no fallback path)")
        handle = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def exported_symbols():
    """Names of the C ABI entry points the loaded library exports."""
    h = lib()
    return [n for n in EXPORTS if hasattr(h, n)]


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _check(fn: str, status: int):
    if status != 0:
        msg = lib().pkv_status_string(status).decode()
        raise PkvError(fn, status, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _bf16(t, name):
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name}: expected bf16 data (bfloat16 or 16-bit patterns), got {t.dtype}")


def _i32(t, name):
    if t.dtype != torch.int32:
        raise TypeError(f"{name}: expected int32, got {t.dtype}")


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def slot_mapping(block_tables, cu_seq_lens_q, cu_seq_lens_k, *, page_size, num_pages,
                 total_tokens, out=None, stream=None):
    """Pool row of every new token (``pkv_slot_mapping``); returns int32 [total_tokens]."""
    _i32(block_tables, "block_tables"); _i32(cu_seq_lens_q, "cu_q"); _i32(cu_seq_lens_k, "cu_k")
    if out is None:
        out = torch.empty(total_tokens, dtype=torch.int32, device=block_tables.device)
    _dev(block_tables, cu_seq_lens_q, cu_seq_lens_k, out)
    num_seqs = cu_seq_lens_q.numel() - 1
    _check("pkv_slot_mapping", lib().pkv_slot_mapping(
        _ptr(block_tables), block_tables.shape[1], _ptr(cu_seq_lens_q), _ptr(cu_seq_lens_k),
        num_seqs, total_tokens, page_size, num_pages, _ptr(out), _stream(stream)))
    return out


def append(k_new, v_new, slot_mapping, k_pool, v_pool, stream=None):
    """Bit-exact copy of ``[T, Hkv, D]`` rows into ``[Hkv, num_slots, D]`` pools (``pkv_append``)."""
    _bf16(k_new, "k_new"); _bf16(v_new, "v_new"); _bf16(k_pool, "k_pool"); _bf16(v_pool, "v_pool")
    _i32(slot_mapping, "slot_mapping")
    _dev(k_new, v_new, slot_mapping, k_pool, v_pool)
    T, hkv, d = k_new.shape
    if v_new.shape != k_new.shape or k_pool.shape != v_pool.shape:
        raise ValueError("shape mismatch")
    if k_pool.shape[0] != hkv or k_pool.shape[2] != d or slot_mapping.numel() < T:
        raise ValueError("pool / slot_mapping shape mismatch")
    _check("pkv_append", lib().pkv_append(
        _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), T, hkv, d, _ptr(k_pool), _ptr(v_pool),
        k_pool.shape[1], _stream(stream)))


def append_mapped(k_new, v_new, block_tables, cu_seq_lens_q, cu_seq_lens_k, k_pool, v_pool, *,
                  page_size, max_seqlen_q=None, slot_mapping_out=None, stream=None):
    """Slot addressing and append in one launch (``pkv_append_mapped``).

    ``k_pool``/``v_pool`` are ``[Hkv, num_pages * page_size, D]``;
    ``max_seqlen_q`` bounds the new rows of any one sequence (default: the
    token count, always a bound); when ``slot_mapping_out`` (int32 ``[T]``)
    is given it receives every token's slot.
    """
    _bf16(k_new, "k_new"); _bf16(v_new, "v_new"); _bf16(k_pool, "k_pool"); _bf16(v_pool, "v_pool")
    _i32(block_tables, "block_tables"); _i32(cu_seq_lens_q, "cu_q"); _i32(cu_seq_lens_k, "cu_k")
    if slot_mapping_out is not None:
        _i32(slot_mapping_out, "slot_mapping_out")
    _dev(k_new, v_new, block_tables, cu_seq_lens_q, cu_seq_lens_k, k_pool, v_pool,
         slot_mapping_out)
    T, hkv, d = k_new.shape
    if v_new.shape != k_new.shape or k_pool.shape != v_pool.shape:
        raise ValueError("shape mismatch")
    if k_pool.shape[0] != hkv or k_pool.shape[2] != d or k_pool.shape[1] % page_size:
        raise ValueError("pool shape must be [Hkv, num_pages * page_size, D]")
    if slot_mapping_out is not None and slot_mapping_out.numel() < T:
        raise ValueError("slot_mapping_out is shorter than the token count")
    _check("pkv_append_mapped", lib().pkv_append_mapped(
        _ptr(k_new), _ptr(v_new), _ptr(block_tables), block_tables.shape[1],
        _ptr(cu_seq_lens_q), _ptr(cu_seq_lens_k), cu_seq_lens_q.numel() - 1, T,
        T if max_seqlen_q is None else max_seqlen_q, page_size,
        k_pool.shape[1] // page_size, hkv, d, _ptr(k_pool), _ptr(v_pool),
        _ptr(slot_mapping_out), _stream(stream)))


def page_alloc(cu_seq_lens_q, cu_seq_lens_k, block_tables, free_pages, free_count, *,
               page_size, status=None, stream=None):
    """Pages for every sequence's new tokens from the device free stack (``pkv_page_alloc``).

    ``block_tables`` int32 ``[B, max_pages]``, ``free_pages`` int32 ``[num_pages]``
    and ``free_count`` / ``status`` int32 ``[1]`` are device tensors updated in place.
    """
    for t, n in ((cu_seq_lens_q, "cu_q"), (cu_seq_lens_k, "cu_k"), (block_tables, "block_tables"),
                 (free_pages, "free_pages"), (free_count, "free_count")):
        _i32(t, n)
    if status is not None:
        _i32(status, "status")
    _dev(cu_seq_lens_q, cu_seq_lens_k, block_tables, free_pages, free_count, status)
    _check("pkv_page_alloc", lib().pkv_page_alloc(
        _ptr(cu_seq_lens_q), _ptr(cu_seq_lens_k), cu_seq_lens_q.numel() - 1, _ptr(block_tables),
        block_tables.shape[1], page_size, _ptr(free_pages), _ptr(free_count), free_pages.numel(),
        _ptr(status), _stream(stream)))


def page_free(seq_lens, release, block_tables, free_pages, free_count, *, page_size,
              status=None, stream=None):
    """Return the pages of released sequences to the device free stack (``pkv_page_free``)."""
    for t, n in ((seq_lens, "seq_lens"), (release, "release"), (block_tables, "block_tables"),
                 (free_pages, "free_pages"), (free_count, "free_count")):
        _i32(t, n)
    if status is not None:
        _i32(status, "status")
    _dev(seq_lens, release, block_tables, free_pages, free_count, status)
    _check("pkv_page_free", lib().pkv_page_free(
        _ptr(seq_lens), _ptr(release), seq_lens.numel(), _ptr(block_tables),
        block_tables.shape[1], page_size, _ptr(free_pages), _ptr(free_count), free_pages.numel(),
        _ptr(status), _stream(stream)))


def device_info():
    """``(compute_units, max_clock_khz)`` of the current device (``pkv_device_info``)."""
    cus, khz = ctypes.c_int32(0), ctypes.c_int32(0)
    _check("pkv_device_info", lib().pkv_device_info(ctypes.byref(cus), ctypes.byref(khz)))
    return cus.value, khz.value


def stream_read(buffer, workgroups, sink, stream=None):
    """Streaming read of a device buffer (``pkv_stream_read``): the practical
    HBM read ceiling; ``sink`` is int32/uint32 ``[4 * workgroups]``."""
    _dev(buffer, sink)
    if sink.numel() < 4 * workgroups:
        raise ValueError("sink needs 4 words per workgroup")
    _check("pkv_stream_read", lib().pkv_stream_read(
        _ptr(buffer), buffer.numel() * buffer.element_size(), workgroups, _ptr(sink),
        _stream(stream)))


DECODE_METHODS = {0: "direct", 1: "split", 2: "stream"}


def decode_method(num_seqs, num_q_heads, num_kv_heads, head_dim, page_size, max_seq_len,
                  window=0, num_splits=0):
    """``(method, count)`` that ``pkv_decode`` uses: ``("direct", 1)``,
    ``("split", splits)`` or ``("stream", waves)`` (``pkv_decode_method``)."""
    m, c = ctypes.c_int32(0), ctypes.c_int32(0)
    _check("pkv_decode_method", lib().pkv_decode_method(
        num_seqs, num_q_heads, num_kv_heads, head_dim, page_size, max_seq_len, window,
        num_splits, ctypes.byref(m), ctypes.byref(c)))
    return DECODE_METHODS[m.value], c.value


def decode_plan(num_seqs, num_kv_heads, page_size, max_seq_len, window=0, num_splits=0):
    """``(num_splits, pages_per_split)`` that ``decode`` uses (``pkv_decode_plan``)."""
    s, p = ctypes.c_int32(0), ctypes.c_int32(0)
    _check("pkv_decode_plan", lib().pkv_decode_plan(
        num_seqs, num_kv_heads, page_size, max_seq_len, window, num_splits,
        ctypes.byref(s), ctypes.byref(p)))
    return s.value, p.value


def decode_workspace_bytes(num_seqs, num_q_heads, head_dim, num_kv_heads, page_size,
                           max_seq_len, window=0, num_splits=0):
    return int(lib().pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, num_kv_heads,
                                                page_size, max_seq_len, window, num_splits))


def _pool_shape(k_pool, page_size):
    hkv, slots, d = k_pool.shape
    if slots % page_size:
        raise ValueError("pool rows must be a multiple of page_size")
    return hkv, slots // page_size, d


def decode(q, k_pool, v_pool, block_tables, seq_lens, max_seq_len, *, page_size, scale=None,
           window=0, num_splits=0, workspace=None, out=None, stream=None):
    """GQA decode attention over the paged pool (``pkv_decode``); returns bf16 [B, Hq, D]."""
    _bf16(q, "q"); _bf16(k_pool, "k_pool"); _bf16(v_pool, "v_pool")
    _i32(block_tables, "block_tables"); _i32(seq_lens, "seq_lens")
    B, hq, d = q.shape
    hkv, num_pages, d2 = _pool_shape(k_pool, page_size)
    if d2 != d or v_pool.shape != k_pool.shape or block_tables.shape[0] < B or seq_lens.numel() < B:
        raise ValueError("shape mismatch")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out is None:
        out = torch.empty((B, hq, d), dtype=torch.bfloat16, device=q.device)
    need = decode_workspace_bytes(B, hq, d, hkv, page_size, max_seq_len, window, num_splits)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _dev(q, k_pool, v_pool, block_tables, seq_lens, out, workspace)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pkv_decode", lib().pkv_decode(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), block_tables.shape[1],
        _ptr(seq_lens), B, hq, hkv, d, page_size, num_pages, max_seq_len, float(scale), window,
        num_splits, _ptr(workspace), wsb, _ptr(out), _stream(stream)))
    return out


def decode_noalloc(q, k_pool, v_pool, block_tables, seq_lens, max_seq_len, *, page_size,
                   scale=None, window=0, num_splits=0, out=None, stream=None):
    """``pkv_decode_noalloc``: decode with the library's own per-GPU scratch
    for its partials (no workspace); returns bf16 [B, Hq, D] (``out`` may be
    given, so that nothing is allocated)."""
    _bf16(q, "q"); _bf16(k_pool, "k_pool"); _bf16(v_pool, "v_pool")
    _i32(block_tables, "block_tables"); _i32(seq_lens, "seq_lens")
    B, hq, d = q.shape
    hkv, num_pages, d2 = _pool_shape(k_pool, page_size)
    if d2 != d or v_pool.shape != k_pool.shape or block_tables.shape[0] < B or seq_lens.numel() < B:
        raise ValueError("shape mismatch")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out is None:
        out = torch.empty((B, hq, d), dtype=torch.bfloat16, device=q.device)
    _dev(q, k_pool, v_pool, block_tables, seq_lens, out)
    _check("pkv_decode_noalloc", lib().pkv_decode_noalloc(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), block_tables.shape[1],
        _ptr(seq_lens), B, hq, hkv, d, page_size, num_pages, max_seq_len, float(scale), window,
        num_splits, _ptr(out), _stream(stream)))
    return out


def decode_append(q, k_new, v_new, k_pool, v_pool, block_tables, seq_lens, max_seq_len, *,
                  page_size, scale=None, window=0, num_splits=0, workspace=None, out=None,
                  stream=None):
    """Decode step with its append fused into the decode launch (``pkv_decode_append``).

    Row ``b``'s new token (``k_new``/``v_new`` ``[B, Hkv, D]``) sits at position
    ``seq_lens[b] - 1``: it is written to its pool slot and attended in the same
    launch.  Returns bf16 ``[B, Hq, D]``.
    """
    _bf16(q, "q"); _bf16(k_new, "k_new"); _bf16(v_new, "v_new")
    _bf16(k_pool, "k_pool"); _bf16(v_pool, "v_pool")
    _i32(block_tables, "block_tables"); _i32(seq_lens, "seq_lens")
    B, hq, d = q.shape
    hkv, num_pages, d2 = _pool_shape(k_pool, page_size)
    if d2 != d or v_pool.shape != k_pool.shape or block_tables.shape[0] < B or seq_lens.numel() < B:
        raise ValueError("shape mismatch")
    if k_new.shape != (B, hkv, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new / v_new must be [B, Hkv, D]")
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out is None:
        out = torch.empty((B, hq, d), dtype=torch.bfloat16, device=q.device)
    need = decode_workspace_bytes(B, hq, d, hkv, page_size, max_seq_len, window, num_splits)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _dev(q, k_new, v_new, k_pool, v_pool, block_tables, seq_lens, out, workspace)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pkv_decode_append", lib().pkv_decode_append(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
        block_tables.shape[1], _ptr(seq_lens), B, hq, hkv, d, page_size, num_pages, max_seq_len,
        float(scale), window, num_splits, _ptr(workspace), wsb, _ptr(out), _stream(stream)))
    return out


def decode_split(q, k_pool, v_pool, block_tables, seq_lens, max_seq_len, *, page_size,
                 num_splits, pages_per_split, scale=None, window=0, out=None, stream=None):
    """Split-K partials (``pkv_decode_split``): returns ``(m, l, acc)`` float32."""
    _bf16(q, "q"); _bf16(k_pool, "k_pool"); _bf16(v_pool, "v_pool")
    _i32(block_tables, "block_tables"); _i32(seq_lens, "seq_lens")
    B, hq, d = q.shape
    hkv, num_pages, _ = _pool_shape(k_pool, page_size)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out is None:
        dev = q.device
        out = (torch.empty((B, hq, num_splits), dtype=torch.float32, device=dev),
               torch.empty((B, hq, num_splits), dtype=torch.float32, device=dev),
               torch.empty((B, hq, num_splits, d), dtype=torch.float32, device=dev))
    m, l, acc = out
    _dev(q, k_pool, v_pool, block_tables, seq_lens, m, l, acc)
    _check("pkv_decode_split", lib().pkv_decode_split(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), block_tables.shape[1],
        _ptr(seq_lens), B, hq, hkv, d, page_size, num_pages, max_seq_len, float(scale), window,
        num_splits, pages_per_split, _ptr(m), _ptr(l), _ptr(acc), _stream(stream)))
    return m, l, acc


def decode_combine(m, l, acc, out=None, stream=None):
    """Merge split-K partials (``pkv_decode_combine``); returns bf16 [B, Hq, D]."""
    B, hq, S, d = acc.shape
    if out is None:
        out = torch.empty((B, hq, d), dtype=torch.bfloat16, device=acc.device)
    _dev(m, l, acc, out)
    _check("pkv_decode_combine", lib().pkv_decode_combine(
        _ptr(m), _ptr(l), _ptr(acc), B, hq, d, S, _ptr(out), _stream(stream)))
    return out


def decode_stream_waves(num_seqs, num_q_heads, num_kv_heads, head_dim, page_size, max_seq_len,
                        window=0):
    """Number of persistent waves ``decode`` uses for stream-K (``pkv_decode_stream_waves``)."""
    n = ctypes.c_int32(0)
    _check("pkv_decode_stream_waves", lib().pkv_decode_stream_waves(
        num_seqs, num_q_heads, num_kv_heads, head_dim, page_size, max_seq_len, window,
        ctypes.byref(n)))
    return n.value


def decode_stream(q, k_pool, v_pool, block_tables, seq_lens, *, page_size, num_waves,
                  scale=None, window=0, workspace=None, out=None, stream=None):
    """Stream-K half of decode (``pkv_decode_stream``); returns ``(out, workspace)``.

    Rows whose (row, KV head) pieces were cut between waves are completed by
    ``decode_stream_merge`` with the same workspace.
    """
    _bf16(q, "q"); _bf16(k_pool, "k_pool"); _bf16(v_pool, "v_pool")
    _i32(block_tables, "block_tables"); _i32(seq_lens, "seq_lens")
    B, hq, d = q.shape
    hkv, num_pages, _ = _pool_shape(k_pool, page_size)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    need = int(lib().pkv_decode_stream_workspace_bytes(num_waves, hq, hkv, d))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, hq, d), dtype=torch.bfloat16, device=q.device)
    _dev(q, k_pool, v_pool, block_tables, seq_lens, out, workspace)
    _check("pkv_decode_stream", lib().pkv_decode_stream(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), block_tables.shape[1],
        _ptr(seq_lens), B, hq, hkv, d, page_size, num_pages, float(scale), window, num_waves,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
        _stream(stream)))
    return out, workspace


def decode_stream_merge(workspace, out, *, num_waves, num_kv_heads, stream=None):
    """Merge half of stream-K decode (``pkv_decode_stream_merge``), in place on ``out``."""
    B, hq, d = out.shape
    _dev(workspace, out)
    _check("pkv_decode_stream_merge", lib().pkv_decode_stream_merge(
        _ptr(workspace), workspace.numel() * workspace.element_size(), num_waves, hq,
        num_kv_heads, d, _ptr(out), _stream(stream)))
    return out


def prefill_varlen(q, k_pool, v_pool, block_tables, cu_seq_lens_q, cu_seq_lens_k,
                   max_seqlen_q, max_seqlen_k, *, page_size, scale=None, window=0, out=None,
                   stream=None):
    """Varlen causal prefill over the paged pool (``pkv_prefill_varlen``); returns bf16 [Tq, Hq, D]."""
    _bf16(q, "q"); _bf16(k_pool, "k_pool"); _bf16(v_pool, "v_pool")
    _i32(block_tables, "block_tables"); _i32(cu_seq_lens_q, "cu_q"); _i32(cu_seq_lens_k, "cu_k")
    Tq, hq, d = q.shape
    hkv, num_pages, _ = _pool_shape(k_pool, page_size)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out is None:
        out = torch.empty((Tq, hq, d), dtype=torch.bfloat16, device=q.device)
    _dev(q, k_pool, v_pool, block_tables, cu_seq_lens_q, cu_seq_lens_k, out)
    n = cu_seq_lens_q.numel() - 1
    _check("pkv_prefill_varlen", lib().pkv_prefill_varlen(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), block_tables.shape[1],
        _ptr(cu_seq_lens_q), _ptr(cu_seq_lens_k), n, Tq, max_seqlen_q, max_seqlen_k, hq, hkv, d,
        page_size, num_pages, float(scale), window, _ptr(out), _stream(stream)))
    return out


def prefill_split_workspace_bytes(total_q, num_q_heads, head_dim, num_splits):
    """Workspace bytes of ``pkv_prefill_varlen_split`` (0 when ``num_splits`` <= 1)."""
    return int(lib().pkv_prefill_split_workspace_bytes(total_q, num_q_heads, head_dim, num_splits))


def prefill_varlen_split(q, k_pool, v_pool, block_tables, cu_seq_lens_q, cu_seq_lens_k,
                         max_seqlen_q, max_seqlen_k, *, page_size, num_splits, scale=None, window=0,
                         out=None, workspace=None, stream=None):
    """``pkv_prefill_varlen_split``: varlen prefill with the key tiles of long work cut
    into at most ``num_splits`` runs, the cut rows merged by a second launch; returns
    bf16 [Tq, Hq, D]."""
    _bf16(q, "q"); _bf16(k_pool, "k_pool"); _bf16(v_pool, "v_pool")
    _i32(block_tables, "block_tables"); _i32(cu_seq_lens_q, "cu_q"); _i32(cu_seq_lens_k, "cu_k")
    Tq, hq, d = q.shape
    hkv, num_pages, _ = _pool_shape(k_pool, page_size)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out is None:
        out = torch.empty((Tq, hq, d), dtype=torch.bfloat16, device=q.device)
    nbytes = prefill_split_workspace_bytes(Tq, hq, d, num_splits)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _dev(q, k_pool, v_pool, block_tables, cu_seq_lens_q, cu_seq_lens_k, out)
    n = cu_seq_lens_q.numel() - 1
    ws = _ptr(workspace) if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("pkv_prefill_varlen_split", lib().pkv_prefill_varlen_split(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), block_tables.shape[1],
        _ptr(cu_seq_lens_q), _ptr(cu_seq_lens_k), n, Tq, max_seqlen_q, max_seqlen_k, hq, hkv, d,
        page_size, num_pages, float(scale), window, num_splits, ws, wsb, _ptr(out),
        _stream(stream)))
    return out


# ---------------------------------------------------------------------------
# step graphs
# ---------------------------------------------------------------------------
class StepGraph:
    """A captured sequence of pkv launches (``pkv_graph_end``), replayed by ``launch``.

    The tensors the launches were captured with must stay alive and keep
    their storage for as long as the graph is replayed.
    """

    def __init__(self, handle: ctypes.c_void_p, keep=()):
        self._h = handle
        self._keep = tuple(keep)

    def launch(self, stream=None):
        if not self._h:
            raise ValueError("graph was destroyed")
        _check("pkv_graph_launch", lib().pkv_graph_launch(self._h, _stream(stream)))

    def nodes(self):
        """``(kernel_nodes, other_nodes)`` of the captured graph (``pkv_graph_nodes``)."""
        k, o = ctypes.c_int32(0), ctypes.c_int32(0)
        _check("pkv_graph_nodes", lib().pkv_graph_nodes(self._h, ctypes.byref(k), ctypes.byref(o)))
        return k.value, o.value

    def destroy(self):
        if self._h:
            h, self._h = self._h, None
            _check("pkv_graph_destroy", lib().pkv_graph_destroy(h))

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def capture_graph(fn, stream, keep=()):
    """Capture the pkv calls ``fn()`` enqueues into a ``StepGraph`` (``pkv_graph_begin/end``).

    ``fn`` runs once with ``stream`` (a non-default ``torch.cuda.Stream``)
    current; it must only enqueue pkv calls on preallocated tensors (no
    allocation, copy or host read).  ``keep`` holds tensors the graph uses.
    """
    if stream is None or stream.cuda_stream == 0:
        raise ValueError("capture needs a non-default stream")
    hs = _stream(stream)
    with torch.cuda.stream(stream):
        _check("pkv_graph_begin", lib().pkv_graph_begin(hs))
        h = ctypes.c_void_p(None)
        try:
            fn()
        except BaseException:
            lib().pkv_graph_end(hs, ctypes.byref(h))
            if h:
                lib().pkv_graph_destroy(h)
            raise
        _check("pkv_graph_end", lib().pkv_graph_end(hs, ctypes.byref(h)))
    return StepGraph(h, keep)
