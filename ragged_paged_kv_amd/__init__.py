"""Python binding of libcbattn.so: ragged paged attention and the paged KV-cache write on MI355X.

Each function here has the name of the C entry point it calls (see include/cbattn.h) and does
argument marshalling only: it checks dtypes, devices and contiguity of torch tensors, passes
their device pointers and the current HIP stream, and turns a non-zero status into CBError.
Every step of the computation runs in the library's HIP kernels. There is no fallback: if the
library is missing or fails to load, importing this package raises.

    import ragged_paged_kv_amd as cb
    cb.cb_slot_mapping(cu, kv_lens, tables, slots, block_size)
    cb.cb_cache_write(k, v, slots, k_cache, v_cache)
    ws = cb.alloc_workspace(...)
    cb.cb_paged_attention(q, cu, kv_lens, tables, k_cache, v_cache, out, scale, ...)
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from ._build import LIB_PATH

__all__ = [
    "CBError", "LIB_PATH", "lib", "cb_status_string", "cb_last_error", "cb_slot_mapping",
    "cb_cache_write", "cb_paged_attention_workspace_size", "cb_paged_attention_split_tokens",
    "cb_paged_attention", "cb_paged_attention_write", "cb_paged_attention_write_noalloc",
    "CB_NOALLOC_SCRATCH_BYTES", "cb_split_kv_reduce", "cb_validate_batch",
    "cb_time_next_kernel", "cb_stream_read", "alloc_workspace", "EXPORTED_SYMBOLS", "CB_KERNEL_DECODE", "CB_KERNEL_PREFILL",
    "cb_copy_blocks", "BlockManager", "CB_ERR_OUT_OF_BLOCKS", "StepGraphs",
    "cb_swap_out_blocks", "cb_swap_in_blocks", "cb_carry_over", "AsyncSteps",
]

EXPORTED_SYMBOLS = (
    "cb_status_string", "cb_last_error", "cb_slot_mapping", "cb_cache_write",
    "cb_paged_attention_workspace_size", "cb_paged_attention_split_tokens", "cb_paged_attention",
    "cb_paged_attention_write", "cb_paged_attention_write_noalloc", "cb_split_kv_reduce",
    "cb_validate_batch", "cb_time_next_kernel", "cb_stream_read",
    # include/cbblocks.h
    "cb_bm_create", "cb_bm_destroy", "cb_bm_add_sequence", "cb_bm_append_tokens",
    "cb_bm_append_batch", "cb_bm_fork",
    "cb_bm_free_sequence", "cb_bm_build_batch", "cb_bm_take_copies", "cb_bm_sequence_info",
    "cb_bm_block_table", "cb_bm_stats", "cb_bm_ref_counts", "cb_copy_blocks",
    "cb_bm_set_swap_slots", "cb_bm_swap_out", "cb_bm_swap_in", "cb_bm_swap_stats",
    "cb_swap_out_blocks", "cb_swap_in_blocks", "cb_bm_append_placeholders", "cb_bm_confirm_tokens",
    "cb_bm_confirm_batch",
    # include/cbgraphs.h
    "cb_graphs_create", "cb_graphs_destroy", "cb_graphs_run", "cb_graphs_stats",
    # include/cbasync.h
    "cb_carry_over", "cb_async_create", "cb_async_destroy", "cb_async_slot", "cb_async_begin",
    "cb_async_attention", "cb_async_end", "cb_async_wait",
)


class CBError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {cb_status_string(status)} ({status}): {detail}")
        self.status = status


def _load():
    # torch ships its own HIP runtime under the same soname (libamdhip64.so.7). Loading torch
    # first makes the library's HIP dependency bind to that runtime, so torch's allocations,
    # streams and our kernels share one device context. Loaded the other way round, the process
    # would hold two HIP runtimes and the second would not see the GPU.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built. Build it with `python ragged_paged_kv_amd/_build.py` "
            "(needs ROCm hipcc).")
    return ctypes.CDLL(LIB_PATH)


lib = _load()

_i32, _i64, _sz, _p, _f = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
_sig = {
    "cb_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "cb_last_error": (ctypes.c_char_p, []),
    "cb_slot_mapping": (ctypes.c_int, [_p, _p, _p, _i32, _i32, _i32, _i32, _p, _p]),
    "cb_cache_write": (ctypes.c_int, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i64, _p]),
    "cb_paged_attention_workspace_size": (_sz, [_i32] * 9),
    "cb_paged_attention_split_tokens": (_i32, [_i32] * 6),
    "cb_paged_attention": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _f, _i32, _i32, _i32, _i32,
                                          _i32, _i32, _i32, _i64, _i32, _i32, _i32, _p, _sz, _p]),
    "cb_paged_attention_write": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _f, _i32, _i32,
                                                _i32, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _i32,
                                                _p, _sz, _p]),
    "cb_paged_attention_write_noalloc": (ctypes.c_int, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _f,
                                                        _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                        _i64, _i32, _i32, _i32, _p]),
    "cb_split_kv_reduce": (ctypes.c_int, [_p, _p, _p, _p, _i32, _i32, _i32, _i32, _p]),
    "cb_validate_batch": (ctypes.c_int, [_p, _p, _p, _p, _i32, _i32, _i32, _i32, _i64, _i32, _i32]),
    "cb_time_next_kernel": (ctypes.c_int, [_i32, _p, _p]),
    "cb_stream_read": (ctypes.c_int, [_p, _sz, _p, _i32, _p]),
    "cb_bm_create": (ctypes.c_int, [_i64, _i32, _p]),
    "cb_bm_destroy": (None, [_p]),
    "cb_bm_add_sequence": (ctypes.c_int, [_p, _i64, _p, _i32, _p]),
    "cb_bm_append_tokens": (ctypes.c_int, [_p, _i64, _p, _i32]),
    "cb_bm_append_batch": (ctypes.c_int, [_p, _p, _p, _p, _i32, _p]),
    "cb_bm_fork": (ctypes.c_int, [_p, _i64, _i64]),
    "cb_bm_free_sequence": (ctypes.c_int, [_p, _i64]),
    "cb_bm_build_batch": (ctypes.c_int, [_p, _p, _p, _i32, _i32, _i32, _p, _p, _p, _p, _p]),
    "cb_bm_take_copies": (ctypes.c_int, [_p, _p, _p, _i32, _p]),
    "cb_bm_sequence_info": (ctypes.c_int, [_p, _i64, _p, _p, _p]),
    "cb_bm_block_table": (ctypes.c_int, [_p, _i64, _p, _i32]),
    "cb_bm_stats": (ctypes.c_int, [_p, _p, _p, _p, _p]),
    "cb_bm_ref_counts": (ctypes.c_int, [_p, _p, _i64]),
    "cb_copy_blocks": (ctypes.c_int, [_p, _p, _p, _p, _i32, _i64, _i64, _i32, _i64, _p]),
    "cb_bm_set_swap_slots": (ctypes.c_int, [_p, _i64]),
    "cb_bm_append_placeholders": (ctypes.c_int, [_p, _i64, _i32]),
    "cb_bm_confirm_tokens": (ctypes.c_int, [_p, _i64, _p, _i32]),
    "cb_bm_confirm_batch": (ctypes.c_int, [_p, _p, _p, _p, _i32, _p]),
    "cb_bm_swap_out": (ctypes.c_int, [_p, _i64, _p, _p, _i32, _p]),
    "cb_bm_swap_in": (ctypes.c_int, [_p, _i64, _p, _p, _i32, _p]),
    "cb_bm_swap_stats": (ctypes.c_int, [_p, _p, _p, _p]),
    "cb_swap_out_blocks": (ctypes.c_int, [_p, _p, _p, _p, _i32, _p, _i64, _i64, _i64, _i32, _i64, _p]),
    "cb_swap_in_blocks": (ctypes.c_int, [_p, _p, _p, _i32, _p, _p, _i64, _i64, _i64, _i32, _i64, _p]),
    "cb_graphs_create": (ctypes.c_int, [_p, _p]),
    "cb_graphs_destroy": (None, [_p]),
    "cb_graphs_run": (ctypes.c_int, [_p, _p, _p, _p, _i32, _p, _p]),
    "cb_graphs_stats": (ctypes.c_int, [_p, _p, _p, _p, _p]),
    "cb_carry_over": (ctypes.c_int, [_p, _p, _i32, _p, _i32, _p]),
    "cb_async_create": (ctypes.c_int, [_p, _p]),
    "cb_async_destroy": (None, [_p]),
    "cb_async_slot": (ctypes.c_int, [_p, _p]),
    "cb_async_begin": (ctypes.c_int, [_p, _p, _p, _p, _i32, _i32, _p]),
    "cb_async_attention": (ctypes.c_int, [_p]),
    "cb_async_end": (ctypes.c_int, [_p, _i32]),
    "cb_async_wait": (ctypes.c_int, [_p, _i32]),
}

CB_KERNEL_DECODE = 1
CB_KERNEL_PREFILL = 2
CB_ERR_OUT_OF_BLOCKS = -5
for _name, (_res, _args) in _sig.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def cb_status_string(status: int) -> str:
    return lib.cb_status_string(int(status)).decode()


def cb_last_error() -> str:
    return lib.cb_last_error().decode()


def _check(status: int, where: str):
    if status != 0:
        raise CBError(status, where, cb_last_error())


# ---------------------------------------------------------------------------------------------
# torch marshalling


def _torch():
    import torch
    return torch


def _dev(t, name, dtype, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)
    if hasattr(stream, "cuda_stream"):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def cb_slot_mapping(cu_seqlens_q, kv_lens, block_tables, slot_mapping, block_size: int,
                    stream=None):
    torch = _torch()
    S = kv_lens.shape[0]
    T = slot_mapping.shape[0]
    _check(lib.cb_slot_mapping(_dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1),
                               _dev(kv_lens, "kv_lens", torch.int32, 1),
                               _dev(block_tables, "block_tables", torch.int32, 2), S, T,
                               block_tables.shape[1], int(block_size),
                               _dev(slot_mapping, "slot_mapping", torch.int32, 1), _stream(stream)),
           "cb_slot_mapping")


def cb_cache_write(k, v, slot_mapping, k_cache, v_cache, stream=None):
    torch = _torch()
    T, Hkv, D = k.shape
    NB, bs = k_cache.shape[0], k_cache.shape[1]
    if tuple(v.shape) != (T, Hkv, D) or tuple(k_cache.shape) != (NB, bs, Hkv, D) \
            or tuple(v_cache.shape) != tuple(k_cache.shape) or slot_mapping.shape[0] != T:
        raise ValueError("cb_cache_write: inconsistent shapes")
    _check(lib.cb_cache_write(_dev(k, "k", torch.bfloat16, 3), _dev(v, "v", torch.bfloat16, 3),
                              _dev(slot_mapping, "slot_mapping", torch.int32, 1),
                              _dev(k_cache, "k_cache", torch.bfloat16, 4),
                              _dev(v_cache, "v_cache", torch.bfloat16, 4), T, Hkv, D, bs, NB,
                              _stream(stream)),
           "cb_cache_write")


def cb_paged_attention_workspace_size(num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim,
                                      block_size, max_q_len, max_kv_len, kv_split_tokens=0) -> int:
    return int(lib.cb_paged_attention_workspace_size(num_seqs, num_tokens, num_q_heads,
                                                     num_kv_heads, head_dim, block_size,
                                                     max_q_len, max_kv_len, kv_split_tokens))


def cb_paged_attention_split_tokens(num_seqs, num_q_heads, num_kv_heads, max_q_len, max_kv_len,
                                    kv_split_tokens=0) -> int:
    return int(lib.cb_paged_attention_split_tokens(num_seqs, num_q_heads, num_kv_heads, max_q_len,
                                                   max_kv_len, kv_split_tokens))


def alloc_workspace(num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, block_size,
                    max_q_len, max_kv_len, kv_split_tokens=0, device="cuda"):
    """A uint8 device tensor of the size cb_paged_attention needs (torch allocations are
    at least 256-byte aligned)."""
    n = cb_paged_attention_workspace_size(num_seqs, num_tokens, num_q_heads, num_kv_heads,
                                          head_dim, block_size, max_q_len, max_kv_len,
                                          kv_split_tokens)
    return _torch().empty(max(n, 256), dtype=_torch().uint8, device=device)


def cb_paged_attention(q_packed, cu_seqlens_q, kv_lens, block_tables, k_cache, v_cache, out,
                       scale: float, max_q_len: int, max_kv_len: int, workspace,
                       kv_split_tokens: int = 0, stream=None):
    torch = _torch()
    T, Hq, D = q_packed.shape
    NB, bs, Hkv, _ = k_cache.shape
    S = kv_lens.shape[0]
    if tuple(out.shape) != (T, Hq, D) or tuple(v_cache.shape) != tuple(k_cache.shape) \
            or k_cache.shape[3] != D or cu_seqlens_q.shape[0] != S + 1 \
            or block_tables.shape[0] != S:
        raise ValueError("cb_paged_attention: inconsistent shapes")
    _check(lib.cb_paged_attention(
        _dev(q_packed, "q_packed", torch.bfloat16, 3),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1), _dev(kv_lens, "kv_lens", torch.int32, 1),
        _dev(block_tables, "block_tables", torch.int32, 2),
        _dev(k_cache, "k_cache", torch.bfloat16, 4), _dev(v_cache, "v_cache", torch.bfloat16, 4),
        _dev(out, "out", torch.bfloat16, 3), float(scale), S, T, Hq, Hkv, D, bs,
        block_tables.shape[1], NB, int(max_q_len), int(max_kv_len), int(kv_split_tokens),
        _dev(workspace, "workspace", torch.uint8, 1), workspace.numel(), _stream(stream)),
        "cb_paged_attention")


def cb_paged_attention_write(q_packed, k_new, v_new, cu_seqlens_q, kv_lens, block_tables, k_cache,
                             v_cache, out, scale: float, max_q_len: int, max_kv_len: int, workspace,
                             kv_split_tokens: int = 0, stream=None):
    """cb_slot_mapping + cb_cache_write + cb_paged_attention in one call (see include/cbattn.h)."""
    torch = _torch()
    T, Hq, D = q_packed.shape
    NB, bs, Hkv, _ = k_cache.shape
    S = kv_lens.shape[0]
    if tuple(out.shape) != (T, Hq, D) or tuple(v_cache.shape) != tuple(k_cache.shape) \
            or k_cache.shape[3] != D or cu_seqlens_q.shape[0] != S + 1 \
            or block_tables.shape[0] != S or tuple(k_new.shape) != (T, Hkv, D) \
            or tuple(v_new.shape) != (T, Hkv, D):
        raise ValueError("cb_paged_attention_write: inconsistent shapes")
    _check(lib.cb_paged_attention_write(
        _dev(q_packed, "q_packed", torch.bfloat16, 3), _dev(k_new, "k_new", torch.bfloat16, 3),
        _dev(v_new, "v_new", torch.bfloat16, 3),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1), _dev(kv_lens, "kv_lens", torch.int32, 1),
        _dev(block_tables, "block_tables", torch.int32, 2),
        _dev(k_cache, "k_cache", torch.bfloat16, 4), _dev(v_cache, "v_cache", torch.bfloat16, 4),
        _dev(out, "out", torch.bfloat16, 3), float(scale), S, T, Hq, Hkv, D, bs,
        block_tables.shape[1], NB, int(max_q_len), int(max_kv_len), int(kv_split_tokens),
        _dev(workspace, "workspace", torch.uint8, 1), workspace.numel(), _stream(stream)),
        "cb_paged_attention_write")


# Bytes of the scratch cb_paged_attention_write_noalloc holds per device (include/cbattn.h).
CB_NOALLOC_SCRATCH_BYTES = 128 << 20


def cb_paged_attention_write_noalloc(q_packed, k_new, v_new, cu_seqlens_q, kv_lens, block_tables,
                                     k_cache, v_cache, out, scale: float, max_q_len: int,
                                     max_kv_len: int, kv_split_tokens: int = 0, stream=None):
    """cb_paged_attention_write with the library's own scratch instead of a workspace (no device
    allocation in the call; see include/cbattn.h)."""
    torch = _torch()
    T, Hq, D = q_packed.shape
    NB, bs, Hkv, _ = k_cache.shape
    S = kv_lens.shape[0]
    if tuple(out.shape) != (T, Hq, D) or tuple(v_cache.shape) != tuple(k_cache.shape) \
            or k_cache.shape[3] != D or cu_seqlens_q.shape[0] != S + 1 \
            or block_tables.shape[0] != S or tuple(k_new.shape) != (T, Hkv, D) \
            or tuple(v_new.shape) != (T, Hkv, D):
        raise ValueError("cb_paged_attention_write_noalloc: inconsistent shapes")
    _check(lib.cb_paged_attention_write_noalloc(
        _dev(q_packed, "q_packed", torch.bfloat16, 3), _dev(k_new, "k_new", torch.bfloat16, 3),
        _dev(v_new, "v_new", torch.bfloat16, 3),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1), _dev(kv_lens, "kv_lens", torch.int32, 1),
        _dev(block_tables, "block_tables", torch.int32, 2),
        _dev(k_cache, "k_cache", torch.bfloat16, 4), _dev(v_cache, "v_cache", torch.bfloat16, 4),
        _dev(out, "out", torch.bfloat16, 3), float(scale), S, T, Hq, Hkv, D, bs,
        block_tables.shape[1], NB, int(max_q_len), int(max_kv_len), int(kv_split_tokens),
        _stream(stream)),
        "cb_paged_attention_write_noalloc")


def cb_split_kv_reduce(o_part, lse_part, num_splits, out, stream=None):
    torch = _torch()
    T, Hq, ms, D = o_part.shape
    if tuple(lse_part.shape) != (T, Hq, ms) or tuple(out.shape) != (T, Hq, D) \
            or num_splits.shape[0] != T:
        raise ValueError("cb_split_kv_reduce: inconsistent shapes")
    _check(lib.cb_split_kv_reduce(_dev(o_part, "o_part", torch.float32, 4),
                                  _dev(lse_part, "lse_part", torch.float32, 3),
                                  _dev(num_splits, "num_splits", torch.int32, 1),
                                  _dev(out, "out", torch.bfloat16, 3), T, Hq, D, ms,
                                  _stream(stream)),
           "cb_split_kv_reduce")


def cb_stream_read(buf, sink, stream=None):
    """Read every byte of the device tensor ``buf`` once (measurement aid: the streaming-read
    ceiling); ``sink`` is an int32 device tensor of at least 256 elements."""
    torch = _torch()
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("cb_stream_read: buf must be a contiguous device tensor")
    _check(lib.cb_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                              _dev(sink, "sink", torch.int32, 1), sink.numel(), _stream(stream)),
           "cb_stream_read")


def _event_handle(ev, stream):
    """Raw hipEvent_t of a torch.cuda.Event (torch creates the event on its first record)."""
    if ev.cuda_event == 0:
        ev.record(stream)
    return ctypes.c_void_p(ev.cuda_event)


def cb_time_next_kernel(which: int, start=None, stop=None, stream=None):
    """Have the next cb_paged_attention call of this thread record torch.cuda.Events `start` and
    `stop` (enable_timing=True) around kernel `which` (CB_KERNEL_DECODE or CB_KERNEL_PREFILL);
    which=0 clears a pending request."""
    if which == 0:
        _check(lib.cb_time_next_kernel(0, None, None), "cb_time_next_kernel")
        return
    torch = _torch()
    st = stream if stream is not None else torch.cuda.current_stream()
    _check(lib.cb_time_next_kernel(int(which), _event_handle(start, st), _event_handle(stop, st)),
           "cb_time_next_kernel")


def _host_i32(a, name):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(a), dtype=np.int32)
    return arr, ctypes.c_void_p(arr.ctypes.data)


def cb_validate_batch(cu_seqlens_q, kv_lens, block_tables, slot_mapping, block_size: int,
                      num_blocks: int, max_q_len: int, max_kv_len: int, raise_on_error=True):
    """Host-only precondition check on host arrays (numpy or CPU tensors). Returns the status
    (0 when valid); raises CBError instead when raise_on_error."""
    cu, pcu = _host_i32(cu_seqlens_q, "cu_seqlens_q")
    kv, pkv = _host_i32(kv_lens, "kv_lens")
    bt, pbt = _host_i32(block_tables, "block_tables")
    sl, psl = _host_i32(slot_mapping, "slot_mapping")
    S = kv.shape[0]
    T = int(cu[-1]) if sl is None else sl.shape[0]
    mb = bt.shape[1] if bt.ndim == 2 else 0
    st = lib.cb_validate_batch(pcu, pkv, pbt, psl, S, T, mb, int(block_size), int(num_blocks),
                               int(max_q_len), int(max_kv_len))
    if raise_on_error:
        _check(st, "cb_validate_batch")
    return int(st)


# ---------------------------------------------------------------------------------------------
# block manager (include/cbblocks.h): host arrays are numpy int32 / int64


def _ptr(a):
    # the raw address: numpy's data_as goes through ctypes.cast, which is slow here (~70 us)
    return ctypes.c_void_p(a.ctypes.data)


class BlockManager:
    """Owner of one cb_block_manager handle. Each method calls the C function of the same name
    (cb_bm_<method>) and raises CBError on a non-zero status."""

    def __init__(self, num_blocks: int, block_size: int):
        h = ctypes.c_void_p()
        _check(lib.cb_bm_create(int(num_blocks), int(block_size), ctypes.byref(h)), "cb_bm_create")
        self._h = h
        self._destroy = lib.cb_bm_destroy  # kept: module globals may be gone at interpreter exit
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self._destroy(self._h)
            self._h = None

    __del__ = close

    def add_sequence(self, seq_id: int, tokens) -> int:
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        n = ctypes.c_int32()
        _check(lib.cb_bm_add_sequence(self._h, int(seq_id), _ptr(t), t.size, ctypes.byref(n)),
               "cb_bm_add_sequence")
        return n.value

    def append_tokens(self, seq_id: int, tokens):
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        _check(lib.cb_bm_append_tokens(self._h, int(seq_id), _ptr(t), t.size), "cb_bm_append_tokens")

    def append_batch(self, seq_ids, counts, tokens) -> int:
        """Appends counts[i] tokens (packed in order in `tokens`; None: placeholders) to
        seq_ids[i] until one is refused; returns how many sequences were appended (all of them,
        or raises CBError with the count in .num_done)."""
        return self._batch(lib.cb_bm_append_batch, "cb_bm_append_batch", seq_ids, counts, tokens)

    def confirm_batch(self, seq_ids, counts, tokens) -> int:
        """Confirms the next counts[i] tokens of seq_ids[i] (values packed in `tokens`)."""
        return self._batch(lib.cb_bm_confirm_batch, "cb_bm_confirm_batch", seq_ids, counts, tokens)

    def _batch(self, fn, name, seq_ids, counts, tokens):
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        c = np.ascontiguousarray(counts, dtype=np.int32)
        t = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
        done = ctypes.c_int32()
        st = fn(self._h, _ptr(ids), _ptr(c), None if t is None else _ptr(t), ids.size, ctypes.byref(done))
        if st != 0:
            e = CBError(st, name, cb_last_error())
            e.num_done = done.value
            raise e
        return done.value

    def append_placeholders(self, seq_id: int, num_tokens: int):
        _check(lib.cb_bm_append_placeholders(self._h, int(seq_id), int(num_tokens)),
               "cb_bm_append_placeholders")

    def confirm_tokens(self, seq_id: int, tokens):
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        _check(lib.cb_bm_confirm_tokens(self._h, int(seq_id), _ptr(t), t.size), "cb_bm_confirm_tokens")

    def fork(self, parent: int, child: int):
        _check(lib.cb_bm_fork(self._h, int(parent), int(child)), "cb_bm_fork")

    def free_sequence(self, seq_id: int):
        _check(lib.cb_bm_free_sequence(self._h, int(seq_id)), "cb_bm_free_sequence")

    def build_batch(self, seq_ids, q_lens, max_blocks_per_seq: int, token_capacity: int | None = None,
                    out=None):
        """Returns (cu_seqlens_q, kv_lens, block_tables, slot_mapping, token_ids), int32 numpy.
        Without `out`, fresh arrays whose table entries past a sequence's table hold -1. With
        out = (cu, kv_lens, tables, slots, token_ids), caller-owned int32 arrays (a serving loop
        keeps them across steps) are filled; table entries past a sequence's table keep their
        contents, and the returned arrays are views of them."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        q = np.ascontiguousarray(q_lens, dtype=np.int32)
        S = ids.size
        if out is None:
            cap = int(q.sum()) if token_capacity is None else int(token_capacity)
            cu = np.zeros(S + 1, np.int32)
            kv = np.zeros(max(S, 1), np.int32)
            bt = np.full((max(S, 1), int(max_blocks_per_seq)), -1, np.int32)
            sl = np.zeros(max(cap, 1), np.int32)
            tk = np.zeros(max(cap, 1), np.int32)
        else:
            cu, kv, bt, sl, tk = out
            for a in out:
                if a.dtype != np.int32 or not a.flags.c_contiguous:
                    raise ValueError("build_batch: out arrays must be C-contiguous int32")
            if cu.size < S + 1 or kv.size < S or bt.shape[0] < S or bt.shape[1] != max_blocks_per_seq:
                raise ValueError("build_batch: out arrays are too small")
            cap = min(sl.size, tk.size)
        _check(lib.cb_bm_build_batch(self._h, _ptr(ids), _ptr(q), S, int(max_blocks_per_seq), cap,
                                     _ptr(cu), _ptr(kv), _ptr(bt), _ptr(sl), _ptr(tk)),
               "cb_bm_build_batch")
        T = int(cu[S])
        return cu[:S + 1], kv[:S], bt[:S], sl[:T], tk[:T]

    def take_copies(self, capacity: int | None = None):
        """Closes the step; returns (src, dst) int32 arrays of the pending copies."""
        n = ctypes.c_int32()
        if capacity is None:
            lib.cb_bm_take_copies(self._h, None, None, 0, ctypes.byref(n))  # count only
            capacity = n.value
        src = np.zeros(max(capacity, 1), np.int32)
        dst = np.zeros(max(capacity, 1), np.int32)
        _check(lib.cb_bm_take_copies(self._h, _ptr(src), _ptr(dst), int(capacity), ctypes.byref(n)),
               "cb_bm_take_copies")
        return src[:n.value], dst[:n.value]

    def sequence_info(self, seq_id: int):
        n, c, b = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
        _check(lib.cb_bm_sequence_info(self._h, int(seq_id), ctypes.byref(n), ctypes.byref(c),
                                       ctypes.byref(b)), "cb_bm_sequence_info")
        return n.value, c.value, b.value

    def block_table(self, seq_id: int):
        nb = self.sequence_info(seq_id)[2]
        out = np.zeros(max(nb, 1), np.int32)
        _check(lib.cb_bm_block_table(self._h, int(seq_id), _ptr(out), out.size), "cb_bm_block_table")
        return out[:nb]

    def stats(self):
        """(never-used free blocks, cached blocks, held blocks, live sequences)."""
        v = [ctypes.c_int64() for _ in range(4)]
        _check(lib.cb_bm_stats(self._h, *[ctypes.byref(x) for x in v]), "cb_bm_stats")
        return tuple(x.value for x in v)

    def set_swap_slots(self, num_slots: int):
        _check(lib.cb_bm_set_swap_slots(self._h, int(num_slots)), "cb_bm_set_swap_slots")

    def _swap(self, fn, name, seq_id):
        nb = self.sequence_info(seq_id)[2] if fn is lib.cb_bm_swap_out else None
        cap = max(nb if nb is not None else self._swapped_len(seq_id), 1)
        a, b = np.zeros(cap, np.int32), np.zeros(cap, np.int32)
        n = ctypes.c_int32()
        _check(fn(self._h, int(seq_id), _ptr(a), _ptr(b), cap, ctypes.byref(n)), name)
        return a[:n.value], b[:n.value]

    def _swapped_len(self, seq_id):
        n, _, _ = self.sequence_info(seq_id)
        return -(-n // self.block_size)

    def swap_out(self, seq_id: int):
        """(blocks, slots): copy block blocks[i] to pool slot slots[i]."""
        return self._swap(lib.cb_bm_swap_out, "cb_bm_swap_out", seq_id)

    def swap_in(self, seq_id: int):
        """(slots, blocks): copy pool slot slots[i] to block blocks[i]."""
        return self._swap(lib.cb_bm_swap_in, "cb_bm_swap_in", seq_id)

    def swap_stats(self):
        """(free, used, held) swap slots."""
        v = [ctypes.c_int64() for _ in range(3)]
        _check(lib.cb_bm_swap_stats(self._h, *[ctypes.byref(x) for x in v]), "cb_bm_swap_stats")
        return tuple(x.value for x in v)

    def ref_counts(self):
        out = np.zeros(self.num_blocks, np.int32)
        _check(lib.cb_bm_ref_counts(self._h, _ptr(out), out.size), "cb_bm_ref_counts")
        return out


def cb_copy_blocks(k_cache, v_cache, src_blocks, dst_blocks, num_layers: int = 1, stream=None):
    """Copy blocks src_blocks[i] -> dst_blocks[i] (int32 device tensors) of K and V. The caches are
    [NB, bs, Hkv, D] bf16, or [L, NB, bs, Hkv, D] with num_layers = L."""
    torch = _torch()
    if tuple(v_cache.shape) != tuple(k_cache.shape) or src_blocks.shape != dst_blocks.shape:
        raise ValueError("cb_copy_blocks: inconsistent shapes")
    nd = 5 if num_layers > 1 else 4
    if k_cache.dim() != nd or (nd == 5 and k_cache.shape[0] != num_layers):
        raise ValueError("cb_copy_blocks: caches must be [NB, bs, Hkv, D] or [L, NB, bs, Hkv, D]")
    NB = k_cache.shape[-4]
    block_bytes = int(np.prod(k_cache.shape[-3:])) * k_cache.element_size()
    layer_stride = NB * block_bytes
    _check(lib.cb_copy_blocks(_dev(k_cache, "k_cache", torch.bfloat16, nd),
                              _dev(v_cache, "v_cache", torch.bfloat16, nd),
                              _dev(src_blocks, "src_blocks", torch.int32, 1),
                              _dev(dst_blocks, "dst_blocks", torch.int32, 1), src_blocks.numel(),
                              block_bytes, NB, int(num_layers), layer_stride, _stream(stream)),
           "cb_copy_blocks")


def _swap_shapes(k_cache, v_cache, pool, blocks, slots, num_layers):
    if tuple(v_cache.shape) != tuple(k_cache.shape) or blocks.shape != slots.shape:
        raise ValueError("swap: inconsistent shapes")
    nd = 5 if num_layers > 1 else 4
    if k_cache.dim() != nd or (nd == 5 and k_cache.shape[0] != num_layers):
        raise ValueError("swap: caches must be [NB, bs, Hkv, D] or [L, NB, bs, Hkv, D]")
    NB = k_cache.shape[-4]
    block_bytes = int(np.prod(k_cache.shape[-3:])) * k_cache.element_size()
    if pool.device.type != "cpu" or not pool.is_pinned() or not pool.is_contiguous():
        raise ValueError("swap: the pool must be a contiguous pinned host tensor")
    if pool.dim() != 6 or tuple(pool.shape[1:]) != (2, num_layers) + tuple(k_cache.shape[-3:]) \
            or pool.dtype != k_cache.dtype:
        raise ValueError("swap: pool must be [num_slots, 2, L, bs, Hkv, D] of the caches' dtype")
    return NB, block_bytes, NB * block_bytes


def cb_swap_out_blocks(k_cache, v_cache, blocks, slots, pool, num_layers: int = 1, stream=None):
    """Gather blocks[i] (K and V, every layer) into pool slot slots[i]; pool is a pinned host
    tensor [num_slots, 2, L, bs, Hkv, D]; blocks, slots int32 device tensors."""
    torch = _torch()
    NB, bb, stride = _swap_shapes(k_cache, v_cache, pool, blocks, slots, num_layers)
    nd = 5 if num_layers > 1 else 4
    _check(lib.cb_swap_out_blocks(_dev(k_cache, "k_cache", torch.bfloat16, nd),
                                  _dev(v_cache, "v_cache", torch.bfloat16, nd),
                                  _dev(blocks, "blocks", torch.int32, 1), _dev(slots, "slots", torch.int32, 1),
                                  blocks.numel(), ctypes.c_void_p(pool.data_ptr()), pool.shape[0], bb, NB,
                                  int(num_layers), stride, _stream(stream)),
           "cb_swap_out_blocks")


def cb_swap_in_blocks(pool, slots, blocks, k_cache, v_cache, num_layers: int = 1, stream=None):
    """Scatter pool slot slots[i] into block blocks[i] (K and V, every layer)."""
    torch = _torch()
    NB, bb, stride = _swap_shapes(k_cache, v_cache, pool, blocks, slots, num_layers)
    nd = 5 if num_layers > 1 else 4
    _check(lib.cb_swap_in_blocks(ctypes.c_void_p(pool.data_ptr()), _dev(slots, "slots", torch.int32, 1),
                                 _dev(blocks, "blocks", torch.int32, 1), blocks.numel(),
                                 _dev(k_cache, "k_cache", torch.bfloat16, nd),
                                 _dev(v_cache, "v_cache", torch.bfloat16, nd), pool.shape[0], bb, NB,
                                 int(num_layers), stride, _stream(stream)),
           "cb_swap_in_blocks")


# ---------------------------------------------------------------------------------------------
# step graphs (include/cbgraphs.h)


class GraphsConfig(ctypes.Structure):
    """cb_step_graphs_config, field for field."""
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_blocks", ctypes.c_int64), ("max_blocks_per_seq", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("max_seqs", ctypes.c_int32),
                ("max_kv_len", ctypes.c_int32), ("token_interval", ctypes.c_int32),
                ("kv_interval", ctypes.c_int32), ("seq_interval", ctypes.c_int32),
                ("max_graphs", ctypes.c_int32), ("use_graphs", ctypes.c_int32),
                ("scale", ctypes.c_float),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p)]


def _graphs_config(q, k, v, out, k_cache, v_cache, scale, max_seqs, max_kv_len,
                   max_blocks_per_seq, token_interval, kv_interval, seq_interval, max_graphs,
                   use_graphs):
    torch = _torch()
    T, Hq, D = q.shape
    NB, bs, Hkv, _ = k_cache.shape
    if tuple(k.shape) != (T, Hkv, D) or tuple(v.shape) != (T, Hkv, D) \
            or tuple(out.shape) != (T, Hq, D) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("step configuration: inconsistent shapes")
    return GraphsConfig(Hq, Hkv, D, bs, NB, int(max_blocks_per_seq), T, int(max_seqs),
                        int(max_kv_len), int(token_interval), int(kv_interval), int(seq_interval),
                        int(max_graphs), int(bool(use_graphs)), float(scale),
                        _dev(q, "q", torch.bfloat16, 3), _dev(k, "k", torch.bfloat16, 3),
                        _dev(v, "v", torch.bfloat16, 3), _dev(out, "out", torch.bfloat16, 3),
                        _dev(k_cache, "k_cache", torch.bfloat16, 4),
                        _dev(v_cache, "v_cache", torch.bfloat16, 4))


class StepGraphs:
    """Owner of one cb_step_graphs executor over fixed torch buffers (kept referenced here):
    q [max_tokens, Hq, D], k, v [max_tokens, Hkv, D], out [max_tokens, Hq, D], caches
    [num_blocks, bs, Hkv, D], all bf16 on the GPU. use_graphs records and replays HIP graphs;
    the default launches the step's kernels directly (less GPU time per step on MI355X)."""

    def __init__(self, q, k, v, out, k_cache, v_cache, scale: float, max_seqs: int,
                 max_kv_len: int, max_blocks_per_seq: int, token_interval: int = 16,
                 kv_interval: int = 256, seq_interval: int = 8, max_graphs: int = 32,
                 use_graphs: bool = False):
        torch = _torch()
        T, Hq, D = q.shape
        NB, bs, Hkv, _ = k_cache.shape
        if tuple(k.shape) != (T, Hkv, D) or tuple(v.shape) != (T, Hkv, D) \
                or tuple(out.shape) != (T, Hq, D) or tuple(v_cache.shape) != tuple(k_cache.shape):
            raise ValueError("StepGraphs: inconsistent shapes")
        self._bufs = (q, k, v, out, k_cache, v_cache)
        cfg = _graphs_config(q, k, v, out, k_cache, v_cache, scale, max_seqs, max_kv_len,
                             max_blocks_per_seq, token_interval, kv_interval, seq_interval,
                             max_graphs, use_graphs)
        h = ctypes.c_void_p()
        _check(lib.cb_graphs_create(ctypes.byref(cfg), ctypes.byref(h)), "cb_graphs_create")
        self._h = h
        self._destroy = lib.cb_graphs_destroy
        self.max_blocks_per_seq = int(max_blocks_per_seq)

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self._destroy(self._h)
            self._h = None

    __del__ = close

    def run(self, cu_seqlens_q, kv_lens, block_tables, stream=None):
        """One step from host metadata (numpy int32); returns the padded shape (Sb, Tb, max q,
        max kv). The stream must not be torch's default (NULL) stream."""
        cu = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
        kv = np.ascontiguousarray(kv_lens, dtype=np.int32)
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        S = kv.size
        if cu.size != S + 1 or (S and bt.shape != (S, self.max_blocks_per_seq)):
            raise ValueError("StepGraphs.run: inconsistent metadata shapes")
        shape = (ctypes.c_int32 * 4)()
        _check(lib.cb_graphs_run(self._h, _ptr(cu), _ptr(kv), _ptr(bt), S, _stream(stream), shape),
               "cb_graphs_run")
        return tuple(shape)

    def stats(self):
        """(graphs recorded, replays, eager first runs, graphs cached)."""
        c, r, e = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        n = ctypes.c_int32()
        _check(lib.cb_graphs_stats(self._h, ctypes.byref(c), ctypes.byref(r), ctypes.byref(e),
                                   ctypes.byref(n)), "cb_graphs_stats")
        return c.value, r.value, e.value, n.value


# ---------------------------------------------------------------------------------------------
# async steps (include/cbasync.h)


def cb_carry_over(prev_outputs, dest, next_inputs, num_prev=None, num_next=None, stream=None):
    """next_inputs[dest[i]] += prev_outputs[i] for dest[i] >= 0 (int32 device tensors)."""
    torch = _torch()
    n = dest.numel() if num_prev is None else int(num_prev)
    m = next_inputs.numel() if num_next is None else int(num_next)
    _check(lib.cb_carry_over(_dev(prev_outputs, "prev_outputs", torch.int32, 1),
                             _dev(dest, "dest", torch.int32, 1), n,
                             _dev(next_inputs, "next_inputs", torch.int32, 1), m, _stream(stream)),
           "cb_carry_over")


class AsyncConfig(ctypes.Structure):
    """cb_async_config, field for field."""
    _fields_ = [("step", GraphsConfig)] + [(name, ctypes.c_void_p * 2) for name in (
        "in_ids", "out_ids", "carry_dest", "in_ids_host", "carry_dest_host", "out_ids_host")]


class AsyncSteps:
    """Owner of one cb_async_steps runtime over fixed torch buffers (as StepGraphs), with its
    A/B token buffers allocated here: in_ids, out_ids, carry_dest (device int32 [2][max_tokens])
    and in_ids_host, carry_dest_host, out_ids_host (pinned host int32 [2][max_tokens])."""

    def __init__(self, q, k, v, out, k_cache, v_cache, scale: float, max_seqs: int,
                 max_kv_len: int, max_blocks_per_seq: int, token_interval: int = 16,
                 kv_interval: int = 256, seq_interval: int = 8, max_graphs: int = 32,
                 use_graphs: bool = False):
        torch = _torch()
        T = q.shape[0]
        dev = q.device
        self.in_ids = [torch.zeros(T, dtype=torch.int32, device=dev) for _ in range(2)]
        self.out_ids = [torch.zeros(T, dtype=torch.int32, device=dev) for _ in range(2)]
        self.carry_dest = [torch.full((T,), -1, dtype=torch.int32, device=dev) for _ in range(2)]
        self.in_ids_host = [torch.zeros(T, dtype=torch.int32, pin_memory=True) for _ in range(2)]
        self.carry_dest_host = [torch.full((T,), -1, dtype=torch.int32).pin_memory() for _ in range(2)]
        self.out_ids_host = [torch.zeros(T, dtype=torch.int32, pin_memory=True) for _ in range(2)]
        self._bufs = (q, k, v, out, k_cache, v_cache)
        step = _graphs_config(q, k, v, out, k_cache, v_cache, scale, max_seqs, max_kv_len,
                              max_blocks_per_seq, token_interval, kv_interval, seq_interval,
                              max_graphs, use_graphs)
        ptrs = lambda ts: (ctypes.c_void_p * 2)(*[t.data_ptr() for t in ts])  # noqa: E731
        cfg = AsyncConfig(step, ptrs(self.in_ids), ptrs(self.out_ids), ptrs(self.carry_dest),
                          ptrs(self.in_ids_host), ptrs(self.carry_dest_host), ptrs(self.out_ids_host))
        h = ctypes.c_void_p()
        _check(lib.cb_async_create(ctypes.byref(cfg), ctypes.byref(h)), "cb_async_create")
        self._h = h
        self._destroy = lib.cb_async_destroy
        self.max_blocks_per_seq = int(max_blocks_per_seq)
        self.compute_stream = None

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self._destroy(self._h)
            self._h = None

    __del__ = close

    def slot(self) -> int:
        s = ctypes.c_int32()
        _check(lib.cb_async_slot(self._h, ctypes.byref(s)), "cb_async_slot")
        return s.value

    def begin(self, cu_seqlens_q, kv_lens, block_tables, num_carried: int):
        """Uploads the step's inputs and runs the carry-over; returns the compute stream as a
        torch stream for the caller's work."""
        cu = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
        kv = np.ascontiguousarray(kv_lens, dtype=np.int32)
        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        if cu.size != kv.size + 1 or bt.shape != (kv.size, self.max_blocks_per_seq):
            raise ValueError("AsyncSteps.begin: inconsistent metadata shapes")
        st = ctypes.c_void_p()
        _check(lib.cb_async_begin(self._h, _ptr(cu), _ptr(kv), _ptr(bt), kv.size, int(num_carried),
                                  ctypes.byref(st)), "cb_async_begin")
        if self.compute_stream is None:
            self.compute_stream = _torch().cuda.ExternalStream(st.value)
        return self.compute_stream

    def attention(self):
        _check(lib.cb_async_attention(self._h), "cb_async_attention")

    def end(self, num_outputs: int):
        _check(lib.cb_async_end(self._h, int(num_outputs)), "cb_async_end")

    def wait(self, slot: int):
        _check(lib.cb_async_wait(self._h, int(slot)), "cb_async_wait")
