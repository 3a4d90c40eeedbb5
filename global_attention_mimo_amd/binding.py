"""ctypes binding of libmimo_attn.so (C ABI: include/mimo_attn.h).

Function names match the C entry points.  The wrappers only marshal
arguments: they take torch tensors that already live on the GPU, pass their
device pointers and the current HIP stream, and raise ``MimoError`` on a
non-OK status.  Every step of the computation runs in the HIP kernels; there is
no fallback path, and a missing library raises ``ImportError`` on first use.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
# The library built in-tree; MIMO_ATTN_LIBRARY names another build of the same
# ABI (the sanitizer test loads a host-only instrumented build of the
# validation layer this way).
LIBRARY = os.environ.get("MIMO_ATTN_LIBRARY") or os.path.join(PKG, "libmimo_attn.so")

MIMO_LAYER_SWA = 0
MIMO_LAYER_GA = 1
MIMO_OK = 0
MIMO_ERR_INVALID_ARG = 1
MIMO_ERR_UNSUPPORTED = 2
MIMO_ERR_WORKSPACE = 3
MIMO_ERR_HIP = 4
MIMO_ERR_PRECONDITION = 5

# Check-mode findings (MIMO_CHECK_* of include/mimo_attn.h).
CHECK_BITS = {"CU_START": 0x001, "CU_ORDER": 0x002, "CU_LENGTH": 0x004, "CU_TOTAL": 0x008, "CTX_RANGE": 0x010,
              "KV_BASE": 0x020, "CAPACITY": 0x040, "BLOCK_TABLE": 0x080, "SINK": 0x100, "FP8_SCALE": 0x200}

ENTRY_POINTS = ("mimo_attn_prefill", "mimo_attn_prefill_chunk", "mimo_attn_decode_workspace_size",
                "mimo_attn_decode", "mimo_attn_decode_noalloc", "mimo_attn_decode_append", "mimo_attn_decode_append_rope",
                "mimo_kv_append", "mimo_kv_append_paged",
                "mimo_attn_decode_paged",
                "mimo_attn_prefill_chunk_paged", "mimo_kv_append_fp8", "mimo_attn_decode_fp8",
                "mimo_kv_append_fp8_paged", "mimo_attn_decode_fp8_paged", "mimo_attn_prefill_chunk_fp8",
                "mimo_attn_prefill_chunk_fp8_paged",
                "mimo_attn_prefill_backward_workspace_size", "mimo_attn_prefill_backward", "mimo_rope_apply",
                "mimo_attn_prefill_rope_workspace_size", "mimo_attn_prefill_rope", "mimo_attn_prefill_chunk_rope",
                "mimo_attn_set_check", "mimo_attn_check_flags", "mimo_status_string",
                "mimo_last_error", "mimo_abi_version")


class mimo_attn_dims(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim_qk", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
                ("sliding_window", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("value_scale", ctypes.c_float)]


class mimo_kv_pages(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("max_blocks", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int64)]


class MimoError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises ImportError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise ImportError(f"{LIBRARY} is missing: build it with `python -m global_attention_mimo_amd.build`")
        _lib = load(LIBRARY)
    return _lib


def load(path: str) -> ctypes.CDLL:
    """Opens a build of the C ABI at `path` with every entry point's signature set."""
    L = ctypes.CDLL(path)
    dims_p = ctypes.POINTER(mimo_attn_dims)
    L.mimo_attn_prefill.restype = ctypes.c_int
    L.mimo_attn_prefill.argtypes = [dims_p, ctypes.c_int, _P, _P, _P, _P, _I32, _I32, _P, _P, _P, _P]
    L.mimo_attn_prefill_chunk.restype = ctypes.c_int
    L.mimo_attn_prefill_chunk.argtypes = [dims_p, ctypes.c_int, _P, _P, _P, _P, _I32, _I32, _P, _P, _P, _P, _P,
                                          _P, _P, _P]
    L.mimo_attn_decode_workspace_size.restype = _SZ
    L.mimo_attn_decode_workspace_size.argtypes = [dims_p, ctypes.c_int, _I32, _I32, _I32]
    L.mimo_attn_decode.restype = ctypes.c_int
    L.mimo_attn_decode.argtypes = [dims_p, ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P,
                                   _P, _P, _SZ, _P]
    L.mimo_attn_decode_noalloc.restype = ctypes.c_int
    L.mimo_attn_decode_noalloc.argtypes = [dims_p, ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P,
                                           _P, _P, _P]
    L.mimo_attn_decode_append.restype = ctypes.c_int
    L.mimo_attn_decode_append.argtypes = [dims_p, ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32,
                                          _P, _P, _P, _P, _SZ, _P]
    L.mimo_attn_decode_append_rope.restype = ctypes.c_int
    L.mimo_attn_decode_append_rope.argtypes = [dims_p, ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32,
                                               _I32, _I32, ctypes.c_float, _I32, _P, _P, _P, _P, _SZ, _P]
    L.mimo_kv_append.restype = ctypes.c_int
    L.mimo_kv_append.argtypes = [dims_p, ctypes.c_int, _P, _P, _P, _P, _I32, _I32, _P, _P, _P, _P, _P]
    pages_p = ctypes.POINTER(mimo_kv_pages)
    L.mimo_kv_append_paged.restype = ctypes.c_int
    L.mimo_kv_append_paged.argtypes = [dims_p, _P, _P, _P, _P, _I32, _I32, _P, _P, pages_p, _P]
    L.mimo_attn_decode_paged.restype = ctypes.c_int
    L.mimo_attn_decode_paged.argtypes = [dims_p, _P, _P, _P, _P, _P, pages_p, _P, _I32, _I32, _I32, _P, _P, _P,
                                         _P, _SZ, _P]
    L.mimo_attn_prefill_chunk_paged.restype = ctypes.c_int
    L.mimo_attn_prefill_chunk_paged.argtypes = [dims_p, _P, _P, _P, _P, _I32, _I32, _P, _P, pages_p, _P, _P, _P,
                                                _P, _P]
    L.mimo_kv_append_fp8.restype = ctypes.c_int
    L.mimo_kv_append_fp8.argtypes = [dims_p, _P, _P, _P, _P, _I32, _I32, _P, _P, _P, _P, _P, _P, _P]
    L.mimo_attn_decode_fp8.restype = ctypes.c_int
    L.mimo_attn_decode_fp8.argtypes = [dims_p, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _P,
                                       _P, _SZ, _P]
    L.mimo_attn_prefill_backward_workspace_size.restype = _SZ
    L.mimo_kv_append_fp8_paged.restype = ctypes.c_int
    L.mimo_kv_append_fp8_paged.argtypes = [dims_p, _P, _P, _P, _P, _I32, _I32, _P, _P, pages_p, _P, _P, _P]
    L.mimo_attn_decode_fp8_paged.restype = ctypes.c_int
    L.mimo_attn_decode_fp8_paged.argtypes = [dims_p, _P, _P, _P, _P, _P, pages_p, _P, _P, _P, _I32, _I32, _I32, _P,
                                             _P, _P, _P, _SZ, _P]
    L.mimo_attn_prefill_chunk_fp8.restype = ctypes.c_int
    L.mimo_attn_prefill_chunk_fp8.argtypes = [dims_p, _P, _P, _P, _P, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P,
                                              _P, _P]
    L.mimo_attn_prefill_chunk_fp8_paged.restype = ctypes.c_int
    L.mimo_attn_prefill_chunk_fp8_paged.argtypes = [dims_p, _P, _P, _P, _P, _I32, _I32, _P, _P, pages_p, _P, _P, _P,
                                                    _P, _P, _P, _P]
    L.mimo_attn_prefill_backward_workspace_size.argtypes = [dims_p, _I32]
    L.mimo_attn_prefill_backward.restype = ctypes.c_int
    L.mimo_attn_prefill_backward.argtypes = [dims_p, ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32,
                                             _P, _P, _P, _P, _P, _P, _SZ, _P]
    L.mimo_rope_apply.restype = ctypes.c_int
    L.mimo_rope_apply.argtypes = [dims_p, _P, _P, _P, _I32, ctypes.c_float, _I32, _P]
    L.mimo_attn_prefill_rope_workspace_size.restype = _SZ
    L.mimo_attn_prefill_rope_workspace_size.argtypes = [dims_p, _I32, _I32]
    L.mimo_attn_prefill_rope.restype = ctypes.c_int
    L.mimo_attn_prefill_rope.argtypes = [dims_p, ctypes.c_int, _P, _P, _P, _P, _P, _I32, _I32, _I32,
                                         ctypes.c_float, _I32, _P, _P, _P, _P, _P, _SZ, _P]
    L.mimo_status_string.restype = ctypes.c_char_p
    L.mimo_attn_prefill_chunk_rope.restype = ctypes.c_int
    L.mimo_attn_prefill_chunk_rope.argtypes = [dims_p, ctypes.c_int, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _P,
                                               pages_p, _P, ctypes.c_float, _I32, _P, _P, _P, _P, _P, _SZ, _P]
    L.mimo_attn_set_check.restype = ctypes.c_int
    L.mimo_attn_set_check.argtypes = [ctypes.c_int]
    L.mimo_attn_check_flags.restype = ctypes.c_int
    L.mimo_attn_check_flags.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int]
    L.mimo_status_string.argtypes = [ctypes.c_int]
    L.mimo_last_error.restype = ctypes.c_char_p
    L.mimo_last_error.argtypes = []
    L.mimo_abi_version.restype = ctypes.c_int
    L.mimo_abi_version.argtypes = []
    return L


def make_dims(num_q_heads=64, num_kv_heads=4, head_dim_qk=192, head_dim_v=128, sliding_window=129,
              softmax_scale: Optional[float] = None, value_scale=1.0) -> mimo_attn_dims:
    if softmax_scale is None:
        softmax_scale = head_dim_qk ** -0.5
    return mimo_attn_dims(num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, sliding_window, softmax_scale,
                          value_scale)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(status: int):
    if status != MIMO_OK:
        raise MimoError(status, lib().mimo_last_error().decode() or mimo_status_string(status))


def mimo_status_string(status: int) -> str:
    return lib().mimo_status_string(status).decode()


def mimo_last_error() -> str:
    return lib().mimo_last_error().decode()


def mimo_abi_version() -> int:
    return int(lib().mimo_abi_version())


def mimo_attn_set_check(enable: bool) -> bool:
    """Switches check mode on or off; returns the previous setting."""
    return bool(lib().mimo_attn_set_check(1 if enable else 0))


def mimo_attn_check_flags(clear: bool = False) -> int:
    """The current device's sticky check-mode word (MIMO_CHECK_* bits)."""
    word = ctypes.c_uint32(0)
    _check(lib().mimo_attn_check_flags(ctypes.byref(word), 1 if clear else 0))
    return int(word.value)


def mimo_attn_prefill(dims: mimo_attn_dims, layer_type: int, q, k, v, cu_seqlens, num_seqs: int, max_seqlen: int,
                      sink, out, lse, stream=None) -> None:
    _check(lib().mimo_attn_prefill(ctypes.byref(dims), layer_type, _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens),
                                   num_seqs, max_seqlen, _ptr(sink), _ptr(out), _ptr(lse), _stream(stream)))


def mimo_attn_prefill_chunk(dims: mimo_attn_dims, layer_type: int, q, k, v, cu_newlens, num_seqs: int,
                            max_newlen: int, k_cache, v_cache, kv_base, ctx_lens, sink, out, lse, stream=None) -> None:
    _check(lib().mimo_attn_prefill_chunk(ctypes.byref(dims), layer_type, _ptr(q), _ptr(k), _ptr(v), _ptr(cu_newlens),
                                         num_seqs, max_newlen, _ptr(k_cache), _ptr(v_cache), _ptr(kv_base),
                                         _ptr(ctx_lens), _ptr(sink), _ptr(out), _ptr(lse), _stream(stream)))


def mimo_attn_decode_workspace_size(dims: mimo_attn_dims, layer_type: int, batch: int, max_ctx: int,
                                    split_tokens: int = 0) -> int:
    return int(lib().mimo_attn_decode_workspace_size(ctypes.byref(dims), layer_type, batch, max_ctx, split_tokens))


def mimo_attn_decode(dims: mimo_attn_dims, layer_type: int, q, k_new, v_new, k_cache, v_cache, kv_base, ctx_lens,
                     batch: int, max_ctx: int, split_tokens: int, sink, out, lse, workspace, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mimo_attn_decode(ctypes.byref(dims), layer_type, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                  _ptr(v_cache), _ptr(kv_base), _ptr(ctx_lens), batch, max_ctx, split_tokens,
                                  _ptr(sink), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def mimo_attn_decode_noalloc(dims: mimo_attn_dims, layer_type: int, q, k_new, v_new, k_cache, v_cache, kv_base,
                             ctx_lens, batch: int, max_ctx: int, split_tokens: int, sink, out, lse,
                             stream=None) -> None:
    _check(lib().mimo_attn_decode_noalloc(ctypes.byref(dims), layer_type, _ptr(q), _ptr(k_new), _ptr(v_new),
                                          _ptr(k_cache), _ptr(v_cache), _ptr(kv_base), _ptr(ctx_lens), batch, max_ctx,
                                          split_tokens, _ptr(sink), _ptr(out), _ptr(lse), _stream(stream)))


def mimo_attn_decode_append(dims: mimo_attn_dims, layer_type: int, q, k_new, v_new, k_cache, v_cache, kv_base,
                            kv_capacity, ctx_lens, batch: int, max_ctx: int, split_tokens: int, sink, out, lse,
                            workspace, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mimo_attn_decode_append(ctypes.byref(dims), layer_type, _ptr(q), _ptr(k_new), _ptr(v_new),
                                         _ptr(k_cache), _ptr(v_cache), _ptr(kv_base), _ptr(kv_capacity),
                                         _ptr(ctx_lens), batch, max_ctx, split_tokens, _ptr(sink), _ptr(out),
                                         _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def mimo_attn_decode_append_rope(dims: mimo_attn_dims, layer_type: int, q, k_new, v_new, positions, k_cache,
                                 v_cache, kv_base, kv_capacity, ctx_lens, batch: int, max_ctx: int, split_tokens: int,
                                 rope_theta: float, rotary_dim: int, sink, out, lse, workspace, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mimo_attn_decode_append_rope(ctypes.byref(dims), layer_type, _ptr(q), _ptr(k_new), _ptr(v_new),
                                              _ptr(positions), _ptr(k_cache), _ptr(v_cache), _ptr(kv_base),
                                              _ptr(kv_capacity), _ptr(ctx_lens), batch, max_ctx, split_tokens,
                                              rope_theta, rotary_dim, _ptr(sink), _ptr(out), _ptr(lse),
                                              _ptr(workspace), ws_bytes, _stream(stream)))


def mimo_kv_append(dims: mimo_attn_dims, layer_type: int, k, v, cu_newlens, ctx_lens, batch: int, total_new: int,
                   k_cache, v_cache, kv_base=None, kv_capacity=None, stream=None) -> None:
    _check(lib().mimo_kv_append(ctypes.byref(dims), layer_type, _ptr(k), _ptr(v), _ptr(cu_newlens), _ptr(ctx_lens),
                                batch, total_new, _ptr(k_cache), _ptr(v_cache), _ptr(kv_base), _ptr(kv_capacity),
                                _stream(stream)))


def make_pages(block_table: torch.Tensor, page_size: int, num_pages: int) -> mimo_kv_pages:
    """mimo_kv_pages for a [batch][max_blocks] int32 device table (kept alive by the caller)."""
    if block_table.dtype != torch.int32 or block_table.dim() != 2:
        raise ValueError("block_table must be a 2-D int32 tensor")
    return mimo_kv_pages(_ptr(block_table), block_table.shape[1], page_size, num_pages)


def _pages_ref(pages: Optional[mimo_kv_pages]):
    return None if pages is None else ctypes.byref(pages)


def mimo_kv_append_paged(dims: mimo_attn_dims, k, v, cu_newlens, ctx_lens, batch: int, total_new: int, k_cache,
                         v_cache, pages: Optional[mimo_kv_pages], stream=None) -> None:
    _check(lib().mimo_kv_append_paged(ctypes.byref(dims), _ptr(k), _ptr(v), _ptr(cu_newlens), _ptr(ctx_lens), batch,
                                      total_new, _ptr(k_cache), _ptr(v_cache), _pages_ref(pages), _stream(stream)))


def mimo_attn_decode_paged(dims: mimo_attn_dims, q, k_new, v_new, k_cache, v_cache, pages: Optional[mimo_kv_pages],
                           ctx_lens, batch: int, max_ctx: int, split_tokens: int, sink, out, lse, workspace,
                           stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mimo_attn_decode_paged(ctypes.byref(dims), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                        _ptr(v_cache), _pages_ref(pages), _ptr(ctx_lens), batch, max_ctx,
                                        split_tokens, _ptr(sink), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                        _stream(stream)))


def mimo_attn_prefill_chunk_paged(dims: mimo_attn_dims, q, k, v, cu_newlens, num_seqs: int, max_newlen: int, k_cache,
                                  v_cache, pages: Optional[mimo_kv_pages], ctx_lens, sink, out, lse,
                                  stream=None) -> None:
    _check(lib().mimo_attn_prefill_chunk_paged(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_newlens),
                                               num_seqs, max_newlen, _ptr(k_cache), _ptr(v_cache), _pages_ref(pages),
                                               _ptr(ctx_lens), _ptr(sink), _ptr(out), _ptr(lse), _stream(stream)))


def mimo_kv_append_fp8(dims: mimo_attn_dims, k, v, cu_newlens, ctx_lens, batch: int, total_new: int, k_cache, v_cache,
                       kv_base, kv_capacity, k_scale, v_scale, stream=None) -> None:
    _check(lib().mimo_kv_append_fp8(ctypes.byref(dims), _ptr(k), _ptr(v), _ptr(cu_newlens), _ptr(ctx_lens), batch,
                                    total_new, _ptr(k_cache), _ptr(v_cache), _ptr(kv_base), _ptr(kv_capacity),
                                    _ptr(k_scale), _ptr(v_scale), _stream(stream)))


def mimo_attn_decode_fp8(dims: mimo_attn_dims, q, k_new, v_new, k_cache, v_cache, kv_base, k_scale, v_scale, ctx_lens,
                         batch: int, max_ctx: int, split_tokens: int, sink, out, lse, workspace, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mimo_attn_decode_fp8(ctypes.byref(dims), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                      _ptr(v_cache), _ptr(kv_base), _ptr(k_scale), _ptr(v_scale), _ptr(ctx_lens),
                                      batch, max_ctx, split_tokens, _ptr(sink), _ptr(out), _ptr(lse), _ptr(workspace),
                                      ws_bytes, _stream(stream)))


def mimo_kv_append_fp8_paged(dims: mimo_attn_dims, k, v, cu_newlens, ctx_lens, batch: int, total_new: int, k_cache,
                             v_cache, pages: Optional[mimo_kv_pages], k_scale, v_scale, stream=None) -> None:
    _check(lib().mimo_kv_append_fp8_paged(ctypes.byref(dims), _ptr(k), _ptr(v), _ptr(cu_newlens), _ptr(ctx_lens),
                                          batch, total_new, _ptr(k_cache), _ptr(v_cache), _pages_ref(pages),
                                          _ptr(k_scale), _ptr(v_scale), _stream(stream)))


def mimo_attn_decode_fp8_paged(dims: mimo_attn_dims, q, k_new, v_new, k_cache, v_cache,
                               pages: Optional[mimo_kv_pages], k_scale, v_scale, ctx_lens, batch: int, max_ctx: int,
                               split_tokens: int, sink, out, lse, workspace, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mimo_attn_decode_fp8_paged(ctypes.byref(dims), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                            _ptr(v_cache), _pages_ref(pages), _ptr(k_scale), _ptr(v_scale),
                                            _ptr(ctx_lens), batch, max_ctx, split_tokens, _ptr(sink), _ptr(out),
                                            _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def mimo_attn_prefill_chunk_fp8(dims: mimo_attn_dims, q, k, v, cu_newlens, num_seqs: int, max_newlen: int, k_cache,
                                v_cache, kv_base, k_scale, v_scale, ctx_lens, sink, out, lse, stream=None) -> None:
    _check(lib().mimo_attn_prefill_chunk_fp8(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_newlens),
                                             num_seqs, max_newlen, _ptr(k_cache), _ptr(v_cache), _ptr(kv_base),
                                             _ptr(k_scale), _ptr(v_scale), _ptr(ctx_lens), _ptr(sink), _ptr(out),
                                             _ptr(lse), _stream(stream)))


def mimo_attn_prefill_chunk_fp8_paged(dims: mimo_attn_dims, q, k, v, cu_newlens, num_seqs: int, max_newlen: int,
                                      k_cache, v_cache, pages: Optional[mimo_kv_pages], k_scale, v_scale, ctx_lens,
                                      sink, out, lse, stream=None) -> None:
    _check(lib().mimo_attn_prefill_chunk_fp8_paged(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_newlens),
                                                   num_seqs, max_newlen, _ptr(k_cache), _ptr(v_cache),
                                                   _pages_ref(pages), _ptr(k_scale), _ptr(v_scale), _ptr(ctx_lens),
                                                   _ptr(sink), _ptr(out), _ptr(lse), _stream(stream)))


def mimo_attn_prefill_backward_workspace_size(dims: mimo_attn_dims, total_tokens: int) -> int:
    return int(lib().mimo_attn_prefill_backward_workspace_size(ctypes.byref(dims), total_tokens))


def mimo_attn_prefill_backward(dims: mimo_attn_dims, layer_type: int, q, k, v, out, lse, dout, cu_seqlens,
                               num_seqs: int, max_seqlen: int, total_tokens: int, sink, dq, dk, dv, dsink, workspace,
                               stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mimo_attn_prefill_backward(ctypes.byref(dims), layer_type, _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                            _ptr(lse), _ptr(dout), _ptr(cu_seqlens), num_seqs, max_seqlen,
                                            total_tokens, _ptr(sink), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsink),
                                            _ptr(workspace), ws_bytes, _stream(stream)))


def mimo_rope_apply(dims: mimo_attn_dims, q, k, positions, total_tokens: int, rope_theta: float, rotary_dim: int,
                    stream=None) -> None:
    _check(lib().mimo_rope_apply(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(positions), total_tokens, rope_theta,
                                 rotary_dim, _stream(stream)))


def mimo_attn_prefill_rope_workspace_size(dims: mimo_attn_dims, total_tokens: int, rotary_dim: int) -> int:
    return int(lib().mimo_attn_prefill_rope_workspace_size(ctypes.byref(dims), total_tokens, rotary_dim))


def mimo_attn_prefill_rope(dims: mimo_attn_dims, layer_type: int, q, k, v, positions, cu_seqlens, num_seqs: int,
                           max_seqlen: int, total_tokens: int, rope_theta: float, rotary_dim: int, sink, out, lse,
                           k_rot, workspace, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mimo_attn_prefill_rope(ctypes.byref(dims), layer_type, _ptr(q), _ptr(k), _ptr(v), _ptr(positions),
                                        _ptr(cu_seqlens), num_seqs, max_seqlen, total_tokens, rope_theta, rotary_dim,
                                        _ptr(sink), _ptr(out), _ptr(lse), _ptr(k_rot), _ptr(workspace), ws_bytes,
                                        _stream(stream)))


# -- tensor-level conveniences (allocation of outputs + the calls above) -------

def prefill(q, k, v, cu_seqlens, max_seqlen: int, layer_type: int, sink=None, dims=None, out=None, lse=None,
            want_lse: bool = True, stream=None):
    dims = dims or make_dims()
    T = q.shape[0]
    if out is None:
        out = torch.empty((T, dims.num_q_heads, dims.head_dim_v), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((T, dims.num_q_heads), dtype=torch.float32, device=q.device)
    mimo_attn_prefill(dims, layer_type, q, k, v, cu_seqlens, cu_seqlens.numel() - 1, max_seqlen, sink, out, lse,
                      stream)
    return out, lse


def prefill_chunk(q, k, v, cu_newlens, max_newlen: int, k_cache, v_cache, ctx_lens, layer_type: int, sink=None,
                  kv_base=None, dims=None, out=None, lse=None, stream=None):
    dims = dims or make_dims()
    T = q.shape[0]
    if out is None:
        out = torch.empty((T, dims.num_q_heads, dims.head_dim_v), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((T, dims.num_q_heads), dtype=torch.float32, device=q.device)
    mimo_attn_prefill_chunk(dims, layer_type, q, k, v, cu_newlens, cu_newlens.numel() - 1, max_newlen, k_cache,
                            v_cache, kv_base, ctx_lens, sink, out, lse, stream)
    return out, lse


def decode(q, k_new, v_new, k_cache, v_cache, ctx_lens, max_ctx: int, layer_type: int, sink=None, kv_base=None,
           split_tokens: int = 0, dims=None, out=None, lse=None, workspace=None, stream=None):
    dims = dims or make_dims()
    B = q.shape[0]
    if out is None:
        out = torch.empty((B, dims.num_q_heads, dims.head_dim_v), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, dims.num_q_heads), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = mimo_attn_decode_workspace_size(dims, layer_type, B, max_ctx, split_tokens)
        workspace = torch.empty(max(nbytes, 16) // 4 + 4, dtype=torch.float32, device=q.device) if nbytes else None
    mimo_attn_decode(dims, layer_type, q, k_new, v_new, k_cache, v_cache, kv_base, ctx_lens, B, max_ctx,
                     split_tokens, sink, out, lse, workspace, stream)
    return out, lse


def decode_append_rope(q, k_new, v_new, positions, k_cache, v_cache, ctx_lens, max_ctx: int, layer_type: int,
                       rope_theta: float, rotary_dim: int, sink=None, kv_base=None, kv_capacity=None,
                       split_tokens: int = 0, dims=None, out=None, lse=None, workspace=None, stream=None):
    dims = dims or make_dims()
    B = q.shape[0]
    if out is None:
        out = torch.empty((B, dims.num_q_heads, dims.head_dim_v), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, dims.num_q_heads), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = mimo_attn_decode_workspace_size(dims, layer_type, B, max_ctx, split_tokens)
        workspace = torch.empty(max(nbytes, 16) // 4 + 4, dtype=torch.float32, device=q.device) if nbytes else None
    mimo_attn_decode_append_rope(dims, layer_type, q, k_new, v_new, positions, k_cache, v_cache, kv_base,
                                 kv_capacity, ctx_lens, B, max_ctx, split_tokens, rope_theta, rotary_dim, sink, out,
                                 lse, workspace, stream)
    return out, lse


def kv_append(k, v, cu_newlens, ctx_lens, k_cache, v_cache, layer_type: int, kv_base=None, kv_capacity=None,
              dims=None, total_new: Optional[int] = None, stream=None):
    dims = dims or make_dims()
    if total_new is None:
        total_new = k.shape[0]
    mimo_kv_append(dims, layer_type, k, v, cu_newlens, ctx_lens, cu_newlens.numel() - 1, total_new, k_cache, v_cache,
                   kv_base, kv_capacity, stream)


def kv_append_paged(k, v, cu_newlens, ctx_lens, k_pool, v_pool, block_table, page_size: int, dims=None,
                    total_new: Optional[int] = None, stream=None):
    dims = dims or make_dims()
    if total_new is None:
        total_new = k.shape[0]
    pages = make_pages(block_table, page_size, k_pool.shape[0] // page_size)
    mimo_kv_append_paged(dims, k, v, cu_newlens, ctx_lens, cu_newlens.numel() - 1, total_new, k_pool, v_pool, pages,
                         stream)


def decode_paged(q, k_new, v_new, k_pool, v_pool, block_table, page_size: int, ctx_lens, max_ctx: int, sink=None,
                 split_tokens: int = 0, dims=None, out=None, lse=None, workspace=None, stream=None):
    dims = dims or make_dims()
    B = q.shape[0]
    if out is None:
        out = torch.empty((B, dims.num_q_heads, dims.head_dim_v), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, dims.num_q_heads), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = mimo_attn_decode_workspace_size(dims, MIMO_LAYER_GA, B, max_ctx, split_tokens)
        workspace = torch.empty(max(nbytes, 16) // 4 + 4, dtype=torch.float32, device=q.device)
    pages = make_pages(block_table, page_size, k_pool.shape[0] // page_size)
    mimo_attn_decode_paged(dims, q, k_new, v_new, k_pool, v_pool, pages, ctx_lens, B, max_ctx, split_tokens, sink,
                           out, lse, workspace, stream)
    return out, lse


def prefill_chunk_paged(q, k, v, cu_newlens, max_newlen: int, k_pool, v_pool, block_table, page_size: int, ctx_lens,
                        sink=None, dims=None, out=None, lse=None, stream=None):
    dims = dims or make_dims()
    T = q.shape[0]
    if out is None:
        out = torch.empty((T, dims.num_q_heads, dims.head_dim_v), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((T, dims.num_q_heads), dtype=torch.float32, device=q.device)
    pages = make_pages(block_table, page_size, k_pool.shape[0] // page_size)
    mimo_attn_prefill_chunk_paged(dims, q, k, v, cu_newlens, cu_newlens.numel() - 1, max_newlen, k_pool, v_pool,
                                  pages, ctx_lens, sink, out, lse, stream)
    return out, lse


def kv_append_fp8(k, v, cu_newlens, ctx_lens, k_cache, v_cache, kv_base, kv_capacity, k_scale, v_scale, dims=None,
                  total_new: Optional[int] = None, stream=None):
    dims = dims or make_dims()
    if total_new is None:
        total_new = k.shape[0]
    mimo_kv_append_fp8(dims, k, v, cu_newlens, ctx_lens, cu_newlens.numel() - 1, total_new, k_cache, v_cache, kv_base,
                       kv_capacity, k_scale, v_scale, stream)


def decode_fp8(q, k_new, v_new, k_cache, v_cache, kv_base, k_scale, v_scale, ctx_lens, max_ctx: int, sink=None,
               split_tokens: int = 0, dims=None, out=None, lse=None, workspace=None, stream=None):
    dims = dims or make_dims()
    B = q.shape[0]
    if out is None:
        out = torch.empty((B, dims.num_q_heads, dims.head_dim_v), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, dims.num_q_heads), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = mimo_attn_decode_workspace_size(dims, MIMO_LAYER_GA, B, max_ctx, split_tokens)
        workspace = torch.empty(max(nbytes, 16) // 4 + 4, dtype=torch.float32, device=q.device)
    mimo_attn_decode_fp8(dims, q, k_new, v_new, k_cache, v_cache, kv_base, k_scale, v_scale, ctx_lens, B, max_ctx,
                         split_tokens, sink, out, lse, workspace, stream)
    return out, lse


def kv_append_fp8_paged(k, v, cu_newlens, ctx_lens, k_pool, v_pool, block_table, page_size: int, k_scale, v_scale,
                        dims=None, total_new: Optional[int] = None, stream=None):
    dims = dims or make_dims()
    if total_new is None:
        total_new = k.shape[0]
    pages = make_pages(block_table, page_size, k_pool.shape[0] // page_size)
    mimo_kv_append_fp8_paged(dims, k, v, cu_newlens, ctx_lens, cu_newlens.numel() - 1, total_new, k_pool, v_pool,
                             pages, k_scale, v_scale, stream)


def decode_fp8_paged(q, k_new, v_new, k_pool, v_pool, block_table, page_size: int, k_scale, v_scale, ctx_lens,
                     max_ctx: int, sink=None, split_tokens: int = 0, dims=None, out=None, lse=None, workspace=None,
                     stream=None):
    dims = dims or make_dims()
    B = q.shape[0]
    if out is None:
        out = torch.empty((B, dims.num_q_heads, dims.head_dim_v), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, dims.num_q_heads), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = mimo_attn_decode_workspace_size(dims, MIMO_LAYER_GA, B, max_ctx, split_tokens)
        workspace = torch.empty(max(nbytes, 16) // 4 + 4, dtype=torch.float32, device=q.device)
    pages = make_pages(block_table, page_size, k_pool.shape[0] // page_size)
    mimo_attn_decode_fp8_paged(dims, q, k_new, v_new, k_pool, v_pool, pages, k_scale, v_scale, ctx_lens, B, max_ctx,
                               split_tokens, sink, out, lse, workspace, stream)
    return out, lse


def prefill_chunk_fp8(q, k, v, cu_newlens, max_newlen: int, k_cache, v_cache, k_scale, v_scale, ctx_lens,
                      kv_base=None, block_table=None, page_size: int = 0, sink=None, dims=None, out=None, lse=None,
                      stream=None):
    """GA chunked prefill over an FP8 pool: contiguous (kv_base) or paged (block_table, page_size)."""
    dims = dims or make_dims()
    T = q.shape[0]
    if out is None:
        out = torch.empty((T, dims.num_q_heads, dims.head_dim_v), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((T, dims.num_q_heads), dtype=torch.float32, device=q.device)
    n = cu_newlens.numel() - 1
    if block_table is not None:
        pages = make_pages(block_table, page_size, k_cache.shape[0] // page_size)
        mimo_attn_prefill_chunk_fp8_paged(dims, q, k, v, cu_newlens, n, max_newlen, k_cache, v_cache, pages, k_scale,
                                          v_scale, ctx_lens, sink, out, lse, stream)
    else:
        mimo_attn_prefill_chunk_fp8(dims, q, k, v, cu_newlens, n, max_newlen, k_cache, v_cache, kv_base, k_scale,
                                    v_scale, ctx_lens, sink, out, lse, stream)
    return out, lse


def prefill_backward(q, k, v, out, lse, dout, cu_seqlens, max_seqlen: int, layer_type: int, sink=None, dims=None,
                     want_dsink: bool = True, stream=None):
    """(dq, dk, dv, dsink) of sum(dout * out) for a prefill call's inputs and outputs."""
    dims = dims or make_dims()
    T = q.shape[0]
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dsink = torch.empty(dims.num_q_heads, dtype=torch.float32, device=q.device) if want_dsink else None
    nbytes = mimo_attn_prefill_backward_workspace_size(dims, T)
    ws = torch.empty(max(nbytes, 16) // 4 + 4, dtype=torch.float32, device=q.device)
    mimo_attn_prefill_backward(dims, layer_type, q, k, v, out, lse, dout, cu_seqlens, cu_seqlens.numel() - 1,
                               max_seqlen, T, sink, dq, dk, dv, dsink, ws, stream)
    return dq, dk, dv, dsink


def prefill_rope(q, k, v, positions, cu_seqlens, max_seqlen: int, layer_type: int, rope_theta: float,
                 rotary_dim: int, sink=None, dims=None, out=None, lse=None, k_rot=None, stream=None):
    """Fused-RoPE prefill; returns (out, lse, k_rot)."""
    dims = dims or make_dims()
    T = q.shape[0]
    if out is None:
        out = torch.empty((T, dims.num_q_heads, dims.head_dim_v), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((T, dims.num_q_heads), dtype=torch.float32, device=q.device)
    if k_rot is None:
        k_rot = torch.empty_like(k)
    nbytes = mimo_attn_prefill_rope_workspace_size(dims, T, rotary_dim)
    ws = torch.empty(max(nbytes, 16) // 4 + 4, dtype=torch.float32, device=q.device)
    mimo_attn_prefill_rope(dims, layer_type, q, k, v, positions, cu_seqlens, cu_seqlens.numel() - 1, max_seqlen, T,
                           rope_theta, rotary_dim, sink, out, lse, k_rot, ws, stream)
    return out, lse, k_rot


def mimo_attn_prefill_chunk_rope(dims: mimo_attn_dims, layer_type: int, q, k, v, positions, cu_newlens, num_seqs: int,
                                 max_newlen: int, total_new: int, k_cache, v_cache, kv_base,
                                 pages: Optional[mimo_kv_pages], ctx_lens, rope_theta: float, rotary_dim: int, sink,
                                 out, lse, k_rot, workspace, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mimo_attn_prefill_chunk_rope(ctypes.byref(dims), layer_type, _ptr(q), _ptr(k), _ptr(v),
                                              _ptr(positions), _ptr(cu_newlens), num_seqs, max_newlen, total_new,
                                              _ptr(k_cache), _ptr(v_cache), _ptr(kv_base), _pages_ref(pages),
                                              _ptr(ctx_lens), rope_theta, rotary_dim, _ptr(sink), _ptr(out),
                                              _ptr(lse), _ptr(k_rot), _ptr(workspace), ws_bytes, _stream(stream)))


def prefill_chunk_rope(q, k, v, positions, cu_newlens, max_newlen: int, k_cache, v_cache, ctx_lens, layer_type: int,
                       rope_theta: float, rotary_dim: int, sink=None, kv_base=None, block_table=None,
                       page_size: int = 0, dims=None, out=None, lse=None, k_rot=None, stream=None):
    """Chunked prefill with fused RoPE; returns (out, lse, k_rot)."""
    dims = dims or make_dims()
    T = q.shape[0]
    if out is None:
        out = torch.empty((T, dims.num_q_heads, dims.head_dim_v), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((T, dims.num_q_heads), dtype=torch.float32, device=q.device)
    if k_rot is None:
        k_rot = torch.empty_like(k)
    nbytes = mimo_attn_prefill_rope_workspace_size(dims, T, rotary_dim)
    ws = torch.empty(max(nbytes, 16) // 4 + 4, dtype=torch.float32, device=q.device)
    pages = None if block_table is None else make_pages(block_table, page_size, k_cache.shape[0] // page_size)
    mimo_attn_prefill_chunk_rope(dims, layer_type, q, k, v, positions, cu_newlens, cu_newlens.numel() - 1, max_newlen,
                                 T, k_cache, v_cache, kv_base, pages, ctx_lens, rope_theta, rotary_dim, sink, out,
                                 lse, k_rot, ws, stream)
    return out, lse, k_rot


def rope_apply(q, k, positions, rope_theta: float, rotary_dim: int, dims=None, stream=None):
    """Rotates q and/or k in place at the tokens' positions."""
    dims = dims or make_dims()
    T = (q if q is not None else k).shape[0]
    mimo_rope_apply(dims, q, k, positions, T, rope_theta, rotary_dim, stream)
