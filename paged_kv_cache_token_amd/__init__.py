"""Python binding of libpa, the paged-attention C ABI for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind ``include/pa.h``.  Tensors are PyTorch device tensors; calls are
enqueued on the current torch stream of the tensors' device and return without
waiting.  Importing this package fails loudly when libpa.so has not been built
(``python paged_kv_cache_token_amd/build.py``); there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")
INCLUDE_DIR = os.path.join(os.path.dirname(_HERE), "include")
HEADER_PATH = os.path.join(INCLUDE_DIR, "pa.h")

PA_F32, PA_BF16 = 0, 1
PA_ERR_NO_FREE_BLOCKS = 6
PA_ERR_HOST_MEMORY = 7
BLOCK_SIZE = 16
_DTYPES = {torch.float32: PA_F32, torch.bfloat16: PA_BF16}

_c_i32, _c_i64, _c_f32, _c_sz, _c_p = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                       ctypes.c_size_t, ctypes.c_void_p)

_SIGNATURES = {
    "pa_version": (_c_i32, []),
    "pa_status_string": (ctypes.c_char_p, [_c_i32]),
    "pa_build_slot_mapping": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_i32, _c_i64, _c_i32, _c_i32, _c_p]),
    "pa_write_kv": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i32, _c_i32, _c_i32, _c_i64,
                             _c_i32, _c_p]),
    "pa_decode_workspace_size": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "pa_decode": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i32, _c_i32, _c_i32,
                           _c_i32, _c_i32, _c_i32, _c_i64, _c_f32, _c_i32, _c_p, _c_sz, _c_p]),
    "pa_decode_noalloc": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i32, _c_i32,
                                   _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_f32, _c_i32, _c_p]),
    "pa_decode_step": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i32,
                                _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_f32, _c_i32,
                                _c_p, _c_sz, _c_p]),
    "pa_cascade_workspace_size": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "pa_cascade_decode": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i32, _c_i32,
                                   _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32, _c_f32, _c_i32,
                                   _c_p, _c_sz, _c_p]),
    "pa_varlen_workspace_size": (_c_sz, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "pa_varlen_prefill": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i32,
                                   _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                   _c_i64, _c_f32, _c_i32, _c_p, _c_sz, _c_p]),
    "pa_varlen_prefill_ex": (_c_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i32,
                                      _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                      _c_i64, _c_f32, _c_i32, _c_i32, _c_p, _c_sz, _c_p]),
    "pa_swap_blocks": (_c_i32, [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_p]),
    # host-side block manager (include/pa_blocks.h)
    "pa_bm_create": (_c_i32, [_c_i64, _c_i32, ctypes.POINTER(_c_p)]),
    "pa_bm_destroy": (None, [_c_p]),
    "pa_bm_num_free_blocks": (_c_i64, [_c_p]),
    "pa_bm_allocate_slots": (_c_i32, [_c_p, _c_i64, _c_i32, _c_i32]),
    "pa_bm_allocate_batch": (_c_i32, [_c_p, _c_p, _c_p, _c_i32, _c_i32, ctypes.POINTER(_c_i32)]),
    "pa_bm_share_prefix": (_c_i32, [_c_p, _c_i64, _c_i64, _c_i32]),
    "pa_bm_free_sequence": (_c_i32, [_c_p, _c_i64]),
    "pa_bm_sequence_info": (_c_i32, [_c_p, _c_i64, ctypes.POINTER(_c_i32), ctypes.POINTER(_c_i32)]),
    "pa_bm_block_refcount": (_c_i32, [_c_p, _c_i64]),
    "pa_bm_block_table": (_c_i32, [_c_p, _c_i64, _c_p, _c_i32]),
    "pa_bm_build_step": (_c_i32, [_c_p, _c_p, _c_p, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_p, _c_p,
                                  _c_i64]),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built: run `python paged_kv_cache_token_amd/build.py` "
            "(hipcc --offload-arch=gfx950). The library has no non-HIP fallback.")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class PAError(RuntimeError):
    def __init__(self, call: str, status: int):
        self.status = status
        super().__init__(f"{call}: status {status} ({status_string(status)})")


def version() -> int:
    return int(lib.pa_version())


def status_string(status: int) -> str:
    return lib.pa_status_string(status).decode()


def header_functions() -> list[str]:
    """Names of the functions the headers under include/ declare."""
    names = set()
    for h in sorted(os.listdir(INCLUDE_DIR)):
        if h.endswith(".h"):
            text = open(os.path.join(INCLUDE_DIR, h)).read()
            names |= set(re.findall(r"^\s*(?:[\w\*]+\s+)+\**(pa_\w+)\s*\(", text, re.M))
    return sorted(names)


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------

def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")


def _need_shape(t: torch.Tensor, name: str, shape: tuple):
    """t has exactly `shape`: the kernels index every array by the counts the
    call passes, so a shorter array would be read or written past its end."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"all tensors must be on one device, got {sorted(map(str, devs))}")


def _check(call: str, status: int):
    if status != 0:
        raise PAError(call, status)


def _cache_dims(k_cache: torch.Tensor):
    num_blocks, num_kv_heads, block_size, head_dim = k_cache.shape
    return num_blocks, num_kv_heads, block_size, head_dim


def _workspace(size: int, like: torch.Tensor, workspace):
    if size == 0:
        return workspace, 0 if workspace is None else workspace.numel()
    if workspace is None:
        workspace = torch.empty(size, dtype=torch.uint8, device=like.device)
    return workspace, workspace.numel() * workspace.element_size()


# --------------------------------------------------------------------------
# calls
# --------------------------------------------------------------------------

def build_slot_mapping(cu_seqlens: torch.Tensor, context_offsets: torch.Tensor,
                       block_tables: torch.Tensor, num_tokens: int,
                       out: torch.Tensor | None = None) -> torch.Tensor:
    """int64 [num_tokens] cache slot of every new token (pa_build_slot_mapping)."""
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _need(context_offsets, "context_offsets", torch.int32, 1)
    _need(block_tables, "block_tables", torch.int32, 2)
    if out is None:
        out = torch.empty(num_tokens, dtype=torch.int64, device=cu_seqlens.device)
    _need(out, "out", torch.int64, 1)
    n = context_offsets.shape[0]
    _need_shape(cu_seqlens, "cu_seqlens", (n + 1,))
    if block_tables.shape[0] != n:
        raise ValueError(f"block_tables must have {n} rows, got {block_tables.shape[0]}")
    if out.shape[0] < num_tokens:
        raise ValueError(f"out holds {out.shape[0]} slots, fewer than num_tokens = {num_tokens}")
    _same_device(cu_seqlens, context_offsets, block_tables, out)
    _check("pa_build_slot_mapping", lib.pa_build_slot_mapping(
        _ptr(out), _ptr(cu_seqlens), _ptr(context_offsets), _ptr(block_tables), n, num_tokens,
        block_tables.shape[1], BLOCK_SIZE, _stream(cu_seqlens)))
    return out


def write_kv(key: torch.Tensor, value: torch.Tensor, k_cache: torch.Tensor,
             v_cache: torch.Tensor, slot_mapping: torch.Tensor) -> None:
    """Store key/value [T, Hkv, d] into their cache slots (pa_write_kv)."""
    for t, nm in ((key, "key"), (value, "value"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, nm)
    _need(slot_mapping, "slot_mapping", torch.int64, 1)
    num_blocks, hkv, bs, d = _cache_dims(k_cache)
    if key.dtype not in _DTYPES or len({key.dtype, value.dtype, k_cache.dtype, v_cache.dtype}) != 1:
        raise TypeError("key, value and caches must share dtype float32 or bfloat16")
    if key.shape != value.shape or key.dim() != 3 or key.shape[1:] != (hkv, d):
        raise ValueError("key/value must be [num_tokens, num_kv_heads, head_dim]")
    if v_cache.shape != k_cache.shape or slot_mapping.shape[0] != key.shape[0]:
        raise ValueError("cache shapes or slot_mapping length mismatch")
    _same_device(key, value, k_cache, v_cache, slot_mapping)
    _check("pa_write_kv", lib.pa_write_kv(
        _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), key.shape[0],
        hkv, d, bs, num_blocks, _DTYPES[key.dtype], _stream(key)))


def _decode_shapes(q, out, k_cache, v_cache, block_tables, context_lens, workspace, *extra):
    n = q.shape[0]
    _need_shape(out, "out", tuple(q.shape))
    _need_shape(v_cache, "v_cache", tuple(k_cache.shape))
    _need_shape(context_lens, "context_lens", (n,))
    if block_tables.shape[0] != n:
        raise ValueError(f"block_tables must have {n} rows, got {block_tables.shape[0]}")
    _same_device(q, out, k_cache, v_cache, block_tables, context_lens, workspace, *extra)


def decode_workspace_size(num_seqs: int, num_q_heads: int, head_dim: int, max_context_len: int,
                          dtype: torch.dtype) -> int:
    return int(lib.pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len,
                                            _DTYPES[dtype]))


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
           scale: float | None = None, out: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Paged decode attention (pa_decode); returns out [num_seqs, Hq, d]."""
    for t, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, nm)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    num_blocks, hkv, bs, d = _cache_dims(k_cache)
    n, hq, dq = q.shape
    if dq != d or q.dtype not in _DTYPES or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q / cache head_dim or dtype mismatch")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype)
    _decode_shapes(q, out, k_cache, v_cache, block_tables, context_lens, workspace)
    scale = float(d ** -0.5 if scale is None else scale)
    size = decode_workspace_size(n, hq, d, max_context_len, q.dtype)
    workspace, ws_bytes = _workspace(size, q, workspace)
    _check("pa_decode", lib.pa_decode(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        n, hq, hkv, d, bs, block_tables.shape[1], int(max_context_len), num_blocks, scale,
        _DTYPES[q.dtype], _ptr(workspace), ws_bytes, _stream(q)))
    return out


def decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                   scale: float | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """pa_decode with no workspace (pa_decode_noalloc): the library's fixed
    per-GPU scratch holds the split-K partials.  Allocates nothing when
    ``out`` is given; calls overlapping on one GPU race."""
    for t, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, nm)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    num_blocks, hkv, bs, d = _cache_dims(k_cache)
    n, hq, dq = q.shape
    if dq != d or q.dtype not in _DTYPES or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q / cache head_dim or dtype mismatch")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype)
    _decode_shapes(q, out, k_cache, v_cache, block_tables, context_lens, None)
    scale = float(d ** -0.5 if scale is None else scale)
    _check("pa_decode_noalloc", lib.pa_decode_noalloc(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        n, hq, hkv, d, bs, block_tables.shape[1], int(max_context_len), num_blocks, scale,
        _DTYPES[q.dtype], _stream(q)))
    return out


def decode_step(q: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                context_lens: torch.Tensor, max_context_len: int, scale: float | None = None,
                out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Store each sequence's new token and attend, in one launch (pa_decode_step)."""
    for t, nm in ((q, "q"), (key, "key"), (value, "value"), (k_cache, "k_cache"),
                  (v_cache, "v_cache")):
        _need(t, nm)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    num_blocks, hkv, bs, d = _cache_dims(k_cache)
    n, hq, dq = q.shape
    if dq != d or q.dtype not in _DTYPES or len({q.dtype, key.dtype, value.dtype, k_cache.dtype,
                                                 v_cache.dtype}) != 1:
        raise ValueError("q / key / value / cache head_dim or dtype mismatch")
    if key.shape != (n, hkv, d) or value.shape != key.shape:
        raise ValueError("key/value must be [num_seqs, num_kv_heads, head_dim]")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype)
    _decode_shapes(q, out, k_cache, v_cache, block_tables, context_lens, workspace, key, value)
    scale = float(d ** -0.5 if scale is None else scale)
    size = decode_workspace_size(n, hq, d, max_context_len, q.dtype)
    workspace, ws_bytes = _workspace(size, q, workspace)
    _check("pa_decode_step", lib.pa_decode_step(
        _ptr(out), _ptr(q), _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_tables), _ptr(context_lens), n, hq, hkv, d, bs, block_tables.shape[1],
        int(max_context_len), num_blocks, scale, _DTYPES[q.dtype], _ptr(workspace), ws_bytes,
        _stream(q)))
    return out


def cascade_workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                           max_context_len: int, num_common_prefix_blocks: int,
                           dtype: torch.dtype) -> int:
    return int(lib.pa_cascade_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                             max_context_len, num_common_prefix_blocks,
                                             _DTYPES[dtype]))


def cascade_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                   num_common_prefix_blocks: int, scale: float | None = None,
                   out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Decode of sequences whose tables share their first blocks
    (pa_cascade_decode); returns out [num_seqs, Hq, d]."""
    for t, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, nm)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    num_blocks, hkv, bs, d = _cache_dims(k_cache)
    n, hq, dq = q.shape
    if dq != d or q.dtype not in _DTYPES or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q / cache head_dim or dtype mismatch")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype)
    _decode_shapes(q, out, k_cache, v_cache, block_tables, context_lens, workspace)
    scale = float(d ** -0.5 if scale is None else scale)
    size = cascade_workspace_size(n, hq, hkv, d, max_context_len, num_common_prefix_blocks,
                                  q.dtype)
    workspace, ws_bytes = _workspace(size, q, workspace)
    _check("pa_cascade_decode", lib.pa_cascade_decode(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        n, hq, hkv, d, bs, block_tables.shape[1], int(max_context_len), num_blocks,
        int(num_common_prefix_blocks), scale, _DTYPES[q.dtype], _ptr(workspace), ws_bytes,
        _stream(q)))
    return out


def varlen_workspace_size(num_seqs: int, total_q_tokens: int, num_q_heads: int,
                          num_kv_heads: int, head_dim: int, max_context_len: int,
                          dtype: torch.dtype) -> int:
    return int(lib.pa_varlen_workspace_size(num_seqs, total_q_tokens, num_q_heads, num_kv_heads,
                                            head_dim, max_context_len, _DTYPES[dtype]))


def varlen_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   cu_seqlens: torch.Tensor, context_offsets: torch.Tensor,
                   block_tables: torch.Tensor, max_q_len: int, max_context_len: int,
                   scale: float | None = None, out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None,
                   num_decode_rows: int | None = None) -> torch.Tensor:
    """Packed super-sequence attention (pa_varlen_prefill); out [total_q, Hq, d].
    ``num_decode_rows``: the host's count of single-token sequences
    (pa_varlen_prefill_ex; 0 launches no decode kernels), None if unknown."""
    for t, nm in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, nm)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _need(context_offsets, "context_offsets", torch.int32, 1)
    _need(block_tables, "block_tables", torch.int32, 2)
    num_blocks, hkv, bs, d = _cache_dims(k_cache)
    total_q, hq, dq = q.shape
    if dq != d or q.dtype not in _DTYPES or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q / cache head_dim or dtype mismatch")
    n = context_offsets.shape[0]
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype)
    _need_shape(out, "out", tuple(q.shape))
    _need_shape(v_cache, "v_cache", tuple(k_cache.shape))
    _need_shape(cu_seqlens, "cu_seqlens", (n + 1,))
    if block_tables.shape[0] != n:
        raise ValueError(f"block_tables must have {n} rows, got {block_tables.shape[0]}")
    _same_device(q, out, k_cache, v_cache, cu_seqlens, context_offsets, block_tables, workspace)
    scale = float(d ** -0.5 if scale is None else scale)
    size = varlen_workspace_size(n, total_q, hq, hkv, d, max_context_len, q.dtype)
    workspace, ws_bytes = _workspace(size, q, workspace)
    if num_decode_rows is None:
        _check("pa_varlen_prefill", lib.pa_varlen_prefill(
            _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens),
            _ptr(context_offsets), _ptr(block_tables), n, total_q, int(max_q_len),
            int(max_context_len), hq, hkv, d, bs, block_tables.shape[1], num_blocks, scale,
            _DTYPES[q.dtype], _ptr(workspace), ws_bytes, _stream(q)))
    else:
        _check("pa_varlen_prefill_ex", lib.pa_varlen_prefill_ex(
            _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens),
            _ptr(context_offsets), _ptr(block_tables), n, total_q, int(max_q_len),
            int(max_context_len), hq, hkv, d, bs, block_tables.shape[1], num_blocks, scale,
            _DTYPES[q.dtype], int(num_decode_rows), _ptr(workspace), ws_bytes, _stream(q)))
    return out


def _need_pool(t: torch.Tensor, name: str):
    """A block pool or pair list for pa_swap_blocks: a contiguous device
    tensor or a contiguous pinned host tensor (the kernel reaches pinned
    host memory over the host link; pageable memory it cannot)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda" and not (t.device.type == "cpu" and t.is_pinned()):
        raise ValueError(f"{name} must be a device tensor or a pinned host tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def swap_blocks(dst: torch.Tensor, src: torch.Tensor, block_pairs: torch.Tensor,
                stream_device: torch.device | None = None) -> None:
    """dst[pair[1]] = src[pair[0]] for every row of block_pairs (pa_swap_blocks):
    whole blocks between two pools of one layout ([num_blocks, ...]), each on
    the device or in pinned host memory.  The copy is enqueued on the current
    stream of the device tensor among the arguments (or stream_device)."""
    _need_pool(dst, "dst")
    _need_pool(src, "src")
    _need_pool(block_pairs, "block_pairs")
    if block_pairs.dtype != torch.int64 or block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be int64 [num_pairs, 2]")
    if dst.dtype != src.dtype or dst.shape[1:] != src.shape[1:]:
        raise ValueError("dst and src must be pools of one layout")
    block_bytes = (dst[0].numel() if dst.shape[0] else src[0].numel()) * dst.element_size()
    dev = stream_device or next((t.device for t in (dst, src, block_pairs) if t.is_cuda),
                                torch.device("cuda", torch.cuda.current_device()))
    _check("pa_swap_blocks", lib.pa_swap_blocks(
        _ptr(dst), _ptr(src), _ptr(block_pairs), block_pairs.shape[0], block_bytes, dst.shape[0],
        src.shape[0], torch.cuda.current_stream(dev).cuda_stream))


class BlockManager:
    """Host-side block manager (include/pa_blocks.h): a pool of num_blocks
    physical blocks, a FIFO free queue, block tables and reference counts,
    and the builder of a step's attention metadata.  Host-side numpy arrays;
    copy them to the device for the attention calls."""

    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE):
        h = _c_p()
        _check("pa_bm_create", lib.pa_bm_create(int(num_blocks), int(block_size), ctypes.byref(h)))
        self._h = h
        self._destroy = lib.pa_bm_destroy  # kept: module globals may be gone at exit
        self.num_blocks = int(num_blocks)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._destroy(h)
            self._h = None

    @property
    def num_free_blocks(self) -> int:
        return int(lib.pa_bm_num_free_blocks(self._h))

    def allocate_slots(self, seq_id: int, num_new_tokens: int, num_lookahead_tokens: int = 0) -> bool:
        """True when the blocks were allocated; False when the free queue is
        too short (nothing changed)."""
        st = lib.pa_bm_allocate_slots(self._h, int(seq_id), int(num_new_tokens),
                                      int(num_lookahead_tokens))
        if st == PA_ERR_NO_FREE_BLOCKS:
            return False
        _check("pa_bm_allocate_slots", st)
        return True

    def allocate_batch(self, seq_ids, num_new_tokens, num_lookahead_tokens: int = 0) -> int:
        """allocate_slots for each sequence in order, in one call; returns how
        many were served (all of them unless the free queue ran short)."""
        import numpy as np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        nt = np.ascontiguousarray(num_new_tokens, dtype=np.int32)
        if ids.shape != nt.shape or ids.ndim != 1:
            raise ValueError("seq_ids and num_new_tokens must be 1-D of one length")
        served = _c_i32(0)
        st = lib.pa_bm_allocate_batch(self._h, ids.ctypes.data, nt.ctypes.data, ids.shape[0],
                                      int(num_lookahead_tokens), ctypes.byref(served))
        if st not in (0, PA_ERR_NO_FREE_BLOCKS):
            _check("pa_bm_allocate_batch", st)
        return int(served.value)

    def share_prefix(self, src_seq: int, dst_seq: int, num_tokens: int) -> None:
        _check("pa_bm_share_prefix", lib.pa_bm_share_prefix(self._h, int(src_seq), int(dst_seq),
                                                             int(num_tokens)))

    def free(self, seq_id: int) -> None:
        _check("pa_bm_free_sequence", lib.pa_bm_free_sequence(self._h, int(seq_id)))

    def info(self, seq_id: int) -> tuple[int, int]:
        """(tokens, blocks) of a sequence."""
        t, b = _c_i32(), _c_i32()
        _check("pa_bm_sequence_info", lib.pa_bm_sequence_info(self._h, int(seq_id), ctypes.byref(t),
                                                               ctypes.byref(b)))
        return t.value, b.value

    def refcount(self, block_id: int) -> int:
        return int(lib.pa_bm_block_refcount(self._h, int(block_id)))

    def block_table(self, seq_id: int):
        import numpy as np
        _, nb = self.info(seq_id)
        out = np.empty(max(nb, 1), dtype=np.int32)
        _check("pa_bm_block_table", lib.pa_bm_block_table(self._h, int(seq_id),
                                                           out.ctypes.data, out.shape[0]))
        return out[:nb]

    def build_step(self, seq_ids, q_lens, max_blocks_per_seq: int) -> dict:
        """Attention metadata of one packed step (host numpy arrays):
        block_tables, cu_seqlens, context_offsets, context_lens, slot_mapping."""
        import numpy as np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        ql = np.ascontiguousarray(q_lens, dtype=np.int32)
        n = ids.shape[0]
        bt = np.empty((max(n, 1), max_blocks_per_seq), dtype=np.int32)
        cu = np.empty(n + 1, dtype=np.int32)
        co = np.empty(max(n, 1), dtype=np.int32)
        cl = np.empty(max(n, 1), dtype=np.int32)
        total = int(ql.sum()) if n else 0
        sm = np.empty(max(total, 1), dtype=np.int64)
        _check("pa_bm_build_step", lib.pa_bm_build_step(
            self._h, ids.ctypes.data, ql.ctypes.data, n, int(max_blocks_per_seq), bt.ctypes.data,
            cu.ctypes.data, co.ctypes.data, cl.ctypes.data, sm.ctypes.data, sm.shape[0]))
        return {"block_tables": bt[:n], "cu_seqlens": cu, "context_offsets": co[:n],
                "context_lens": cl[:n], "slot_mapping": sm[:total]}


__all__ = ["BlockManager", "PAError", "swap_blocks", "PA_F32", "PA_BF16", "PA_ERR_NO_FREE_BLOCKS",
           "PA_ERR_HOST_MEMORY", "BLOCK_SIZE", "build_slot_mapping",
           "cascade_decode", "cascade_workspace_size", "decode", "decode_noalloc", "decode_step",
           "decode_workspace_size", "header_functions", "lib", "status_string", "varlen_prefill",
           "varlen_workspace_size", "version", "write_kv"]
