"""ctypes binding of libpa.so (C ABI in include/pa.h).

Argument marshalling only: every computation runs in the library's HIP
kernels. torch provides device memory and the current HIP stream. There is no
fallback: if the library cannot be loaded, every call raises RuntimeError.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PA_LIB", os.path.join(_PKG, "libpa.so"))

PA_DTYPE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.float8_e4m3fn: 3}
PA_INDEX_DTYPE = {torch.int32: 4, torch.int64: 5}  # index arrays, in tensor descriptors only
STATUS = {0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_DTYPE", 3: "PA_ERR_SHAPE", 4: "PA_ERR_UNSUPPORTED",
          5: "PA_ERR_WORKSPACE", 6: "PA_ERR_LAUNCH", 7: "PA_ERR_CAPACITY", 8: "PA_ERR_STATE"}

EXPORTS = ("pa_reshape_and_cache", "pa_decode", "pa_reshape_and_cache_t", "pa_decode_t", "pa_decode_split", "pa_decode_workspace_bytes",
           "pa_decode_shared_prefix", "pa_decode_shared_prefix_workspace_bytes", "pa_decode_append",
           "pa_decode_partition_blocks", "pa_decode_scratch", "pa_decode_scratch_bytes", "pa_prefill", "pa_copy_blocks", "pa_bm_create", "pa_bm_destroy", "pa_bm_num_free_blocks",
           "pa_bm_block_refcount", "pa_bm_add_sequence", "pa_bm_fork", "pa_bm_free_sequence", "pa_bm_append_slots",
           "pa_bm_block_tables", "pa_bm_shared_prefix", "pa_last_error", "pa_version")

_lock = threading.Lock()
_lib = None

_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class PaTensor(ctypes.Structure):
    """pa_tensor: pointer, dtype, rank, shape and strides (in elements) of one array."""
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


def tensor_desc(t: torch.Tensor) -> PaTensor:
    """The pa_tensor of a torch tensor (its own shape and strides: the library checks them)."""
    code = PA_DTYPE.get(t.dtype, PA_INDEX_DTYPE.get(t.dtype))
    if code is None:
        raise ValueError(f"unsupported dtype {t.dtype}")
    if not 1 <= t.dim() <= 4:
        raise ValueError("tensors of 1 to 4 dimensions")
    d = PaTensor()
    d.data, d.dtype, d.ndim = t.data_ptr(), code, t.dim()
    for i in range(t.dim()):
        d.shape[i], d.stride[i] = t.shape[i], t.stride(i)
    return d


class PAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libpa.so once and declare its signatures."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(f"libpa.so not found at {p}: build it with `python -m paged_kv_cache_380_amd.build`")
        lib = ctypes.CDLL(p)
        lib.pa_reshape_and_cache.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i64, _i32, _i32, _i32,
                                             _f32, _f32, _vp]
        lib.pa_reshape_and_cache.restype = _i32
        desc = ctypes.POINTER(PaTensor)
        lib.pa_reshape_and_cache_t.argtypes = [desc] * 5 + [_f32, _f32, _vp]
        lib.pa_reshape_and_cache_t.restype = _i32
        lib.pa_decode_t.argtypes = [desc] * 6 + [_f32, _i32, _i32, _f32, _f32, _vp, _sz, _vp]
        lib.pa_decode_t.restype = _i32
        dec = [_vp, _vp, _vp, _vp, _vp, _vp, _f32, _i32, _i32, _i32, _i32, _i32, _i32, _i64, _i32, _i32, _i32, _f32,
               _f32]
        lib.pa_decode.argtypes = dec + [_vp, _sz, _vp]
        lib.pa_decode.restype = _i32
        lib.pa_decode_split.argtypes = dec + [_i32, _vp, _sz, _vp]
        lib.pa_decode_split.restype = _i32
        lib.pa_decode_shared_prefix.argtypes = dec + [_vp, _i32, _vp, _sz, _vp]
        lib.pa_decode_shared_prefix.restype = _i32
        lib.pa_decode_append.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _f32, _i32, _i32, _i32,
                                         _i32, _i32, _i32, _i64, _i32, _i32, _i32, _f32, _f32, _vp, _sz, _vp]
        lib.pa_decode_append.restype = _i32
        lib.pa_decode_scratch.argtypes = dec + [_vp]
        lib.pa_decode_scratch.restype = _i32
        lib.pa_decode_scratch_bytes.argtypes = []
        lib.pa_decode_scratch_bytes.restype = _sz
        lib.pa_decode_shared_prefix_workspace_bytes.argtypes = [_i32] * 7
        lib.pa_decode_shared_prefix_workspace_bytes.restype = _sz
        lib.pa_decode_workspace_bytes.argtypes = [_i32] * 7
        lib.pa_decode_workspace_bytes.restype = _sz
        lib.pa_decode_partition_blocks.argtypes = [_i32] * 6
        lib.pa_decode_partition_blocks.restype = _i32
        lib.pa_prefill.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _i32, _i32, _i32, _i32, _i32, _i32, _i64,
                                   _i32, _i32, _i32, _i32, _f32, _f32, _vp]
        lib.pa_prefill.restype = _i32
        lib.pa_copy_blocks.argtypes = [_vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32, _i32, _vp]
        lib.pa_copy_blocks.restype = _i32
        lib.pa_bm_create.argtypes = [_i64, _i32, _i32]
        lib.pa_bm_create.restype = _vp
        lib.pa_bm_destroy.argtypes = [_vp]
        lib.pa_bm_destroy.restype = None
        lib.pa_bm_num_free_blocks.argtypes = [_vp]
        lib.pa_bm_num_free_blocks.restype = _i64
        lib.pa_bm_block_refcount.argtypes = [_vp, _i32]
        lib.pa_bm_block_refcount.restype = _i32
        for name in ("pa_bm_add_sequence", "pa_bm_free_sequence"):
            getattr(lib, name).argtypes = [_vp, _i64]
            getattr(lib, name).restype = _i32
        lib.pa_bm_fork.argtypes = [_vp, _i64, _i64]
        lib.pa_bm_fork.restype = _i32
        lib.pa_bm_append_slots.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp, ctypes.POINTER(_i32)]
        lib.pa_bm_append_slots.restype = _i32
        lib.pa_bm_block_tables.argtypes = [_vp, _vp, _i32, _vp, _i32, _vp]
        lib.pa_bm_block_tables.restype = _i32
        lib.pa_bm_shared_prefix.argtypes = [_vp, _vp, _i32, _i32, _vp, _i32, ctypes.POINTER(_i32)]
        lib.pa_bm_shared_prefix.restype = _i32
        lib.pa_last_error.argtypes = []
        lib.pa_last_error.restype = ctypes.c_char_p
        lib.pa_version.argtypes = []
        lib.pa_version.restype = ctypes.c_char_p
        if path is None:
            _lib = lib
        return lib


def _check(lib, code: int):
    if code != 0:
        raise PAError(code, lib.pa_last_error().decode())


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor, stream=None) -> int | None:
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in PA_DTYPE:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return PA_DTYPE[t.dtype]


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, k_scale: float = 1.0, v_scale: float = 1.0,
                      stream=None) -> None:
    """Write key/value [T, Hkv, D] into caches [N, Hkv, 16, D] at slot_mapping [T] (int32/int64).

    FP8 caches are torch.float8_e4m3fn tensors; k_scale/v_scale are their per-tensor scales.
    """
    lib = load()
    for t in (key, value, k_cache, v_cache, slot_mapping):
        _need(t.is_cuda and t.is_contiguous(), "all tensors must be contiguous device tensors")
    _need(key.dim() == 3 and value.shape == key.shape, "key/value must be [T, Hkv, D] of one shape")
    _need(k_cache.dim() == 4 and v_cache.shape == k_cache.shape, "caches must be [N, Hkv, B, D] of one shape")
    _need(key.dtype == value.dtype and k_cache.dtype == v_cache.dtype, "key/value and the caches must pair dtypes")
    _need(slot_mapping.dim() == 1 and slot_mapping.shape[0] == key.shape[0], "slot_mapping must be [T]")
    _need(slot_mapping.dtype in (torch.int32, torch.int64), "slot_mapping must be int32 or int64")
    T, Hkv, D = key.shape
    N, Hkv2, B, D2 = k_cache.shape
    _need(Hkv2 == Hkv and D2 == D, "cache heads/head_size must match key")
    _check(lib, lib.pa_reshape_and_cache(
        _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping),
        int(slot_mapping.dtype == torch.int64), T, Hkv, D, N, B, _dtype(key), _dtype(k_cache),
        float(k_scale), float(v_scale), _stream(key, stream)))


def reshape_and_cache_t(key, value, k_cache, v_cache, slot_mapping, k_scale: float = 1.0, v_scale: float = 1.0,
                        stream=None) -> None:
    """pa_reshape_and_cache_t: reshape_and_cache with the arrays passed as descriptors (the library checks them)."""
    lib = load()
    ds = [tensor_desc(x) for x in (key, value, k_cache, v_cache, slot_mapping)]
    _check(lib, lib.pa_reshape_and_cache_t(*[ctypes.byref(d) for d in ds], float(k_scale), float(v_scale),
                                           _stream(key, stream)))


def decode_t(out, q, k_cache, v_cache, block_tables, context_lens, scale: float, num_kv_heads: int,
             block_size: int = 16, k_scale: float = 1.0, v_scale: float = 1.0, workspace: torch.Tensor | None = None,
             stream=None) -> torch.Tensor:
    """pa_decode_t: decode with the arrays passed as descriptors (the library checks them)."""
    lib = load()
    ds = [tensor_desc(x) for x in (out, q, k_cache, v_cache, block_tables, context_lens)]
    if workspace is None:
        workspace = workspace_for(q, num_kv_heads, block_tables)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib, lib.pa_decode_t(*[ctypes.byref(d) for d in ds], float(scale), num_kv_heads, block_size,
                                float(k_scale), float(v_scale), _ptr(workspace), ws_bytes, _stream(q, stream)))
    return out


def decode_workspace_bytes(num_seqs: int, num_heads: int, num_kv_heads: int, head_size: int,
                           max_blocks_per_seq: int, block_size: int = 16, partition_blocks: int = 0) -> int:
    lib = load()
    return int(lib.pa_decode_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_size, max_blocks_per_seq,
                                             block_size, partition_blocks))


def decode_partition_blocks(num_seqs: int, num_heads: int, num_kv_heads: int, head_size: int,
                            max_blocks_per_seq: int, block_size: int = 16) -> int:
    lib = load()
    return int(lib.pa_decode_partition_blocks(num_seqs, num_heads, num_kv_heads, head_size, max_blocks_per_seq,
                                              block_size))


def workspace_for(q: torch.Tensor, num_kv_heads: int, block_tables: torch.Tensor, partition_blocks: int = 0,
                  block_size: int = 16) -> torch.Tensor | None:
    """Allocate (with torch) the workspace decode needs for these shapes, or None if none is needed."""
    S, H, D = q.shape
    nbytes = decode_workspace_bytes(S, H, num_kv_heads, D, block_tables.shape[1], block_size, partition_blocks)
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=q.device)  # torch's allocator aligns to >= 512 B


def decode(out, q, k_cache, v_cache, block_tables, context_lens, scale: float, num_kv_heads: int,
           block_size: int = 16, k_scale: float = 1.0, v_scale: float = 1.0, partition_blocks: int = 0,
           workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """One paged decode step: out[S, H, D] = softmax(q K^T scale) V through block_tables [S, M] (int32).

    ``workspace`` may be passed to avoid a torch allocation per call (see
    :func:`workspace_for`). ``partition_blocks`` = 0 lets the library choose.
    """
    lib = load()
    for t in (out, q, k_cache, v_cache, block_tables, context_lens):
        _need(t.is_cuda and t.is_contiguous(), "all tensors must be contiguous device tensors")
    _need(q.dim() == 3 and out.shape == q.shape, "q/out must be [S, H, D] of one shape")
    _need(k_cache.dim() == 4 and v_cache.shape == k_cache.shape and k_cache.dtype == v_cache.dtype,
          "caches must be [N, Hkv, B, D] of one shape and dtype")
    _need(block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32,
          "block_tables and context_lens must be int32")
    S, H, D = q.shape
    _need(block_tables.dim() == 2 and block_tables.shape[0] == S and context_lens.shape == (S,),
          "block_tables must be [S, M] and context_lens [S]")
    N, Hkv, B, D2 = k_cache.shape
    _need(Hkv == num_kv_heads and B == block_size and D2 == D, "cache shape does not match the arguments")
    M = block_tables.shape[1]
    if workspace is None:
        workspace = workspace_for(q, num_kv_heads, block_tables, partition_blocks, block_size)
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib, lib.pa_decode_split(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), float(scale),
        num_kv_heads, block_size, S, H, D, M, N, _dtype(q), _dtype(k_cache), _dtype(out), float(k_scale),
        float(v_scale), int(partition_blocks), ws_ptr, ws_bytes, _stream(q, stream)))
    return out


def decode_scratch_bytes() -> int:
    """Size of the library's fixed scratch array used by :func:`decode_scratch`."""
    return int(load().pa_decode_scratch_bytes())


def decode_scratch(out, q, k_cache, v_cache, block_tables, context_lens, scale: float, num_kv_heads: int,
                   block_size: int = 16, k_scale: float = 1.0, v_scale: float = 1.0, stream=None) -> torch.Tensor:
    """:func:`decode` without a workspace: the library's fixed per-GPU scratch array serves instead, so
    nothing is allocated (pa_decode_scratch). Calls that may overlap on one GPU must be serialised."""
    lib = load()
    for t in (out, q, k_cache, v_cache, block_tables, context_lens):
        _need(t.is_cuda and t.is_contiguous(), "all tensors must be contiguous device tensors")
    _need(q.dim() == 3 and out.shape == q.shape, "q/out must be [S, H, D] of one shape")
    _need(k_cache.dim() == 4 and v_cache.shape == k_cache.shape and k_cache.dtype == v_cache.dtype,
          "caches must be [N, Hkv, B, D] of one shape and dtype")
    _need(block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32,
          "block_tables and context_lens must be int32")
    S, H, D = q.shape
    _need(block_tables.dim() == 2 and block_tables.shape[0] == S and context_lens.shape == (S,),
          "block_tables must be [S, M] and context_lens [S]")
    N, Hkv, B, D2 = k_cache.shape
    _need(Hkv == num_kv_heads and B == block_size and D2 == D, "cache shape does not match the arguments")
    with torch.cuda.device(q.device):
        _check(lib, lib.pa_decode_scratch(
            _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), float(scale),
            num_kv_heads, block_size, S, H, D, block_tables.shape[1], N, _dtype(q), _dtype(k_cache), _dtype(out),
            float(k_scale), float(v_scale), _stream(q, stream)))
    return out


def shared_prefix_workspace_bytes(num_seqs: int, num_heads: int, num_kv_heads: int, head_size: int,
                                  max_blocks_per_seq: int, max_shared_blocks: int, block_size: int = 16) -> int:
    lib = load()
    return int(lib.pa_decode_shared_prefix_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_size,
                                                           max_blocks_per_seq, block_size, max_shared_blocks))


def decode_shared_prefix(out, q, k_cache, v_cache, block_tables, context_lens, scale: float, num_kv_heads: int,
                         prefix_groups, block_size: int = 16, k_scale: float = 1.0, v_scale: float = 1.0,
                         workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """pa_decode where groups of sequences share their first blocks: ``prefix_groups`` is a list of
    (first_seq, num_seqs, shared_blocks) triples (kept on the host); the shared blocks are read once per
    16 / (num_heads / num_kv_heads) sequences of a group. Same result as :func:`decode`."""
    lib = load()
    for t in (out, q, k_cache, v_cache, block_tables, context_lens):
        _need(t.is_cuda and t.is_contiguous(), "all tensors must be contiguous device tensors")
    _need(q.dim() == 3 and out.shape == q.shape, "q/out must be [S, H, D] of one shape")
    _need(k_cache.dim() == 4 and v_cache.shape == k_cache.shape and k_cache.dtype == v_cache.dtype,
          "caches must be [N, Hkv, B, D] of one shape and dtype")
    _need(block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32,
          "block_tables and context_lens must be int32")
    S, H, D = q.shape
    _need(block_tables.dim() == 2 and block_tables.shape[0] == S and context_lens.shape == (S,),
          "block_tables must be [S, M] and context_lens [S]")
    N, Hkv, B, D2 = k_cache.shape
    _need(Hkv == num_kv_heads and B == block_size and D2 == D, "cache shape does not match the arguments")
    M = block_tables.shape[1]
    groups = [tuple(int(x) for x in g) for g in prefix_groups]
    _need(all(len(g) == 3 for g in groups), "prefix_groups must hold (first_seq, num_seqs, shared_blocks) triples")
    flat = (ctypes.c_int32 * max(1, 3 * len(groups)))(*[x for g in groups for x in g])
    if workspace is None:
        max_shared = max([g[2] for g in groups], default=0)
        nbytes = shared_prefix_workspace_bytes(S, H, num_kv_heads, D, M, min(max(max_shared, 0), M), block_size)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib, lib.pa_decode_shared_prefix(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), float(scale),
        num_kv_heads, block_size, S, H, D, M, N, _dtype(q), _dtype(k_cache), _dtype(out), float(k_scale),
        float(v_scale), ctypes.cast(flat, _vp), len(groups), ws_ptr, ws_bytes, _stream(q, stream)))
    return out


def decode_append(out, q, key, value, k_cache, v_cache, slot_mapping, block_tables, context_lens, scale: float,
                  num_kv_heads: int, block_size: int = 16, k_scale: float = 1.0, v_scale: float = 1.0,
                  workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """A whole decode step: write row s of key/value [S, Hkv, D] into slot_mapping[s] (int32 or int64), then
    decode. Same result as :func:`reshape_and_cache` followed by :func:`decode`."""
    lib = load()
    for t in (out, q, key, value, k_cache, v_cache, slot_mapping, block_tables, context_lens):
        _need(t.is_cuda and t.is_contiguous(), "all tensors must be contiguous device tensors")
    _need(q.dim() == 3 and out.shape == q.shape, "q/out must be [S, H, D] of one shape")
    S, H, D = q.shape
    _need(k_cache.dim() == 4 and v_cache.shape == k_cache.shape and k_cache.dtype == v_cache.dtype,
          "caches must be [N, Hkv, B, D] of one shape and dtype")
    N, Hkv, B, D2 = k_cache.shape
    _need(Hkv == num_kv_heads and B == block_size and D2 == D, "cache shape does not match the arguments")
    _need(key.shape == (S, Hkv, D) and value.shape == key.shape and key.dtype == q.dtype and value.dtype == q.dtype,
          "key/value must be [S, Hkv, D] in the query dtype")
    _need(slot_mapping.dtype in (torch.int32, torch.int64) and slot_mapping.shape == (S,),
          "slot_mapping must be int32 or int64 [S]")
    _need(block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == S and context_lens.shape == (S,), "block_tables [S, M] and context_lens [S] int32")
    M = block_tables.shape[1]
    if workspace is None:
        workspace = workspace_for(q, num_kv_heads, block_tables, 0, block_size)
    ws_ptr = _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib, lib.pa_decode_append(
        _ptr(out), _ptr(q), _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping),
        1 if slot_mapping.dtype == torch.int64 else 0, _ptr(block_tables), _ptr(context_lens), float(scale),
        num_kv_heads, block_size, S, H, D, M, N, _dtype(q), _dtype(k_cache), _dtype(out), float(k_scale),
        float(v_scale), ws_ptr, ws_bytes, _stream(q, stream)))
    return out


def copy_blocks(k_cache, v_cache, src_blocks, dst_blocks, stream=None) -> None:
    """Copy physical blocks src_blocks[i] -> dst_blocks[i] (int32 device tensors) in both caches."""
    lib = load()
    for t in (k_cache, v_cache, src_blocks, dst_blocks):
        _need(t.is_cuda and t.is_contiguous(), "all tensors must be contiguous device tensors")
    _need(k_cache.dim() == 4 and v_cache.shape == k_cache.shape and k_cache.dtype == v_cache.dtype,
          "caches must be [N, Hkv, B, D] of one shape and dtype")
    _need(src_blocks.dtype == torch.int32 and dst_blocks.dtype == torch.int32 and src_blocks.dim() == 1
          and dst_blocks.shape == src_blocks.shape, "src/dst blocks must be int32 [n] of one shape")
    N, Hkv, B, D = k_cache.shape
    _check(lib, lib.pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(src_blocks), _ptr(dst_blocks),
                                   src_blocks.shape[0], N, Hkv, D, B, _dtype(k_cache), _stream(k_cache, stream)))


class BlockManager:
    """Host-side block pool bookkeeping (pa_bm_* in include/pa.h): free list, sharing, copy-on-write."""

    def __init__(self, num_blocks: int, max_blocks_per_seq: int, block_size: int = 16):
        self._lib = load()
        self._h = self._lib.pa_bm_create(num_blocks, block_size, max_blocks_per_seq)
        if not self._h:
            raise PAError(3, self._lib.pa_last_error().decode())
        self.num_blocks = num_blocks
        self.max_blocks_per_seq = max_blocks_per_seq
        self.block_size = block_size

    def close(self):
        if self._h:
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def num_free_blocks(self) -> int:
        return int(self._lib.pa_bm_num_free_blocks(self._h))

    def refcount(self, block: int) -> int:
        return int(self._lib.pa_bm_block_refcount(self._h, block))

    def add_sequence(self, seq_id: int) -> None:
        _check(self._lib, self._lib.pa_bm_add_sequence(self._h, seq_id))

    def fork(self, parent: int, child: int) -> None:
        _check(self._lib, self._lib.pa_bm_fork(self._h, parent, child))

    def free_sequence(self, seq_id: int) -> None:
        _check(self._lib, self._lib.pa_bm_free_sequence(self._h, seq_id))

    def append_slots(self, seq_ids):
        """One new token per sequence: returns (slots int64 [n], cow_src int32 [k], cow_dst int32 [k]) as numpy."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        n = len(ids)
        slots = np.empty(n, np.int64)
        src = np.empty(max(n, 1), np.int32)
        dst = np.empty(max(n, 1), np.int32)
        k = _i32(0)
        _check(self._lib, self._lib.pa_bm_append_slots(self._h, ids.ctypes.data, n, slots.ctypes.data,
                                                       src.ctypes.data, dst.ctypes.data, ctypes.byref(k)))
        return slots, src[:k.value].copy(), dst[:k.value].copy()

    def block_tables(self, seq_ids, max_blocks: int | None = None):
        """Dense int32 tables [n, max_blocks] (-1 padded) and int32 lengths [n], as numpy."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        m = max_blocks or self.max_blocks_per_seq
        tables = np.empty((len(ids), m), np.int32)
        lens = np.empty(len(ids), np.int32)
        _check(self._lib, self._lib.pa_bm_block_tables(self._h, ids.ctypes.data, len(ids), tables.ctypes.data, m,
                                                       lens.ctypes.data))
        return tables, lens

    def shared_prefix(self, seq_ids, min_blocks: int = 1, max_groups: int = 16):
        """Shared-prefix groups of the batch listed in this order: [(first index, count, shared blocks), ...]."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        out = np.empty((max(max_groups, 1), 3), np.int32)
        k = _i32(0)
        _check(self._lib, self._lib.pa_bm_shared_prefix(self._h, ids.ctypes.data, len(ids), min_blocks,
                                                        out.ctypes.data, max_groups, ctypes.byref(k)))
        return [tuple(int(x) for x in out[g]) for g in range(k.value)]


def prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale: float, num_kv_heads: int,
            max_query_len: int, block_size: int = 16, k_scale: float = 1.0, v_scale: float = 1.0,
            stream=None) -> torch.Tensor:
    """Chunked-prefill attention: q/out [T, H, D]; query_start_loc int32 [S+1]; causal within each chunk."""
    lib = load()
    for t in (out, q, k_cache, v_cache, block_tables, context_lens, query_start_loc):
        _need(t.is_cuda and t.is_contiguous(), "all tensors must be contiguous device tensors")
    _need(q.dim() == 3 and out.shape == q.shape, "q/out must be [T, H, D] of one shape")
    _need(k_cache.dim() == 4 and v_cache.shape == k_cache.shape and k_cache.dtype == v_cache.dtype,
          "caches must be [N, Hkv, B, D] of one shape and dtype")
    _need(block_tables.dtype == torch.int32 and context_lens.dtype == torch.int32
          and query_start_loc.dtype == torch.int32, "tables, lengths and query_start_loc must be int32")
    S = context_lens.shape[0]
    _need(block_tables.dim() == 2 and block_tables.shape[0] == S and query_start_loc.shape == (S + 1,),
          "block_tables must be [S, M] and query_start_loc [S + 1]")
    T, H, D = q.shape
    N, Hkv, B, D2 = k_cache.shape
    _need(Hkv == num_kv_heads and B == block_size and D2 == D, "cache shape does not match the arguments")
    _check(lib, lib.pa_prefill(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        _ptr(query_start_loc), float(scale), num_kv_heads, block_size, S, H, D, block_tables.shape[1], N,
        int(max_query_len), _dtype(q), _dtype(k_cache), _dtype(out), float(k_scale), float(v_scale),
        _stream(q, stream)))
    return out
