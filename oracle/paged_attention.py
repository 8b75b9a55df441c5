"""fp64 CPU oracle of the two paged-KV-cache operations (test infrastructure).

Storage conventions, shared with the HIP side only through the data itself:

* dtype names: "f32", "f16", "bf16" (activations and caches) and "fp8_e4m3"
  (caches only);
* raw arrays: f32 -> numpy.float32, f16 -> numpy.float16, bf16 -> numpy.uint16
  holding the bf16 bit patterns, fp8_e4m3 -> numpy.uint8 holding the codes;
* a K or V cache is one array of shape [num_blocks, num_kv_heads, block_size,
  head_size]: every (block, kv head) pair owns block_size contiguous token rows;
* a slot is physical_block * block_size + offset_in_block.

Readings taken where the pages are silent (each also listed in the design
notes): the cache layout above; the block table is a dense int32 array
[num_seqs, max_blocks] (the note page calls a request's pages a linked list,
the history page a block table; the dense table is the plainest form of both);
query head h reads KV head h // (num_heads / num_kv_heads); a context length of
zero gives an all-zero output; the query attends to every one of its
context_len tokens, the newest included (no causal mask inside a decode step);
``scale`` and the FP8 scales are float32 numbers, used here exactly, widened to
float64.
"""

from __future__ import annotations

import numpy as np

from .e4m3 import e4m3_decode, e4m3_encode

DTYPES = ("f32", "f16", "bf16", "fp8_e4m3")
_RAW = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8_e4m3": np.uint8}


def _check_raw(a: np.ndarray, dtype: str) -> None:
    if dtype not in _RAW:
        raise ValueError(f"unknown dtype {dtype!r}")
    if a.dtype != _RAW[dtype]:
        raise TypeError(f"{dtype} data must be stored as {np.dtype(_RAW[dtype])}, got {a.dtype}")


def widen(raw: np.ndarray, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Exact float64 value of raw storage.

    FP8 codes are multiplied by the float32 ``scale`` (the per-tensor
    dequantisation scale); for the other dtypes ``scale`` must be 1.
    """
    raw = np.asarray(raw)
    _check_raw(raw, dtype)
    if dtype == "bf16":
        # A bf16 number is the top half of the float32 with the same bits.
        return (raw.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "fp8_e4m3":
        return e4m3_decode(raw) * float(np.float32(scale))
    if scale != 1.0:
        raise ValueError("a scale only applies to fp8 data")
    return raw.astype(np.float64)


def quantize_for_cache(x_raw: np.ndarray, src_dtype: str, cache_dtype: str, scale: float = 1.0) -> np.ndarray:
    """What reshape-and-cache stores for activations ``x_raw``.

    Same dtype: the bits are copied. FP8 cache ([vLLM-history] §5.2): the value
    is widened to float32 (exact), its magnitude divided by the float32 scale
    with one correctly rounded float32 division, the input's sign bit put back
    (so a NaN keeps its sign too; for every other input this equals x / scale),
    and the quotient encoded to E4M3 (RNE, saturating).
    """
    _check_raw(x_raw, src_dtype)
    if cache_dtype == src_dtype:
        return np.array(x_raw, copy=True)
    if cache_dtype != "fp8_e4m3" or src_dtype == "fp8_e4m3":
        raise ValueError(f"cannot store {src_dtype} activations in a {cache_dtype} cache")
    if src_dtype in ("f16", "bf16"):
        # The stored code is a function of the input's 16 bits alone: evaluate it once for each of the 65536
        # bit patterns and look every element up (the same values as encoding element by element, without
        # float64 temporaries the size of a whole cache).
        patterns = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        table = _quantize_e4m3(patterns if src_dtype == "bf16" else patterns.view(np.float16), src_dtype, scale)
        return table[np.asarray(x_raw).view(np.uint16)]
    return _quantize_e4m3(x_raw, src_dtype, scale)


def _quantize_e4m3(x_raw: np.ndarray, src_dtype: str, scale: float) -> np.ndarray:
    """E4M3 code of each element: float32 widening, |x| / scale in float32, sign put back, then encode."""
    x32 = widen(x_raw, src_dtype).astype(np.float32)  # exact: every source dtype fits in float32
    with np.errstate(invalid="ignore", over="ignore"):
        y = np.copysign(np.divide(np.abs(x32), np.float32(scale), dtype=np.float32), x32)
    return e4m3_encode(y)


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, block_size, src_dtype, cache_dtype,
                      k_scale=1.0, v_scale=1.0) -> None:
    """Scatter new tokens' K and V into their cache slots, in place.

    [vLLM-note] "PagedAttention": the page holding a token is its slot divided
    by the block size, the row inside the page is the remainder. A negative slot
    means the token is padding and is skipped. key/value: [T, num_kv_heads,
    head_size]; caches: [num_blocks, num_kv_heads, block_size, head_size].
    Slots must be distinct (two writers of one slot have no defined winner).
    """
    slots = np.asarray(slot_mapping).astype(np.int64)
    _check_raw(k_cache, cache_dtype)
    _check_raw(v_cache, cache_dtype)
    valid = slots >= 0
    if len(np.unique(slots[valid])) != int(valid.sum()):
        raise ValueError("duplicate slots in one reshape_and_cache call")
    blocks = slots[valid] // block_size
    offsets = slots[valid] % block_size
    if blocks.size and blocks.max() >= k_cache.shape[0]:
        raise IndexError("slot beyond the cache")
    k_cache[blocks, :, offsets, :] = quantize_for_cache(np.asarray(key)[valid], src_dtype, cache_dtype, k_scale)
    v_cache[blocks, :, offsets, :] = quantize_for_cache(np.asarray(value)[valid], src_dtype, cache_dtype, v_scale)


def decode_attention(q, k_cache, v_cache, block_tables, context_lens, scale, num_kv_heads, block_size,
                     q_dtype, cache_dtype, k_scale=1.0, v_scale=1.0, seqs=None) -> np.ndarray:
    """Decode attention over a paged cache, in float64. Returns [num_seqs, num_heads, head_size].

    For sequence s with n = context_lens[s] tokens, token position p lives in
    physical block block_tables[s, p // block_size], row p % block_size
    ([vLLM-history] §3.2; [vLLM-note] "PagedAttention"). Query head h reads KV
    head h // G with G = num_heads / num_kv_heads (grouped-query attention,
    [vLLM-note] "内核优化"). The output is softmax(K q · scale) weighted V
    (Vaswani et al., eq. 1, one query row), evaluated with the row maximum
    subtracted before exp. n = 0 gives zeros. Only the n addressed token rows
    are ever read. ``seqs`` limits the work to a subset of sequences (the
    others stay zero).
    """
    q = np.asarray(q)
    S, H, D = q.shape
    if H % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    group = H // num_kv_heads
    scale64 = float(np.float32(scale))
    k_scale = k_scale if cache_dtype == "fp8_e4m3" else 1.0
    v_scale = v_scale if cache_dtype == "fp8_e4m3" else 1.0
    out = np.zeros((S, H, D), dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        n = int(context_lens[s])
        if n == 0:
            continue
        pos = np.arange(n)
        phys = np.asarray(block_tables[s], dtype=np.int64)[pos // block_size]
        rows = pos % block_size
        keys = widen(k_cache[phys, :, rows, :], cache_dtype, k_scale)    # [n, num_kv_heads, D]
        values = widen(v_cache[phys, :, rows, :], cache_dtype, v_scale)  # [n, num_kv_heads, D]
        qs = widen(q[s], q_dtype)                                        # [H, D]
        for h in range(H):
            kv = h // group
            logits = scale64 * (keys[:, kv, :] @ qs[h])
            weights = np.exp(logits - logits.max())
            out[s, h] = (weights @ values[:, kv, :]) / weights.sum()
    return out


def copy_blocks(k_cache, v_cache, src_blocks, dst_blocks) -> None:
    """Copy-on-write step, in place: block dst[i] becomes a copy of block src[i] in both caches.

    [vLLM-history] §3.2: before a sequence writes into a physical block that
    other sequences share, the block is copied and the sequence continues in
    the copy. Destinations must be distinct and disjoint from the sources
    (the GPU copies run concurrently, so an overlap would have no defined order).
    """
    src = np.asarray(src_blocks, dtype=np.int64)
    dst = np.asarray(dst_blocks, dtype=np.int64)
    if src.shape != dst.shape:
        raise ValueError("src and dst must pair up")
    if len(np.unique(dst)) != len(dst) or np.intersect1d(src, dst).size:
        raise ValueError("destinations must be distinct and disjoint from the sources")
    k_cache[dst] = k_cache[src]
    v_cache[dst] = v_cache[src]


def prefill_attention(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale, num_kv_heads,
                      block_size, q_dtype, cache_dtype, k_scale=1.0, v_scale=1.0) -> np.ndarray:
    """Chunked-prefill attention over a paged cache, in float64. Returns [num_tokens, num_heads, head_size].

    [vLLM-history] §5.4 and §7.3 (chunked prefill: a long prompt is cut into
    chunks that run next to decode steps). Sequence s contributes the query
    rows query_start_loc[s] .. query_start_loc[s+1]-1, the last q_len of its
    context_lens[s] tokens, whose K and V are already in the cache. Query i of
    the chunk sits at position p = context_lens[s] - q_len + i and attends to
    the cached tokens 0..p (causal), reached through the block table as in
    decode_attention: softmax(K q . scale) weighted V over those tokens.
    """
    q = np.asarray(q)
    T, H, D = q.shape
    if H % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    starts = np.asarray(query_start_loc, dtype=np.int64)
    group = H // num_kv_heads
    scale64 = float(np.float32(scale))
    k_scale = k_scale if cache_dtype == "fp8_e4m3" else 1.0
    v_scale = v_scale if cache_dtype == "fp8_e4m3" else 1.0
    out = np.zeros((T, H, D), dtype=np.float64)
    for s in range(len(starts) - 1):
        q0, q1 = int(starts[s]), int(starts[s + 1])
        n = int(context_lens[s])
        qlen = q1 - q0
        if qlen == 0:
            continue
        if qlen > n:
            raise ValueError("a chunk cannot be longer than its context")
        pos = np.arange(n)
        phys = np.asarray(block_tables[s], dtype=np.int64)[pos // block_size]
        rows = pos % block_size
        keys = widen(k_cache[phys, :, rows, :], cache_dtype, k_scale)    # [n, num_kv_heads, D]
        values = widen(v_cache[phys, :, rows, :], cache_dtype, v_scale)
        for i in range(qlen):
            p = n - qlen + i                                             # this query's position
            qs = widen(q[q0 + i], q_dtype)                               # [H, D]
            for h in range(H):
                kv = h // group
                logits = scale64 * (keys[:p + 1, kv, :] @ qs[h])
                weights = np.exp(logits - logits.max())
                out[q0 + i, h] = (weights @ values[:p + 1, kv, :]) / weights.sum()
    return out
