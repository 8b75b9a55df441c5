"""Seeded synthetic inputs for paged-KV-cache decode.

This module draws random numbers and lays out block tables; it computes none of
the method (no attention, no cache writes, no quantisation). Both the HIP path
and the CPU oracle consume what it returns, so it must stay free of the
method's arithmetic.

Shapes follow the pages' setting: fixed 16-token KV blocks scattered through a
shared pool and reached through per-sequence block tables ([vLLM-history]
§3.2); grouped-query heads ([vLLM-note] "内核优化"); physical blocks shared by
sequences with a common prompt prefix ([vLLM-history] §3.2, [vLLM-note]
"前缀缓存"); an FP8 KV cache ([vLLM-history] §5.2).

Draw order inside one ``torch.Generator`` seeded with ``seed``:
1. context lengths (only where they are random);
2. the pool permutation ``randperm(num_blocks)``;
3. q, N(0, 1) float32, rounded (RNE) to the activation dtype;
4. K then V for every context token that is already cached, same recipe;
5. K then V for the new token of every sequence, same recipe.

Blocks are dealt from the permuted pool: first the shared-prefix blocks, then
each sequence's private blocks in sequence order. Everything not dealt is free.
A step appends token ``context_len - 1`` of each sequence (context lengths
count the new token), so the cached tokens are positions 0..context_len-2, and
the slot of the new token still holds poison until the step writes it.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

BLOCK_SIZE = 16

TORCH_DTYPES = {
    "f32": torch.float32,
    "f16": torch.float16,
    "bf16": torch.bfloat16,
    "fp8_e4m3": torch.float8_e4m3fn,
}


@dataclass
class Workload:
    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    num_blocks: int
    dtype: str          # q / key / value activations: "f32" | "f16" | "bf16"
    cache_dtype: str    # dtype or "fp8_e4m3"
    scale: float        # float32-representable softmax scale
    k_scale: float
    v_scale: float
    context_lens: torch.Tensor    # int32 [S], counts the new token
    block_tables: torch.Tensor    # int32 [S, M], -1 past the last used entry
    q: torch.Tensor               # [S, H, D]
    fill_key: torch.Tensor        # [Tf, Hkv, D] already-cached tokens
    fill_value: torch.Tensor
    fill_slots: torch.Tensor      # int64 [Tf], distinct
    new_key: torch.Tensor         # [S, Hkv, D] one new token per sequence
    new_value: torch.Tensor
    new_slots: torch.Tensor       # int64 [S], -1 for a sequence with no tokens
    shared_blocks: int = 0
    sharing_seqs: int = 0         # sequences 0 .. sharing_seqs - 1 share the first shared_blocks blocks
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    def cache_shape(self) -> tuple:
        return (self.num_blocks, self.num_kv_heads, self.block_size, self.head_size)

    def poisoned_cache(self, device="cpu") -> torch.Tensor:
        """A cache whose every slot holds NaN of the cache dtype (never-read data made visible)."""
        return poisoned(self.cache_shape(), self.cache_dtype, device)

    def kv_bytes_per_elem(self) -> int:
        return torch.empty((), dtype=TORCH_DTYPES[self.cache_dtype]).element_size()


def poisoned(shape, cache_dtype: str, device="cpu") -> torch.Tensor:
    if cache_dtype == "fp8_e4m3":
        return torch.full(shape, 0x7F, dtype=torch.uint8, device=device).view(torch.float8_e4m3fn)
    return torch.full(shape, float("nan"), dtype=TORCH_DTYPES[cache_dtype], device=device)


def _randn(gen: torch.Generator, shape, dtype: str) -> torch.Tensor:
    return torch.randn(shape, generator=gen, dtype=torch.float32).to(TORCH_DTYPES[dtype])


def build(name: str, context_lens, num_heads: int, num_kv_heads: int, head_size: int, dtype: str,
          cache_dtype: str | None = None, seed: int = 0, num_blocks: int | None = None,
          free_fraction: float = 0.0, shared_prefix_blocks: int = 0, sharing_seqs: int = 0,
          scale: float | None = None, kv_scale: float = 1.0, block_size: int = BLOCK_SIZE,
          gen: torch.Generator | None = None) -> Workload:
    """Lay out one decode step.

    ``context_lens`` may be a list or a callable ``f(gen) -> list`` (random
    lengths are drawn first). Sequences ``0..sharing_seqs-1`` start with the
    same ``shared_prefix_blocks`` physical blocks; their lengths must exceed
    the prefix so the new token lands in a private block.
    """
    cache_dtype = cache_dtype or dtype
    if gen is None:
        gen = torch.Generator().manual_seed(seed)
    lens = context_lens(gen) if callable(context_lens) else context_lens
    lens = np.asarray([int(x) for x in lens], dtype=np.int64)
    S = len(lens)
    prefix_tokens = shared_prefix_blocks * block_size
    if sharing_seqs and np.any(lens[:sharing_seqs] <= prefix_tokens):
        raise ValueError("a sequence sharing the prefix must extend past it")

    nblk = -(-lens // block_size)
    private = nblk.copy()
    private[:sharing_seqs] -= shared_prefix_blocks
    used = int(private.sum()) + (shared_prefix_blocks if sharing_seqs else 0)
    if num_blocks is None:
        num_blocks = used + math.ceil(used * free_fraction)
    if num_blocks < used:
        raise ValueError("pool too small")

    perm = torch.randperm(num_blocks, generator=gen).numpy().astype(np.int64)
    M = max(1, int(nblk.max()) if S else 1)
    tables = np.full((S, M), -1, dtype=np.int64)
    cursor = 0
    prefix = perm[:shared_prefix_blocks] if sharing_seqs else perm[:0]
    cursor += len(prefix)
    for s in range(S):
        own = perm[cursor:cursor + private[s]]
        cursor += private[s]
        row = np.concatenate([prefix, own]) if s < sharing_seqs else own
        tables[s, :len(row)] = row

    # Slots of every already-cached token (positions 0..len-2), first writer wins
    # for blocks that several sequences share.
    slot_lists = []
    for s in range(S):
        n_cached = max(int(lens[s]) - 1, 0)
        pos = np.arange(n_cached)
        slot_lists.append(tables[s, pos // block_size] * block_size + pos % block_size)
    all_slots = np.concatenate(slot_lists) if slot_lists else np.zeros(0, np.int64)
    _, first = np.unique(all_slots, return_index=True)
    fill_slots = all_slots[np.sort(first)]
    new_slots = np.array(
        [tables[s, (lens[s] - 1) // block_size] * block_size + (lens[s] - 1) % block_size if lens[s] > 0 else -1
         for s in range(S)], dtype=np.int64)

    q = _randn(gen, (S, num_heads, head_size), dtype)
    Tf = len(fill_slots)
    fill_key = _randn(gen, (Tf, num_kv_heads, head_size), dtype)
    fill_value = _randn(gen, (Tf, num_kv_heads, head_size), dtype)
    new_key = _randn(gen, (S, num_kv_heads, head_size), dtype)
    new_value = _randn(gen, (S, num_kv_heads, head_size), dtype)

    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(head_size)))
    fp8 = cache_dtype == "fp8_e4m3"
    return Workload(
        name=name, num_seqs=S, num_heads=num_heads, num_kv_heads=num_kv_heads, head_size=head_size,
        block_size=block_size, num_blocks=num_blocks, dtype=dtype, cache_dtype=cache_dtype,
        scale=float(np.float32(scale)), k_scale=float(np.float32(kv_scale)) if fp8 else 1.0,
        v_scale=float(np.float32(kv_scale)) if fp8 else 1.0,
        context_lens=torch.from_numpy(lens.astype(np.int32)),
        block_tables=torch.from_numpy(tables.astype(np.int32)),
        q=q, fill_key=fill_key, fill_value=fill_value, fill_slots=torch.from_numpy(fill_slots),
        new_key=new_key, new_value=new_value, new_slots=torch.from_numpy(new_slots),
        shared_blocks=shared_prefix_blocks if sharing_seqs else 0,
        sharing_seqs=sharing_seqs if shared_prefix_blocks else 0, seed=seed,
        meta={"used_blocks": used},
    )


# --- the five named workloads -------------------------------------------------

def tiny_fp32(seed: int = 1) -> Workload:
    """4 sequences, contexts {1, 17, 100, 255}, 8 heads = 8 KV heads, head 64, fp32, pool of 64 blocks."""
    return build("tiny_fp32", [1, 17, 100, 255], 8, 8, 64, "f32", seed=seed, num_blocks=64)


def llama7b_mha_fp16(seed: int = 2) -> Workload:
    """Llama-2-7B-shaped MHA: 32 sequences x 2048 tokens, 32 heads, head 128, fp16, pool 4608 blocks."""
    return build("llama7b_mha_fp16_b32_ctx2048", [2048] * 32, 32, 32, 128, "f16", seed=seed, num_blocks=4608)


def llama3_8b_gqa_bf16(seed: int = 3) -> Workload:
    """Llama-3-8B-shaped GQA, ragged: 64 sequences, lengths U{16..4096}, 32/8 heads, bf16, +10% free blocks."""
    return build("llama3_8b_gqa_bf16_ragged_b64",
                 lambda g: torch.randint(16, 4097, (64,), generator=g).tolist(),
                 32, 8, 128, "bf16", seed=seed, free_fraction=0.10)


def longctx_bf16(seed: int = 4) -> Workload:
    """Long context: 8 sequences x 32768 tokens, 64/8 heads, bf16, pool of 16384 blocks (none free)."""
    return build("longctx_bf16_b8_ctx32768", [32768] * 8, 64, 8, 128, "bf16", seed=seed, num_blocks=16384)


def prefix_fp8(seed: int = 5) -> Workload:
    """256 sequences, fp8 E4M3 cache (scale 0.05), bf16 queries, 32/8 heads.

    Sequences 0..127 share one 1024-token prefix (64 physical blocks) and add a
    private tail of U{16..2048} tokens; sequences 128..255 hold U{16..3072}
    private tokens. Pool = blocks in use + 10% free.
    """
    def lengths(g):
        tails = torch.randint(16, 2049, (128,), generator=g)
        priv = torch.randint(16, 3073, (128,), generator=g)
        return (1024 + tails).tolist() + priv.tolist()
    return build("prefix_fp8_b256", lengths, 32, 8, 128, "bf16", cache_dtype="fp8_e4m3", seed=seed,
                 free_fraction=0.10, shared_prefix_blocks=64, sharing_seqs=128, kv_scale=0.05)


def prefix_long_fp8(seed: int = 6) -> Workload:
    """Long shared prompt: 256 sequences share one 4096-token prefix (256 physical blocks) and add private
    tails of U{16..512} tokens; fp8 E4M3 cache (scale 0.05), bf16 queries, 32/8 heads, pool + 10% free.
    Not one of the five reference shapes: it measures the shared-prefix pass where the prefix dominates."""
    def lengths(g):
        return (4096 + torch.randint(16, 513, (256,), generator=g)).tolist()
    return build("prefix_long_fp8_b256", lengths, 32, 8, 128, "bf16", cache_dtype="fp8_e4m3", seed=seed,
                 free_fraction=0.10, shared_prefix_blocks=256, sharing_seqs=256, kv_scale=0.05)


def mqa_bf16(group: int, seed: int = 7) -> Workload:
    """Multi-query decode ([vLLM-note] "内核优化": GQA/MQA kernels): one KV head shared by ``group`` query heads;
    64 sequences x 32768 tokens, head 128, bf16 (1 GiB of K/V, as the Llama-2-7B-shaped batch), pool with no
    free blocks. Not one of the five reference shapes: it measures large query groups."""
    return build(f"mqa_g{group}_bf16_b64_ctx32768", [32768] * 64, group, 1, 128, "bf16", seed=seed,
                 num_blocks=64 * 2048)


NAMED = {
    "tiny_fp32": tiny_fp32,
    "llama7b_mha_fp16": llama7b_mha_fp16,
    "llama3_8b_gqa_bf16": llama3_8b_gqa_bf16,
    "longctx_bf16": longctx_bf16,
    "prefix_fp8": prefix_fp8,
    "prefix_long_fp8": prefix_long_fp8,
    "mqa_g32_bf16": lambda seed=7: mqa_bf16(32, seed),
    "mqa_g64_bf16": lambda seed=7: mqa_bf16(64, seed),
    "mqa_g128_bf16": lambda seed=7: mqa_bf16(128, seed),
}


def named(name: str, seed: int | None = None) -> Workload:
    fn = NAMED[name]
    return fn() if seed is None else fn(seed)


def algorithmic_kv_bytes(w: Workload, unique: bool = False) -> int:
    """Bytes of K and V the decode must read: sum over sequences of ctx * Hkv * D * 2 * elem.

    With ``unique`` the shared-prefix tokens are counted once (the lower bound
    on HBM traffic when the shared blocks stay in cache).
    """
    per_tok = w.num_kv_heads * w.head_size * 2 * w.kv_bytes_per_elem()
    toks = int(w.context_lens.to(torch.int64).sum())
    if unique and w.shared_blocks:
        sharing = int((w.block_tables[:, :w.shared_blocks] == w.block_tables[0, :w.shared_blocks]).all(1).sum())
        toks -= (sharing - 1) * w.shared_blocks * w.block_size
    return toks * per_tok


def algorithmic_step_bytes(w: Workload, unique: bool = False) -> int:
    """KV bytes plus q, out, block table, context lengths, and the appended token (read + write)."""
    act = torch.empty((), dtype=TORCH_DTYPES[w.dtype]).element_size()
    qo = 2 * w.num_seqs * w.num_heads * w.head_size * act
    table = w.block_tables.numel() * 4 + w.num_seqs * 4
    appended = int((w.new_slots >= 0).sum()) * w.num_kv_heads * w.head_size * 2 * (act + w.kv_bytes_per_elem())
    return algorithmic_kv_bytes(w, unique) + qo + table + appended
