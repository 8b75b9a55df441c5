"""The seeded input generator lays out what the decode shapes describe (no GPU)."""

import numpy as np
import pytest
import torch

from paged_kv_cache_380_amd import workloads as wl


def check_layout(w: wl.Workload):
    S, M = w.block_tables.shape
    lens = w.context_lens.numpy()
    t = w.block_tables.numpy()
    nb = -(-lens // 16)
    used = []
    for s in range(S):
        assert (t[s, :nb[s]] >= 0).all() and (t[s, :nb[s]] < w.num_blocks).all()
        assert (t[s, nb[s]:] == -1).all()
        used.append(t[s, :nb[s]])
    allb = np.concatenate(used) if used else np.zeros(0, int)
    uniq, counts = np.unique(allb, return_counts=True)
    shared = set(t[0, :w.shared_blocks]) if w.shared_blocks else set()
    for b, c in zip(uniq, counts):  # only the shared prefix blocks appear in more than one table
        assert c == 1 or b in shared
    # cached-token slots are distinct, inside the pool, and are exactly positions 0..len-2
    fs = w.fill_slots.numpy()
    assert len(np.unique(fs)) == len(fs)
    expect = set()
    for s in range(S):
        for p in range(max(lens[s] - 1, 0)):
            expect.add(int(t[s, p // 16]) * 16 + p % 16)
    assert set(fs.tolist()) == expect
    for s in range(S):
        if lens[s]:
            p = lens[s] - 1
            assert w.new_slots[s] == t[s, p // 16] * 16 + p % 16
            assert int(w.new_slots[s]) not in expect
        else:
            assert w.new_slots[s] == -1
    assert w.fill_key.shape == (len(fs), w.num_kv_heads, w.head_size)
    assert w.q.shape == (S, w.num_heads, w.head_size)


def test_tiny_fp32():
    w = wl.tiny_fp32()
    check_layout(w)
    assert w.context_lens.tolist() == [1, 17, 100, 255]
    assert w.num_blocks == 64 and w.meta["used_blocks"] == 26 and w.max_blocks_per_seq == 16
    assert w.q.dtype == torch.float32 and w.scale == np.float32(0.125)


def test_seed_determinism_and_draw_order():
    a, b = wl.tiny_fp32(seed=7), wl.tiny_fp32(seed=7)
    assert torch.equal(a.block_tables, b.block_tables) and torch.equal(a.fill_key, b.fill_key)
    c = wl.tiny_fp32(seed=8)
    assert not torch.equal(a.block_tables, c.block_tables)
    # draw order: lengths, permutation, q, cached K, cached V, new K, new V
    g = torch.Generator().manual_seed(7)
    perm = torch.randperm(64, generator=g)
    assert a.block_tables[0, 0] == perm[0]
    q = torch.randn(a.q.shape, generator=g)
    assert torch.equal(a.q, q)


def test_ragged_gqa_shape():
    w = wl.llama3_8b_gqa_bf16()
    check_layout(w)
    lens = w.context_lens.numpy()
    assert w.num_seqs == 64 and lens.min() >= 16 and lens.max() <= 4096
    used = int((-(-lens // 16)).sum())
    assert w.num_blocks == used + -(-used // 10)
    assert w.group == 4 and w.q.dtype == torch.bfloat16


def test_prefix_sharing_fp8_shape():
    w = wl.prefix_fp8()
    check_layout(w)
    lens = w.context_lens.numpy()
    t = w.block_tables.numpy()
    assert w.shared_blocks == 64
    assert (t[:128, :64] == t[0, :64]).all()
    assert ((lens[:128] >= 1024 + 16) & (lens[:128] <= 1024 + 2048)).all()
    assert ((lens[128:] >= 16) & (lens[128:] <= 3072)).all()
    assert not np.isin(t[128:][t[128:] >= 0], t[0, :64]).any()
    assert w.cache_dtype == "fp8_e4m3" and w.k_scale == np.float32(0.05)
    assert wl.algorithmic_kv_bytes(w, unique=True) == wl.algorithmic_kv_bytes(w) - 127 * 1024 * 8 * 128 * 2


def test_small_edge_layouts():
    w = wl.build("edge", [0, 1, 16, 17, 0], 6, 3, 64, "f16", seed=3, free_fraction=0.2)
    check_layout(w)
    assert w.new_slots[0] == -1 and w.new_slots[4] == -1
    assert w.max_blocks_per_seq == 2


@pytest.mark.parametrize("name", ["llama7b_mha_fp16", "longctx_bf16"])
def test_uniform_configs_tables_only(name, monkeypatch):
    # Only the layout (no K/V draws): replace randn by zeros of the right shape.
    monkeypatch.setattr(wl, "_randn", lambda g, shape, dtype: torch.zeros(shape, dtype=wl.TORCH_DTYPES[dtype]))
    w = wl.named(name)
    check_layout(w)
    if name == "llama7b_mha_fp16":
        assert w.num_blocks == 4608 and w.meta["used_blocks"] == 4096
        assert wl.algorithmic_kv_bytes(w) == 1024 ** 3
    else:
        assert w.num_blocks == 16384 and w.meta["used_blocks"] == 16384
        assert wl.algorithmic_kv_bytes(w) == 1024 ** 3


@pytest.mark.parametrize("make,sharing,blocks", [(wl.prefix_fp8, 128, 64), (wl.prefix_long_fp8, 256, 256)])
def test_shared_prefix_group_is_what_the_tables_hold(make, sharing, blocks):
    # The group bench.py and the tests pass to pa_decode_shared_prefix, (0, sharing_seqs, shared_blocks), must
    # be true of the tables: those sequences agree on their first shared_blocks entries, every one of them
    # holds more than that many blocks' worth of tokens, and no other sequence touches those blocks.
    w = make()
    assert (w.sharing_seqs, w.shared_blocks) == (sharing, blocks)
    t = w.block_tables.numpy()
    lens = w.context_lens.numpy()
    assert (t[:sharing, :blocks] == t[0, :blocks]).all()
    assert (lens[:sharing] > blocks * 16).all()
    others = t[sharing:]
    assert not np.isin(others, t[0, :blocks]).any()
    check_layout(w)


def test_no_group_without_sharing():
    w = wl.llama3_8b_gqa_bf16()
    assert (w.sharing_seqs, w.shared_blocks) == (0, 0)
