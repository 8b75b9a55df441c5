"""Parity of pa_decode_shared_prefix with the fp64 oracle and with pa_decode.

Sequences that share a prompt prefix hold the same physical blocks at the
start of their block tables ("vLLM 前世今生" §3.2). pa_decode_shared_prefix
reads those blocks once per 16 query columns (16 / group sequences of one
group) in a pass of its own, streams only the rest of every sequence in the
balanced schedule, and merges the two. The result must be pa_decode's: it is
checked against the oracle (at the usual tolerance) and against pa_decode at
1e-4, far tighter than the FP8 tolerance, so a wrong weight or a block read
twice or never cannot hide. Cases: groups anywhere in the batch (sequences
reordered), groups whose size is not a multiple of the sequences per tile,
16 / 8 / 4 query heads per KV head (1, 2 and 4 sequences per tile), shared
prefixes that are not a multiple of the pass's parts (64 blocks, or 256 and
512 where the call has the sequences to keep 512 workgroups), a group named
shorter than the blocks its members really share, single-sequence groups
whose private part is empty or only a masked tail, FP8, bf16 and f16 caches,
head size 64, and the prefix-sharing FP8 batch at full size.
"""

import dataclasses

import numpy as np
import pytest
import torch

from paged_kv_cache_380_amd import workloads as wl
from pa_testlib import GpuCase, oracle_decode, oracle_fill, tolerance

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_380_amd import binding
    binding.load()
    yield
    torch.cuda.synchronize()


def reorder(w: wl.Workload, order) -> wl.Workload:
    """The same batch with its sequences in another order (cache contents unchanged)."""
    idx = torch.as_tensor(order, dtype=torch.long)
    return dataclasses.replace(w, context_lens=w.context_lens[idx].clone(), block_tables=w.block_tables[idx].clone(),
                               q=w.q[idx].clone(), new_key=w.new_key[idx].clone(),
                               new_value=w.new_value[idx].clone(), new_slots=w.new_slots[idx].clone())


def run_both(w: wl.Workload, groups, out_dtype=torch.float32):
    """(shared-prefix output, pa_decode output, oracle) for one appended step."""
    from paged_kv_cache_380_amd import binding
    case = GpuCase(w)
    case.append()
    ref_gpu = case.decode(out_dtype=out_dtype)
    out = torch.full(case.q.shape, float("nan"), dtype=out_dtype, device="cuda")
    binding.decode_shared_prefix(out, case.q, case.kc, case.vc, case.tables, case.lens, w.scale, w.num_kv_heads,
                                 groups, w.block_size, w.k_scale, w.v_scale)
    torch.cuda.synchronize()
    kc, vc = oracle_fill(w)
    return out, ref_gpu, oracle_decode(w, kc, vc)


def check(w, groups, out_dtype=torch.float32):
    out, ref_gpu, ref = run_both(w, groups, out_dtype)
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    if out_dtype != torch.float32:
        return out  # a 16-bit output is gated through the float32 one (its rounding can exceed the tolerance)
    err = float(np.abs(got - ref).max())
    assert err <= tolerance(w), f"{w.name} {groups}: max|err| vs oracle = {err}"
    diff = float((out.float() - ref_gpu.float()).abs().max())
    assert diff <= 1e-4, f"{w.name} {groups}: max|diff| vs pa_decode = {diff}"
    return out


def sharing(name, H, Hkv, D, dtype, cache, shared, tails, private, seed, kv_scale=0.05):
    """sequences 0..len(tails)-1 share `shared` blocks, then own `tails` tokens; then private sequences."""
    lens = [shared * 16 + t for t in tails] + list(private)
    return wl.build(name, lens, H, Hkv, D, dtype, cache_dtype=cache, seed=seed, free_fraction=0.1,
                    shared_prefix_blocks=shared, sharing_seqs=len(tails), kv_scale=kv_scale)


@pytest.mark.parametrize("H,Hkv,dtype,cache", [(32, 8, "bf16", "fp8_e4m3"), (32, 8, "bf16", "bf16"),
                                               (16, 2, "f16", "f16"), (16, 1, "bf16", "bf16"),
                                               (16, 2, "f16", "fp8_e4m3"), (16, 1, "bf16", "fp8_e4m3")])
def test_group_in_the_middle(H, Hkv, dtype, cache):
    # 7 sharing sequences (not a multiple of 4 or 2) between private ones; 75 shared blocks (2 parts, the
    # second of 11 blocks); tails from one token to several ranges
    rng = np.random.default_rng(11)
    tails = [1, 15, 16, 17, 300, 2000, int(rng.integers(1, 900))]
    private = [int(rng.integers(1, 1500)) for _ in range(9)]
    w = sharing("shared_mid", H, Hkv, 128, dtype, cache, 75, tails, private, seed=21)
    order = list(range(7, 12)) + list(range(7)) + list(range(12, 16))
    check(reorder(w, order), [(5, 7, 75)])


def test_group_named_shorter_and_split():
    # 12 sequences share 40 blocks; the call names two groups of them, one with 33 shared blocks
    # (fewer than really shared: still equal entries) and one with 40, and a private batch after
    rng = np.random.default_rng(12)
    w = sharing("shared_split", 32, 8, 128, "bf16", "fp8_e4m3", 40,
                [int(rng.integers(1, 700)) for _ in range(12)], [int(rng.integers(1, 3000)) for _ in range(20)],
                seed=22)
    check(w, [(0, 5, 33), (5, 7, 40)])


def test_single_sequence_groups():
    # a group of one: its own first blocks. Context exactly the shared blocks (nothing past them), a
    # masked tail just past them, and many private blocks after them.
    w = wl.build("shared_single", [64, 64 + 3, 48, 16 * 70 + 9, 16 * 70 + 9, 200], 32, 8, 128, "bf16", seed=23,
                 free_fraction=0.1)
    check(w, [(0, 1, 4), (1, 1, 4), (2, 1, 3), (3, 1, 70), (4, 1, 5)])


@pytest.mark.parametrize("cache", ["fp8_e4m3", "f16"])
def test_head_size_64_other_caches(cache):
    rng = np.random.default_rng(17)
    dtype = "f16" if cache == "f16" else "bf16"
    w = sharing("shared_d64_" + cache, 32, 8, 64, dtype, cache, 40, [int(rng.integers(1, 700)) for _ in range(13)],
                [int(rng.integers(1, 900)) for _ in range(5)], seed=29)
    check(reorder(w, list(range(13, 15)) + list(range(13)) + list(range(15, 18))), [(2, 13, 40)])


def test_head_size_64_and_native_output():
    rng = np.random.default_rng(13)
    w = sharing("shared_d64", 16, 4, 64, "bf16", "bf16", 18, [int(rng.integers(1, 500)) for _ in range(10)],
                [int(rng.integers(1, 800)) for _ in range(6)], seed=24)
    out32 = check(w, [(0, 10, 18)])
    out16 = check(w, [(0, 10, 18)], out_dtype=torch.bfloat16)
    # the native output is the float32 result rounded to nearest-even
    assert torch.equal(out16, out32.to(torch.bfloat16))


def test_deterministic():
    from paged_kv_cache_380_amd import binding
    rng = np.random.default_rng(14)
    w = sharing("shared_det", 32, 8, 128, "bf16", "fp8_e4m3", 30, [int(rng.integers(1, 600)) for _ in range(9)],
                [int(rng.integers(1, 600)) for _ in range(9)], seed=25)
    case = GpuCase(w)
    case.append()
    outs = []
    for _ in range(2):
        out = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")
        binding.decode_shared_prefix(out, case.q, case.kc, case.vc, case.tables, case.lens, w.scale,
                                     w.num_kv_heads, [(0, 9, 30)], w.block_size, w.k_scale, w.v_scale)
        outs.append(out)
    assert torch.equal(outs[0], outs[1])


def test_groups_ignored_where_the_pass_does_not_apply():
    # 6 query heads per KV head (no 16-column tile of whole sequences) and MHA: the groups change nothing
    rng = np.random.default_rng(15)
    for H, Hkv in [(12, 2), (8, 8)]:
        w = sharing(f"shared_na_{H}_{Hkv}", H, Hkv, 128, "bf16", "bf16", 10,
                    [int(rng.integers(1, 300)) for _ in range(5)], [40, 77], seed=26)
        check(w, [(0, 5, 10)])


def test_prefix_fp8_full_size():
    w = wl.prefix_fp8()
    assert w.sharing_seqs == 128 and w.shared_blocks == 64
    check(w, [(0, w.sharing_seqs, w.shared_blocks)])


def test_prefix_long_fp8_full_size_sampled():
    # 256 sequences on one 4096-token prefix: every sequence against pa_decode, sampled ones against the oracle
    from paged_kv_cache_380_amd import binding
    w = wl.prefix_long_fp8()
    case = GpuCase(w)
    case.append()
    ref_gpu = case.decode(out_dtype=torch.float32)
    out = torch.full(case.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    binding.decode_shared_prefix(out, case.q, case.kc, case.vc, case.tables, case.lens, w.scale, w.num_kv_heads,
                                 [(0, w.sharing_seqs, w.shared_blocks)], w.block_size, w.k_scale, w.v_scale)
    torch.cuda.synchronize()
    assert float((out - ref_gpu).abs().max()) <= 1e-4
    seqs = [0, 1, 77, 128, 255]
    kc, vc = oracle_fill(w)
    ref = oracle_decode(w, kc, vc, seqs=seqs)
    got = out.cpu().numpy()[seqs]
    assert float(np.abs(got - ref[seqs]).max()) <= tolerance(w)  # the oracle fills only the sampled rows


@pytest.mark.parametrize("seqs,shared", [(256, 600), (128, 300)])
def test_long_parts(seqs, shared):
    # Parts longer than 64 blocks, where the call still gives 512 workgroups: 256 sequences (64 tiles of 4
    # per KV head) on 600 shared blocks take parts of 512 (the second of 88 blocks); 128 sequences on 300
    # take parts of 256 (the second of 44). Every sequence against pa_decode, sampled ones against the oracle.
    from paged_kv_cache_380_amd import binding
    rng = np.random.default_rng(31 + seqs)
    w = sharing(f"shared_long_parts_{seqs}", 32, 8, 128, "bf16", "fp8_e4m3", shared,
                [int(rng.integers(1, 100)) for _ in range(seqs)], [], seed=33)
    case = GpuCase(w)
    case.append()
    ref_gpu = case.decode(out_dtype=torch.float32)
    out = torch.full(case.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    binding.decode_shared_prefix(out, case.q, case.kc, case.vc, case.tables, case.lens, w.scale, w.num_kv_heads,
                                 [(0, seqs, shared)], w.block_size, w.k_scale, w.v_scale)
    torch.cuda.synchronize()
    assert float((out - ref_gpu).abs().max()) <= 1e-4
    sample = [0, 3, seqs // 2 + 1, seqs - 1]
    kc, vc = oracle_fill(w)
    ref = oracle_decode(w, kc, vc, seqs=sample)
    assert float(np.abs(out.cpu().numpy()[sample] - ref[sample]).max()) <= tolerance(w)


def test_groups_ignored_past_the_balanced_batch_and_for_float32():
    # 1025 sequences take the partitioned schedule; float32 queries the vector-ALU kernel: the groups are
    # ignored and the result is pa_decode's (here bit for bit: the same kernels run)
    rng = np.random.default_rng(16)
    w = sharing("shared_past_max", 16, 4, 64, "bf16", "bf16", 3, [int(rng.integers(1, 40)) for _ in range(6)],
                [int(rng.integers(0, 40)) for _ in range(1019)], seed=27)
    out, ref_gpu, ref = run_both(w, [(0, 6, 3)])
    assert torch.equal(out, ref_gpu)
    assert float(np.abs(out.cpu().numpy() - ref).max()) <= tolerance(w)
    w = sharing("shared_f32", 8, 2, 64, "f32", "f32", 4, [5, 30, 70], [12, 1], seed=28)
    out, ref_gpu, ref = run_both(w, [(0, 3, 4)])
    assert torch.equal(out, ref_gpu)
    assert float(np.abs(out.cpu().numpy() - ref).max()) <= tolerance(w)
