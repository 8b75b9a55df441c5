"""pa_decode_append (a whole decode step: append the newest token, then attend) against the oracle and
against pa_reshape_and_cache followed by pa_decode.

Where the vector-ALU kernel runs with one workgroup per (sequence, KV head), the decode kernel writes the new
rows itself (one launch); elsewhere the reshape kernel runs first. Either way the caches must equal the
oracle's byte for byte, the output must match the oracle, and it must equal the two-call result bit for bit
(the attention arithmetic is the same). Cases: MHA and two query heads per KV head in 16 bits (fused), float32
with 1 to 8 query heads per KV head (fused), an FP8 cache written by the fused path, contexts split over
partitions (the last partition's workgroup writes), empty sequences and negative slots, int32 slots, grouped
queries on the matrix cores (two launches), and the Llama-2-7B-shaped batch at full size.
"""

import numpy as np
import pytest
import torch

from paged_kv_cache_380_amd import workloads as wl
from pa_testlib import GpuCase, oracle_decode, oracle_fill, raw, tolerance

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_380_amd import binding
    binding.load()
    yield
    torch.cuda.synchronize()


def run(w: wl.Workload, slot_dtype=torch.int64, check_oracle=True):
    from paged_kv_cache_380_amd import binding
    fused = GpuCase(w, slot_dtype=slot_dtype)
    out = torch.full(fused.q.shape, float("nan"), dtype=torch.float32, device="cuda")
    binding.decode_append(out, fused.q, fused.new_key, fused.new_value, fused.kc, fused.vc, fused.new_slots,
                          fused.tables, fused.lens, w.scale, w.num_kv_heads, w.block_size, w.k_scale, w.v_scale)
    two = GpuCase(w, slot_dtype=slot_dtype)
    ref_gpu = two.step(out_dtype=torch.float32)
    torch.cuda.synchronize()
    kc, vc = oracle_fill(w)
    assert np.array_equal(raw(fused.kc).view(np.uint8), kc.view(np.uint8)), f"{w.name}: K cache differs"
    assert np.array_equal(raw(fused.vc).view(np.uint8), vc.view(np.uint8)), f"{w.name}: V cache differs"
    assert torch.equal(out, ref_gpu), f"{w.name}: differs from reshape + decode"
    if check_oracle:
        err = float(np.abs(out.cpu().numpy() - oracle_decode(w, kc, vc)).max())
        assert err <= tolerance(w), f"{w.name}: max|err| = {err}"


@pytest.mark.parametrize("H,Hkv,dtype,cache", [
    (8, 8, "f16", "f16"), (8, 8, "bf16", "bf16"), (8, 4, "f16", "f16"), (8, 8, "bf16", "fp8_e4m3"),
    (8, 8, "f32", "f32"), (8, 2, "f32", "f32"), (8, 1, "f32", "f32"),
])
def test_fused_shapes(H, Hkv, dtype, cache):
    rng = np.random.default_rng(H * 10 + Hkv)
    lens = [int(rng.integers(1, 700)) for _ in range(9)] + [16, 17, 1]
    w = wl.build(f"append_{H}_{Hkv}_{dtype}_{cache}", lens, H, Hkv, 128, dtype, cache_dtype=cache, seed=41,
                 free_fraction=0.1, kv_scale=0.05)
    run(w)


def test_split_contexts_empty_sequences_and_int32_slots():
    # long contexts spread over partitions (the last partition's workgroup writes the new row), empty
    # sequences (slot -1: nothing written, zeros out), head size 64
    w = wl.build("append_split", [5000, 17, 0, 4096, 300, 1, 0], 8, 8, 64, "f16", seed=42, free_fraction=0.1)
    run(w, slot_dtype=torch.int32)


@pytest.mark.parametrize("H,Hkv,cache", [(32, 8, "bf16"), (32, 8, "fp8_e4m3"), (12, 2, "bf16")])
def test_two_launch_shapes(H, Hkv, cache):
    # grouped queries on the matrix cores, or groups of 6 on the vector ALU with several workgroups per KV head
    rng = np.random.default_rng(H + Hkv)
    w = wl.build(f"append_two_{H}_{Hkv}_{cache}", [int(rng.integers(0, 900)) for _ in range(11)], H, Hkv, 128,
                 "bf16", cache_dtype=cache, seed=43, free_fraction=0.1, kv_scale=0.05)
    run(w)


def test_llama7b_mha_full_size():
    run(wl.llama7b_mha_fp16())
