"""A decode step captured in a HIP graph (torch.cuda.CUDAGraph) gives the eager result on every replay.

The C ABI only queues kernels on the caller's stream (no allocation, no
synchronisation, no memset), so a serving loop can capture a step. Each case
captures append + decode for one schedule: the balanced matrix-core kernel
and its merge (ragged grouped-query batch), the partitioned vector-ALU kernel
and its merge (MHA, contexts split over partitions), the shared-prefix
pass with the balanced kernel and the merge, the wide decode of a 64-head
group over one KV head (partitions and their merge), the one-call step
pa_decode_append (the matrix-core kernel writing the new rows itself), and
pa_decode_scratch (the library's fixed scratch array as workspace: nothing
allocated during capture). The graph is replayed several
times with other eager work and synchronisations in between; every replay
must equal the eager output bit for bit (same kernels, same inputs, a fixed
merge order).
"""

import numpy as np
import pytest
import torch

from paged_kv_cache_380_amd import workloads as wl
from pa_testlib import GpuCase

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_380_amd import binding
    binding.load()
    yield
    torch.cuda.synchronize()


def _ragged_gqa():
    rng = np.random.default_rng(31)
    return wl.build("graph_gqa", [int(rng.integers(0, 3000)) for _ in range(40)], 32, 8, 128, "bf16", seed=31,
                    free_fraction=0.1), None, 0, "decode"


def _split_mha():
    return wl.build("graph_mha", [5000, 17, 1, 4096, 300], 8, 8, 128, "f16", seed=32, free_fraction=0.1), None, 32, \
        "decode"


def _wide_mqa():
    return wl.build("graph_mqa", [9000, 17, 0, 4096, 2500], 64, 1, 128, "bf16", seed=34, free_fraction=0.1), None, 0, \
        "decode"


def _append_gqa():
    w, _, _, _ = _ragged_gqa()
    return w, None, 0, "append"


def _scratch_gqa():
    w, _, _, _ = _ragged_gqa()
    return w, None, 0, "scratch"


def _shared_fp8():
    rng = np.random.default_rng(33)
    lens = [40 * 16 + int(rng.integers(1, 500)) for _ in range(9)] + [int(rng.integers(1, 900)) for _ in range(7)]
    w = wl.build("graph_prefix", lens, 32, 8, 128, "bf16", cache_dtype="fp8_e4m3", seed=33, free_fraction=0.1,
                 shared_prefix_blocks=40, sharing_seqs=9, kv_scale=0.05)
    return w, [(0, 9, 40)], 0, "decode"


@pytest.mark.parametrize("make", [_ragged_gqa, _split_mha, _shared_fp8, _wide_mqa, _append_gqa, _scratch_gqa],
                         ids=["balanced", "partitioned", "prefix", "wide", "append", "scratch"])
def test_graph_replays_equal_eager(make):
    from paged_kv_cache_380_amd import binding
    w, groups, pb, mode = make()
    case = GpuCase(w)
    out = torch.empty(case.q.shape, dtype=torch.float32, device="cuda")
    S, H, D = case.q.shape
    if groups:
        nbytes = binding.shared_prefix_workspace_bytes(S, H, w.num_kv_heads, D, w.max_blocks_per_seq,
                                                       max(g[2] for g in groups))
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    else:
        ws = binding.workspace_for(case.q, w.num_kv_heads, case.tables, pb)

    def step():
        if mode == "append":
            binding.decode_append(out, case.q, case.new_key, case.new_value, case.kc, case.vc, case.new_slots,
                                  case.tables, case.lens, w.scale, w.num_kv_heads, w.block_size, w.k_scale,
                                  w.v_scale, workspace=ws)
            return
        case.append()
        if mode == "scratch":
            binding.decode_scratch(out, case.q, case.kc, case.vc, case.tables, case.lens, w.scale, w.num_kv_heads,
                                   w.block_size, w.k_scale, w.v_scale)
        elif groups:
            binding.decode_shared_prefix(out, case.q, case.kc, case.vc, case.tables, case.lens, w.scale,
                                         w.num_kv_heads, groups, w.block_size, w.k_scale, w.v_scale, workspace=ws)
        else:
            binding.decode(out, case.q, case.kc, case.vc, case.tables, case.lens, w.scale, w.num_kv_heads,
                           w.block_size, w.k_scale, w.v_scale, partition_blocks=pb, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    assert torch.isfinite(eager).all()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the capture stream, as torch recommends before capturing
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        out.fill_(float("nan"))
        scratch = torch.randn(1 << 20, device="cuda") * (i + 1)  # other eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from the eager result"
        del scratch
