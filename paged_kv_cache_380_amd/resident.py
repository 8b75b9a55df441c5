"""A decode batch resident in device memory, its cache filled through the library.

Used by bench.py and by the GPU tests: uploads a workload's inputs (from
``workloads``), writes every already-cached token into fresh caches with
pa_reshape_and_cache, and runs the step's calls through the binding. It holds
no arithmetic of the method: every write and every attention value comes from
the library's kernels.
"""

from __future__ import annotations

import torch

from . import binding
from . import workloads as wl


class ResidentBatch:
    """A workload resident on the GPU, filled through pa_reshape_and_cache."""

    def __init__(self, w: wl.Workload, device="cuda", slot_dtype=torch.int64):
        self.w = w
        self.dev = device
        self.kc = w.poisoned_cache(device)
        self.vc = w.poisoned_cache(device)
        self.q = w.q.to(device)
        self.tables = w.block_tables.to(device)
        self.lens = w.context_lens.to(device)
        self.new_key = w.new_key.to(device)
        self.new_value = w.new_value.to(device)
        self.new_slots = w.new_slots.to(device=device, dtype=slot_dtype)
        if len(w.fill_slots):
            binding.reshape_and_cache(w.fill_key.to(device), w.fill_value.to(device), self.kc, self.vc,
                                      w.fill_slots.to(device=device, dtype=slot_dtype), w.k_scale, w.v_scale)

    def append(self):
        """Write the step's new token of every sequence (pa_reshape_and_cache)."""
        binding.reshape_and_cache(self.new_key, self.new_value, self.kc, self.vc, self.new_slots,
                                  self.w.k_scale, self.w.v_scale)

    def decode(self, out_dtype=None, partition_blocks=0, workspace=None) -> torch.Tensor:
        """pa_decode over every context into a fresh (NaN-filled) output."""
        w = self.w
        out = torch.empty(self.q.shape, dtype=out_dtype or self.q.dtype, device=self.dev)
        out.fill_(float("nan"))
        binding.decode(out, self.q, self.kc, self.vc, self.tables, self.lens, w.scale, w.num_kv_heads,
                       w.block_size, w.k_scale, w.v_scale, partition_blocks=partition_blocks, workspace=workspace)
        return out

    def decode_append(self, out_dtype=None, workspace=None) -> torch.Tensor:
        """The whole step in one call (pa_decode_append): append the new tokens, then attend."""
        w = self.w
        out = torch.empty(self.q.shape, dtype=out_dtype or self.q.dtype, device=self.dev)
        out.fill_(float("nan"))
        binding.decode_append(out, self.q, self.new_key, self.new_value, self.kc, self.vc, self.new_slots,
                              self.tables, self.lens, w.scale, w.num_kv_heads, w.block_size, w.k_scale, w.v_scale,
                              workspace=workspace)
        return out

    def step(self, out_dtype=None, partition_blocks=0) -> torch.Tensor:
        """Append, then decode, as two calls."""
        self.append()
        return self.decode(out_dtype, partition_blocks)
