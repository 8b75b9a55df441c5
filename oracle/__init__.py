"""Plain, slow, obviously correct CPU oracle for paged-KV-cache decode attention.

THIS PACKAGE IS TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it. The HIP library and
its Python binding never import, link or call anything here, and nothing here
imports them: the two sides share no code. The only thing both sides consume is
the seeded input generator in ``paged_kv_cache_380_amd/workloads.py``, which
draws random numbers and lays out block tables but computes nothing of the
method.

Sources (cited by title and section; the pages are three web pages about vLLM):

* [vLLM-history] "vLLM 前世今生：从 PagedAttention 到分布式推理引擎的演进之路",
  §3.2 (PagedAttention design: each sequence's KV cache cut into fixed blocks of
  16 tokens by default, reached through a block table; physical blocks may be
  shared by several sequences), §5.2 and §7.3 (FP8 KV cache).
* [vLLM-note] "vLLM" (Spark Notes), section "PagedAttention" (the page that holds
  a position is position // block_size; the cache engine reads and writes pages)
  and section "内核优化" (kernel optimisation: grouped-query attention kernels).
* Attention itself, softmax(q Kᵀ · scale) V, is not written out on the pages; it
  is the textbook definition (Vaswani et al., 2017, "Attention Is All You Need",
  eq. 1), which the decode step evaluates for one query position per sequence.
* The FP8 E4M3 format is the OCP "8-bit Floating Point Specification (OFP8)"
  v1.0 (2023), table of E4M3 encodings.

Pins: every function here is checked in ``tests/test_oracle.py`` against things
other than itself (a library attention routine, closed forms, invariances,
brute force, the OCP format's published code points and an independent FP8
cast). No function in this package is "parity unpinned".
"""

from .e4m3 import e4m3_code_values, e4m3_decode, e4m3_encode
from .paged_attention import (
    DTYPES,
    copy_blocks,
    decode_attention,
    prefill_attention,
    quantize_for_cache,
    reshape_and_cache,
    widen,
)

__all__ = [
    "DTYPES",
    "copy_blocks",
    "decode_attention",
    "prefill_attention",
    "e4m3_code_values",
    "e4m3_decode",
    "e4m3_encode",
    "quantize_for_cache",
    "reshape_and_cache",
    "widen",
]
