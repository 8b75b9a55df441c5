"""Throughput of one paged decode step on one MI355X.

A step is the whole hot path on one batch: pa_reshape_and_cache appends the
newest token of every sequence, then pa_decode attends over every context.
Inputs are seeded synthetic data already resident in HBM when timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints one JSON line on stdout. Besides the step throughput it reports the
roofline position of the dominant kernel (decode; its duration measured with
HIP events on the stream it runs on) and the CPU oracle's speed on a bounded
sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import resource
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_380_amd", "csrc", f)
                  for f in ("pa_decode.hip", "pa_device.h", "pa_internal.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic(workload: str, algorithmic_bytes: float):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, if it is current."""
    path = os.path.join(PROFILES, f"decode_main_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    def field(name):
        m = re.search(rf"^{name}:\s*([0-9.eE+-]+)\s*$", text, re.M)
        return float(m.group(1)) if m else None
    sha = re.search(r"^kernel_source_sha:\s*(\S+)", text, re.M)
    if not sha or sha.group(1) != kernel_source_sha():
        return None  # the kernel changed since the counters were taken
    b = field("hbm_bytes_per_dispatch")
    return b


def cpu_baseline(w, target_seconds: float):
    """The oracle as it stands, on a bounded sample of sequences of the same workload."""
    import numpy as np
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    from pa_testlib import oracle_fill, raw
    from paged_kv_cache_380_amd import workloads as wl

    kc, vc = oracle_fill(w, with_new=False)  # the cached context (setup, not timed)
    q = raw(w.q)
    tables, lens = w.block_tables.numpy(), w.context_lens.numpy()
    nk, nv, ns = raw(w.new_key), raw(w.new_value), w.new_slots.numpy()
    order = np.random.default_rng(0).permutation(w.num_seqs)
    done, kv_bytes = [], 0
    per_tok = w.num_kv_heads * w.head_size * 2 * w.kv_bytes_per_elem()
    r0 = resource.getrusage(resource.RUSAGE_SELF)
    t0 = time.perf_counter()
    for s in order:
        oracle.reshape_and_cache(nk[s:s + 1], nv[s:s + 1], kc, vc, ns[s:s + 1], w.block_size, w.dtype,
                                 w.cache_dtype, w.k_scale, w.v_scale)
        oracle.decode_attention(q, kc, vc, tables, lens, w.scale, w.num_kv_heads, w.block_size, w.dtype,
                                w.cache_dtype, w.k_scale, w.v_scale, seqs=[int(s)])
        done.append(int(s))
        kv_bytes += int(lens[s]) * per_tok
        if time.perf_counter() - t0 >= target_seconds:
            break
    wall = time.perf_counter() - t0
    r1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (r1.ru_utime - r0.ru_utime) + (r1.ru_stime - r0.ru_stime)
    del kc, vc
    return {
        "value": kv_bytes / wall / 1e9, "unit": "GB/s", "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": f"{len(done)} of {w.num_seqs} sequences (reshape of their new token + fp64 decode), "
                  f"{wall:.1f} s wall, {cpu:.1f} s CPU, {len(os.sched_getaffinity(0))} host cores visible",
        "seq_steps_per_s": len(done) / wall,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama7b_mha_fp16")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--partition-blocks", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="bound on the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB (for counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(max(args.steps, 1)):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {n} bytes x {max(args.steps, 1)}")
        return

    from paged_kv_cache_380_amd import binding
    from paged_kv_cache_380_amd import workloads as wl
    binding.load()
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from pa_testlib import GpuCase

    log(f"[bench] building {args.workload}")
    w = wl.named(args.workload, args.seed)
    case = GpuCase(w, device=dev)
    out = torch.empty(case.q.shape, dtype=case.q.dtype, device=dev)
    ws = binding.workspace_for(case.q, w.num_kv_heads, case.tables, args.partition_blocks)
    pb = args.partition_blocks or binding.decode_partition_blocks(w.num_seqs, w.num_heads, w.num_kv_heads,
                                                                  w.head_size, w.max_blocks_per_seq)
    stream = torch.cuda.current_stream(dev)

    def step():
        case.append()
        binding.decode(out, case.q, case.kc, case.vc, case.tables, case.lens, w.scale, w.num_kv_heads,
                       w.block_size, w.k_scale, w.v_scale, partition_blocks=args.partition_blocks, workspace=ws)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Whole-step throughput: exactly K steps between two synchronisations.
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # Decode launches alone, timed with events on the stream the kernels run on.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in ev:
        case.append()
        a.record(stream)
        binding.decode(out, case.q, case.kc, case.vc, case.tables, case.lens, w.scale, w.num_kv_heads,
                       w.block_size, w.k_scale, w.v_scale, partition_blocks=args.partition_blocks, workspace=ws)
        b.record(stream)
    torch.cuda.synchronize()
    durs = sorted(a.elapsed_time(b) for a, b in ev)
    decode_ms = sum(durs) / len(durs)

    kv_bytes = wl.algorithmic_kv_bytes(w)
    kv_unique = wl.algorithmic_kv_bytes(w, unique=True)
    step_bytes = wl.algorithmic_step_bytes(w)
    act = torch.empty((), dtype=case.q.dtype).element_size()
    decode_bytes = kv_unique + 2 * w.num_seqs * w.num_heads * w.head_size * act + w.block_tables.numel() * 4 \
        + w.num_seqs * 4
    achieved = decode_bytes / (decode_ms * 1e-3) / 1e9
    traffic = counter_traffic(w.name, decode_bytes)

    res = {
        "metric": "paged-attn decode KV-read HBM GB/s (% of peak) + seq-steps/s, 7B shape b32",
        "value": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "f16": "f16", "bf16": "bf16"}[w.dtype] + ("+fp8kv" if w.cache_dtype == "fp8_e4m3"
                                                                          else ""),
        "data": "synthetic (seeded N(0,1) q/K/V, random block tables; inputs resident in HBM)",
        "config": {
            "workload": w.name, "num_seqs": w.num_seqs, "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads,
            "head_size": w.head_size, "block_size": w.block_size, "context_tokens": int(w.context_lens.sum()),
            "kv_cache_dtype": w.cache_dtype, "partition_blocks": pb, "seed": w.seed,
        },
        "pct_of_hbm_peak": round(100 * kv_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "seq_steps_per_s": round(w.num_seqs / (ms_per_step * 1e-3), 1),
        "decode_ms": round(decode_ms, 5),
        "decode_ms_p10_p90": [round(durs[len(durs) // 10], 5), round(durs[(9 * len(durs)) // 10], 5)],
        "roofline": {
            "kernel": "decode_main" + ("" if wl_parts(w, pb) == 1 else " + decode_reduce"),
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else round(traffic),
            "algorithmic_bytes_per_launch": decode_bytes,
        },
    }
    if w.shared_blocks:
        res["kv_bytes_logical"] = kv_bytes
        res["kv_bytes_unique"] = kv_unique

    if not args.no_cpu_baseline:
        log(f"[bench] oracle sample (~{args.cpu_seconds:.0f} s)")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def wl_parts(w, pb: int) -> int:
    return -(-w.max_blocks_per_seq // pb)


if __name__ == "__main__":
    main()
