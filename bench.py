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
                  for f in ("pa_decode.hip", "pa_decode_mfma.hip", "pa_prefill.hip", "pa_decode_common.h",
                            "pa_device.h", "pa_mfma.h", "pa_internal.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic(workload: str, shared_prefix: bool):
    """HBM bytes per decode call from the committed rocprofv3 counter summary, if it is current (same kernel
    sources, same use of the shared-prefix pass)."""
    path = os.path.join(PROFILES, f"decode_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    def field(name):
        m = re.search(rf"^{name}:\s*([0-9.eE+-]+)\s*$", text, re.M)
        return float(m.group(1)) if m else None
    sha = re.search(r"^kernel_source_sha:\s*(\S+)", text, re.M)
    if not sha or sha.group(1) != kernel_source_sha():
        return None  # the kernel changed since the counters were taken
    mode = re.search(r"^shared_prefix:\s*(\S+)", text, re.M)
    if (mode.group(1) if mode else "no") != ("yes" if shared_prefix else "no"):
        return None
    return field("hbm_bytes_per_call")


def decode_algorithmic_bytes(w) -> int:
    """Bytes one decode launch must move: each K/V tile once (shared-prefix tiles once), q, out, table, lengths."""
    from paged_kv_cache_380_amd import workloads as wl
    act = wl.TORCH_DTYPES[w.dtype].itemsize
    return (wl.algorithmic_kv_bytes(w, unique=True) + 2 * w.num_seqs * w.num_heads * w.head_size * act
            + w.block_tables.numel() * 4 + w.num_seqs * 4)


# --- rocprofv3 summaries (run on the host, over the CSV files a profiled run left) -------------

def _csv_rows(directory: str, suffix: str):
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no *{suffix} under {directory}")
    return rows


def _col(row: dict, *names):
    low = {k.lower(): v for k, v in row.items()}
    for n in names:
        if n.lower() in low:
            return low[n.lower()]
    raise KeyError(f"none of {names} in {list(row)}")


def _short(name: str) -> str:
    m = re.search(r"([A-Za-z_][A-Za-z0-9_]*)(<[^()]*>)?\(", name)
    return (m.group(1) + (m.group(2) or "")) if m else name[:80]


def summarize_stats(directory: str, out_path: str, command: str):
    rows = _csv_rows(directory, "kernel_stats.csv")
    lines = [f"# rocprofv3 kernel statistics", f"command: {command}", "",
             f"{'kernel':<60} {'calls':>7} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}"]
    for r in sorted(rows, key=lambda r: -float(_col(r, "TotalDurationNs"))):
        lines.append(f"{_short(_col(r, 'Name')):<60} {int(_col(r, 'Calls')):>7} "
                     f"{float(_col(r, 'AverageNs')) / 1e3:>10.2f} {float(_col(r, 'MinNs')) / 1e3:>10.2f} "
                     f"{float(_col(r, 'MaxNs')) / 1e3:>10.2f} {float(_col(r, 'Percentage')):>6.2f}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter_means(directory: str, counter: str, select) -> tuple[float, int, str]:
    """Per selected kernel, the mean of the counter over its dispatches; returns the sum of those means
    (one call's worth when each selected kernel runs once per call), the dispatch count of the most
    frequent kernel, and the kernel names."""
    vals = {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        name = _col(r, "Kernel_Name")
        if _col(r, "Counter_Name") != counter or not select(name):
            continue
        per = vals.setdefault(_short(name), {})
        key = _col(r, "Dispatch_Id", "Correlation_Id")
        per[key] = per.get(key, 0.0) + float(_col(r, "Counter_Value"))
    if not vals:
        raise SystemExit(f"no {counter} rows for the selected kernel under {directory}")
    total = sum(sum(per.values()) / len(per) for per in vals.values())
    return total, max(len(per) for per in vals.values()), ", ".join(sorted(vals))


def summarize_counters(workload: str, fetch_dir: str, write_dir: str, cal_fetch_dir: str, cal_write_dir: str,
                       copy_mib: int, out_path: str, commands: list[str], shared_prefix_mode: str = "auto"):
    """HBM bytes per decode call (all its kernels: prefix pass, main kernel, merge): FETCH_SIZE and
    WRITE_SIZE (KiB) scaled by what they read for a plain copy."""
    from paged_kv_cache_380_amd import workloads as wl
    is_decode = lambda n: "decode_" in n or "prefill_mfma" in n  # groups of 32+ decode on the prefill kernel
    is_copy = lambda n: "copy" in n.lower()
    fetch, nf, kname = _counter_means(fetch_dir, "FETCH_SIZE", is_decode)
    write, nw, _ = _counter_means(write_dir, "WRITE_SIZE", is_decode)
    cfetch, _, cname = _counter_means(cal_fetch_dir, "FETCH_SIZE", is_copy)
    cwrite, _, _ = _counter_means(cal_write_dir, "WRITE_SIZE", is_copy)
    copy_bytes = copy_mib << 20
    ff, fw = copy_bytes / (cfetch * 1024), copy_bytes / (cwrite * 1024)
    hbm = ff * fetch * 1024 + fw * write * 1024
    w = wl.named(workload)
    algo = decode_algorithmic_bytes(w)
    prefix = shared_prefix_applies(w, 0) if shared_prefix_mode == "auto" else shared_prefix_mode == "on"
    lines = [
        "# rocprofv3 HBM counters of one decode call (sum over its kernels of each kernel's mean per dispatch)",
        f"workload: {w.name}", f"kernel: {kname}", f"kernel_source_sha: {kernel_source_sha()}",
        f"shared_prefix: {'yes' if prefix else 'no'}",
        f"dispatches: {nf} (FETCH_SIZE run), {nw} (WRITE_SIZE run)",
        f"FETCH_SIZE_KiB_per_call: {fetch:.1f}", f"WRITE_SIZE_KiB_per_call: {write:.1f}",
        f"calibration_kernel: {cname} ({copy_mib} MiB read + {copy_mib} MiB written)",
        f"calibration_FETCH_SIZE_KiB: {cfetch:.1f}", f"calibration_WRITE_SIZE_KiB: {cwrite:.1f}",
        f"fetch_factor: {ff:.4f}", f"write_factor: {fw:.4f}",
        f"hbm_bytes_per_call: {hbm:.0f}", f"algorithmic_bytes_per_call: {algo}",
        f"traffic_over_algorithmic: {hbm / algo:.4f}", "commands:"] + [f"  {c}" for c in commands]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_pmc(directory: str, out_path: str, commands: list[str], select: str = ""):
    """Mean per dispatch of every counter a rocprofv3 --pmc run collected, per kernel (kernels whose name
    contains ``select``), one row per kernel. Several run directories may be joined with ':'."""
    per = {}   # kernel -> counter -> dispatch -> value
    for d in directory.split(":"):
        for r in _csv_rows(d, "counter_collection.csv"):
            name = _col(r, "Kernel_Name")
            if select and select not in name:
                continue
            c = per.setdefault(_short(name), {}).setdefault(_col(r, "Counter_Name"), {})
            key = (d, _col(r, "Dispatch_Id", "Correlation_Id"))
            c[key] = c.get(key, 0.0) + float(_col(r, "Counter_Value"))
    if not per:
        raise SystemExit(f"no counter rows under {directory}")
    lines = ["# rocprofv3 counters: mean per dispatch over the run, per kernel", "commands:"]
    lines += [f"  {c}" for c in commands] + [""]
    for k in sorted(per):
        lines.append(f"kernel: {k}")
        for cname in sorted(per[k]):
            vals = list(per[k][cname].values())
            lines.append(f"  {cname:<40} {sum(vals) / len(vals):>18.1f}   ({len(vals)} dispatches)")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


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
    passes = 0
    while True:  # whole passes over the sampled order until the time bound (one sequence = one unit)
        for s in order:
            oracle.reshape_and_cache(nk[s:s + 1], nv[s:s + 1], kc, vc, ns[s:s + 1], w.block_size, w.dtype,
                                     w.cache_dtype, w.k_scale, w.v_scale)
            oracle.decode_attention(q, kc, vc, tables, lens, w.scale, w.num_kv_heads, w.block_size, w.dtype,
                                    w.cache_dtype, w.k_scale, w.v_scale, seqs=[int(s)])
            done.append(int(s))
            kv_bytes += int(lens[s]) * per_tok
            if time.perf_counter() - t0 >= target_seconds:
                break
        else:
            passes += 1
            continue
        break
    wall = time.perf_counter() - t0
    r1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (r1.ru_utime - r0.ru_utime) + (r1.ru_stime - r0.ru_stime)
    del kc, vc
    try:
        from threadpoolctl import threadpool_info
        blas = sorted({(i.get("internal_api"), i.get("num_threads")) for i in threadpool_info()
                       if i.get("user_api") == "blas"})
        blas_threads = max((n for _, n in blas if n), default=None)
        blas_desc = ", ".join(f"{api} {n} threads" for api, n in blas) or "none loaded"
    except Exception as e:  # threadpoolctl missing or failing: say so rather than guess
        blas_threads, blas_desc = None, f"unknown ({type(e).__name__})"
    used = max(1, round(cpu / wall))
    return {
        "value": kv_bytes / wall / 1e9, "unit": "GB/s", "cores": used,
        "kind": "oracle",
        "sample": f"{len(done)} sequence-steps ({passes} whole passes over the {w.num_seqs} sequences, then "
                  f"{len(done) - passes * w.num_seqs} more; reshape of the new token + fp64 decode each), "
                  f"{wall:.1f} s wall, {cpu:.1f} s CPU, {len(os.sched_getaffinity(0))} host cores visible; "
                  f"the oracle's per-head products are small gemv calls, so it ran on {used} core(s) "
                  f"although BLAS ({blas_desc}) could use more",
        "blas_threads": blas_threads,
        "host_cores_visible": len(os.sched_getaffinity(0)),
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
    ap.add_argument("--summarize-stats", nargs=3, metavar=("DIR", "OUT", "COMMAND"),
                    help="write a kernel-statistics summary of a rocprofv3 --kernel-trace --stats run and exit")
    ap.add_argument("--summarize-counters", nargs=6,
                    metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR", "COPY_MIB", "OUT"),
                    help="write the HBM-traffic summary of rocprofv3 --pmc runs for --workload and exit")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("DIRS", "OUT"),
                    help="write the per-kernel mean of every counter of rocprofv3 --pmc runs (DIRS joined by ':') "
                         "and exit; --select limits the kernels")
    ap.add_argument("--select", default="", help="kernel-name filter for --summarize-pmc")
    ap.add_argument("--command", action="append", default=[], help="profiling commands recorded in a summary")
    ap.add_argument("--shared-prefix", choices=("auto", "on", "off"), default="auto",
                    help="decode through pa_decode_shared_prefix with the workload's prefix group (auto: when "
                         "its sequences share a prefix and the grouped reading applies)")
    ap.add_argument("--op", choices=("decode", "prefill", "copy"), default="decode",
                    help="decode: the decode step (default, the headline); prefill: chunked-prefill attention "
                         "(TFLOP/s); copy: copy-on-write block copies (GB/s)")
    args = ap.parse_args()

    if args.summarize_stats:
        summarize_stats(*args.summarize_stats)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.command, args.select)
        return
    if args.summarize_counters:
        fd, wd, cfd, cwd, mib, out = args.summarize_counters
        summarize_counters(args.workload, fd, wd, cfd, cwd, int(mib), out, args.command, args.shared_prefix)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this library has no multi-GPU path.",
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
    from paged_kv_cache_380_amd.resident import ResidentBatch as GpuCase

    if args.op == "prefill":
        return bench_prefill(args, dev)
    if args.op == "copy":
        return bench_copy(args, dev)

    log(f"[bench] building {args.workload}")
    w = wl.named(args.workload, args.seed)
    case = GpuCase(w, device=dev)
    out = torch.empty(case.q.shape, dtype=case.q.dtype, device=dev)
    pb = args.partition_blocks or binding.decode_partition_blocks(w.num_seqs, w.num_heads, w.num_kv_heads,
                                                                  w.head_size, w.max_blocks_per_seq)
    stream = torch.cuda.current_stream(dev)
    prefix = shared_prefix_applies(w, args.partition_blocks) if args.shared_prefix == "auto" else \
        args.shared_prefix == "on"
    if prefix:
        if not w.sharing_seqs:
            raise SystemExit(f"--shared-prefix on: {w.name} has no shared prefix")
        groups = [(0, w.sharing_seqs, w.shared_blocks)]
        nbytes = binding.shared_prefix_workspace_bytes(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_size,
                                                       w.max_blocks_per_seq, w.shared_blocks)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None

        def run_decode():
            binding.decode_shared_prefix(out, case.q, case.kc, case.vc, case.tables, case.lens, w.scale,
                                         w.num_kv_heads, groups, w.block_size, w.k_scale, w.v_scale, workspace=ws)
    else:
        ws = binding.workspace_for(case.q, w.num_kv_heads, case.tables, args.partition_blocks)

        def run_decode():
            binding.decode(out, case.q, case.kc, case.vc, case.tables, case.lens, w.scale, w.num_kv_heads,
                           w.block_size, w.k_scale, w.v_scale, partition_blocks=args.partition_blocks, workspace=ws)

    # The step: append the newest token of every sequence, then attend. pa_decode_append does both (one launch
    # where the decode kernel writes the rows itself); with the shared-prefix pass or an explicit partition
    # length the append is its own pa_reshape_and_cache launch.
    one_call = not prefix and args.partition_blocks == 0

    def step():
        if one_call:
            binding.decode_append(out, case.q, case.new_key, case.new_value, case.kc, case.vc, case.new_slots,
                                  case.tables, case.lens, w.scale, w.num_kv_heads, w.block_size, w.k_scale,
                                  w.v_scale, workspace=ws)
        else:
            case.append()
            run_decode()

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
        run_decode()
        b.record(stream)
    torch.cuda.synchronize()
    durs = sorted(a.elapsed_time(b) for a, b in ev)
    decode_ms = sum(durs) / len(durs)

    # The same launches with the caches cold: 512 MiB written before each one (outside its events)
    # evicts the L2s and the 256 MB Infinity Cache, so nothing of the previous launch's reads is left.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(min(args.steps, 50))]
    for a, b in cold_ev:
        case.append()
        flush.fill_(1)
        a.record(stream)
        run_decode()
        b.record(stream)
    torch.cuda.synchronize()
    cold = sorted(a.elapsed_time(b) for a, b in cold_ev)
    decode_ms_cold = sum(cold) / len(cold)
    del flush

    kv_bytes = wl.algorithmic_kv_bytes(w)
    kv_unique = wl.algorithmic_kv_bytes(w, unique=True)
    step_bytes = wl.algorithmic_step_bytes(w)
    decode_bytes = decode_algorithmic_bytes(w)
    achieved = decode_bytes / (decode_ms * 1e-3) / 1e9
    traffic = counter_traffic(w.name, prefix)

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
            "kv_cache_dtype": w.cache_dtype, "seed": w.seed,
            "schedule": "balanced" if balanced_schedule(w, args.partition_blocks) else f"partitions of {pb} blocks",
            "decode_path": os.environ.get("PA_DECODE_PATH", "auto"),
            "decode_loads": os.environ.get("PA_DECODE_LOADS", "stream"),
            "shared_prefix": [0, w.sharing_seqs, w.shared_blocks] if prefix else None,
            "append": ("in the decode kernel" if one_call and append_fuses(w) else "reshape_and_cache kernel"),
        },
        "pct_of_hbm_peak": round(100 * kv_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "seq_steps_per_s": round(w.num_seqs / (ms_per_step * 1e-3), 1),
        "decode_ms": round(decode_ms, 5),
        "decode_ms_p10_p90": [round(durs[len(durs) // 10], 5), round(durs[(9 * len(durs)) // 10], 5)],
        "decode_ms_cold_cache": round(decode_ms_cold, 5),
        "roofline": {
            "kernel": ("decode_mfma[shared prefix] + " if prefix else "") + decode_kernels(w, args.partition_blocks, pb),
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


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix peak, published


def _events_ms(fn, steps: int, stream) -> list:
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in ev)


def bench_prefill(args, dev):
    """Chunked-prefill attention, Llama-3-8B-shaped GQA: 8 prompts of 2048 tokens each as one chunk."""
    import numpy as np
    import torch
    from paged_kv_cache_380_amd import binding
    from paged_kv_cache_380_amd import workloads as wl
    from paged_kv_cache_380_amd.resident import ResidentBatch as GpuCase
    S, L, H, Hkv, D = 8, 2048, 32, 8, 128
    w = wl.build("prefill_llama3_8b_bf16_b8x2048", [L] * S, H, Hkv, D, "bf16", seed=6, free_fraction=0.05)
    log(f"[bench] building {w.name}")
    case = GpuCase(w, device=dev)
    case.append()
    g = torch.Generator().manual_seed(7)
    q = torch.randn((S * L, H, D), generator=g).to(torch.bfloat16).to(dev)
    out = torch.empty_like(q)
    starts = torch.arange(0, S * L + 1, L, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    run = lambda: binding.prefill(out, q, case.kc, case.vc, case.tables, case.lens, starts, w.scale, Hkv, L)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    durs = _events_ms(run, args.steps, stream)
    k_ms = sum(durs) / len(durs)
    pairs = S * L * (L + 1) // 2                       # (query, key) pairs under the causal mask, per head
    flops = 4.0 * D * H * pairs                        # q.k and p.v, 2 flops per multiply-add
    tflops = flops / (k_ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "paged chunked-prefill attention TFLOP/s (algorithmic, causal)", "value": round(tflops, 1),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": S, "prompt_tokens": L, "num_heads": H, "num_kv_heads": Hkv,
                   "head_size": D, "block_size": 16},
        "roofline": {"kernel": "prefill_mfma", "bound": "mfma", "achieved": round(tflops, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "algorithmic_flops_per_launch": flops},
        "kernel_ms": round(k_ms, 5),
    }), flush=True)


def bench_copy(args, dev):
    """Copy-on-write block copies: 512 (source, destination) pairs of Llama-3-8B-shaped bf16 blocks."""
    import numpy as np
    import torch
    from paged_kv_cache_380_amd import binding
    N, Hkv, D, P = 4096, 8, 128, 512
    kc = torch.randn((N, Hkv, 16, D), device=dev).to(torch.bfloat16)
    vc = torch.randn((N, Hkv, 16, D), device=dev).to(torch.bfloat16)
    perm = np.random.default_rng(8).permutation(N)
    src = torch.from_numpy(perm[:P].astype(np.int32)).to(dev)
    dst = torch.from_numpy(perm[P:2 * P].astype(np.int32)).to(dev)
    stream = torch.cuda.current_stream(dev)
    run = lambda: binding.copy_blocks(kc, vc, src, dst)
    for _ in range(args.warmup):
        run()
    durs = _events_ms(run, args.steps, stream)
    k_ms = sum(durs) / len(durs)
    moved = 2 * 2 * P * Hkv * 16 * D * 2               # K and V, read + write
    gbs = moved / (k_ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "copy-on-write block copies GB/s (read + write)", "value": round(gbs, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(k_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "copy_blocks_512_pairs_bf16", "pairs": P, "num_kv_heads": Hkv, "head_size": D},
        "roofline": {"kernel": "copy_blocks_kernel", "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": moved},
    }), flush=True)


def decode_kernel(w) -> str:
    """Name of the decode kernel the library runs for this workload (its selection rule, restated)."""
    group = w.num_heads // w.num_kv_heads
    path = os.environ.get("PA_DECODE_PATH", "auto")
    if w.dtype in ("f16", "bf16") and group >= 32 and group % 32 == 0 and path != "valu":
        return "prefill_mfma[decode]"
    if w.dtype in ("f16", "bf16") and group % 4 == 0 and path != "valu":
        return "decode_mfma"
    if w.dtype in ("f16", "bf16") and group % 4 == 0:
        return "decode_gqa"
    return "decode_main"


def wl_parts(w, pb: int) -> int:
    return -(-w.max_blocks_per_seq // pb)


def balanced_schedule(w, partition_blocks: int) -> bool:
    """Whether the library picks its balanced schedule here (its selection rule, restated)."""
    return (decode_kernel(w) == "decode_mfma" and partition_blocks == 0 and w.num_seqs <= 1024
            and w.num_seqs * w.max_blocks_per_seq <= 2**31 - 1)


def append_fuses(w) -> bool:
    """Whether pa_decode_append writes the new rows inside the decode kernel (the library's rule, restated):
    the vector-ALU kernel with one workgroup per KV head, or the matrix-core kernel with one head tile per KV
    head (4, 8 or 16 query heads per KV head)."""
    group = w.num_heads // w.num_kv_heads
    if decode_kernel(w) == "decode_mfma":
        return group in (4, 8, 16)
    tile = next(t for t in (8, 4, 2, 1) if group % t == 0)
    return decode_kernel(w) == "decode_main" and tile == group


def shared_prefix_applies(w, partition_blocks: int) -> bool:
    """Whether the shared-prefix pass runs for this workload's prefix group (the library's rule, restated)."""
    group = w.num_heads // w.num_kv_heads
    return bool(w.sharing_seqs) and balanced_schedule(w, partition_blocks) and group >= 4 and 16 % group == 0


def decode_kernels(w, partition_blocks: int, pb: int) -> str:
    if balanced_schedule(w, partition_blocks):
        return "decode_mfma[balanced] + decode_bal_reduce"
    return decode_kernel(w) + ("" if wl_parts(w, pb) == 1 else " + decode_reduce")


if __name__ == "__main__":
    main()
