#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X: KV GB/s (share of 8 TB/s HBM) and tokens/s.

    python bench.py [--steps K] [--warmup W] [--workload gqa_32k|split_128k|prefix_shared|mla_16k|tiny_fp32]

A step is one whole decode step of the hot path over one batch: kvattn_decode_partial (all
sequences, KV heads and partitions) followed by kvattn_merge_lse, with every input already
resident in HBM.  The default workload is the Qwen3-30B-A3B-shaped layer: 16 sequences x
32768 tokens, 32 query / 4 KV heads, head dim 128, bf16 cache, 16-token blocks scattered by a
seeded random block table, 512-token partitions.  Prints one JSON line on stdout; progress
goes to stderr.

Fields beyond the contract: `roofline` (dominant kernel vs 8 TB/s, timed with HIP events on
the launch stream), `cpu_baseline` (the float64 oracle on a bounded sample, on this host's
cores), `copy_GBps` (a plain device-to-device copy on this GPU, for scale), `gather_ceiling`
(the decode kernel's own loads with no arithmetic, timed after the steps: the access pattern's
bandwidth ceiling on this GPU, and the decode kernel's fraction of it).
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
LAYERS = {"gqa_32k": 48, "split_128k": 32, "prefix_shared": None, "mla_16k": 27, "tiny_fp32": None}
DESCR = {
    "gqa_32k": "Qwen3-30B-A3B-shaped GQA decode layer, bs16 x 32K",
    "split_128k": "Mixtral-8x7B-shaped split decode, B4 x 128K, device share (1-r)",
    "prefix_shared": "prefix-shared pool, 64 seqs in groups of 8, two regions",
    "mla_16k": "DeepSeek-V2-Lite-shaped MLA latent decode, B32 x 16K",
    "tiny_fp32": "tiny fp32 paged decode",
}
KERNEL_SOURCES = {
    "mla_16k": ["decode_mla.hip", "device_common.h"],
}
DEFAULT_KERNEL_SOURCES = ["decode_gqa.hip", "device_common.h"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _code_only(text):
    """C++ source without comments and with whitespace runs collapsed (string and character
    literals kept as they are), so that editing a comment does not void stored readings."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":  # a literal: copy through its closing quote
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_hash(workload):
    """Hash of the code (comments and whitespace aside) of the sources the workload's dominant
    kernel is built from, plus the device compile flags: stored counter readings apply only
    while this hash is unchanged."""
    from paged_kv_cache_mla_amd.build import ARCH, COMMON, DEVICE
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_mla_amd", "csrc")
    for f in KERNEL_SOURCES.get(workload, DEFAULT_KERNEL_SOURCES):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    flags = [f for f in COMMON + DEVICE if not f.startswith("-I")]  # include paths vary by host
    h.update(" ".join([ARCH] + flags).encode())
    return h.hexdigest()[:16]


def profile_path(workload):
    return os.path.join(ROOT, "profiles", f"decode_partial_and_merge.{workload}.md")


def read_profile_values(path):
    """`key: value` lines of a profile summary (the lines between the two `values` markers)."""
    vals = {}
    inside = False
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if line == "<!-- values -->":
                inside = not inside
                continue
            if inside and ":" in line:
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    return vals


def stored_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; None otherwise."""
    path = profile_path(workload)
    if not os.path.exists(path):
        return None
    vals = read_profile_values(path)
    if vals.get("kernel_hash") != kernel_hash(workload) or "hbm_bytes_per_launch" not in vals:
        return None
    return int(vals["hbm_bytes_per_launch"])


# --------------------------------------------------------------- rocprofv3 summaries
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 2 << 30  # the device-to-device copy of copy_bandwidth(): 2 GiB read, 2 GiB written


def _short(name):
    name = name.split("(")[0]
    return name.replace("void ", "")


def _read_csv(path):
    import csv
    with open(path) as fh:
        return list(csv.DictReader(fh))


def _is_probe(kernel_name):
    """The gather probe's kernels (kvattn_gather_probe), not the decode's."""
    return "gqa_probe_kernel" in kernel_name or "mla_decode_kernel<true>" in kernel_name


def _counter_by_kernel(rows, counter):
    out = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        out.setdefault(r["Kernel_Name"], []).append((int(r["Grid_Size"]), float(r["Counter_Value"])))
    return out


def _copy_factor(per_kernel):
    """Known bytes / counter bytes for the large device-to-device copies of copy_bandwidth()."""
    runs = per_kernel.get(COPY_KERNEL, [])
    if not runs:
        raise RuntimeError("no copy kernel in the counter run")
    big = max(g for g, _ in runs)
    vals = [v for g, v in runs if g == big]
    return COPY_BYTES / (1024.0 * sum(vals) / len(vals))


def summarize_profile(workload, fetch_dir, write_dir, stats_dir, out_path, commands):
    """Write the text summary of one workload's rocprofv3 runs: kernel-trace statistics and
    FETCH_SIZE / WRITE_SIZE per dispatch, scaled by the copy-kernel calibration."""
    import glob
    stats = _read_csv(glob.glob(os.path.join(stats_dir, "*kernel_stats.csv"))[0])
    fetch = _counter_by_kernel(_read_csv(glob.glob(os.path.join(fetch_dir, "*counter_collection.csv"))[0]), "FETCH_SIZE")
    write = _counter_by_kernel(_read_csv(glob.glob(os.path.join(write_dir, "*counter_collection.csv"))[0]), "WRITE_SIZE")
    f_fetch, f_write = _copy_factor(fetch), _copy_factor(write)
    ours = [r for r in stats if "kvattn::" in r["Name"]]
    ours.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"# rocprofv3 summary: {workload} ({DESCR[workload]})", "",
             "Commands (from the repository root; rocprofv3 runs were started from /tmp):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", "## Kernel trace (--kernel-trace --stats)", "",
              "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in ours:
        lines.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    lines += ["", "## HBM counters (--pmc, one counter per run), KiB per dispatch", "",
              f"Calibration: a {COPY_BYTES >> 30} GiB device-to-device copy ({COPY_KERNEL}) reads "
              f"FETCH_SIZE x {f_fetch:.4f} and WRITE_SIZE x {f_write:.4f} of its known size; the "
              "bytes below are scaled by these factors.", "",
              "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read bytes | scaled write bytes |",
              "|---|---|---|---|---|"]
    dom = None  # the decode kernel: the gather probe's own launches are timed beside it
    for r in ours:
        name = r["Name"]
        fv = [v for _, v in fetch.get(name, [])]
        wv = [v for _, v in write.get(name, [])]
        if not fv or not wv:
            continue
        fk, wk = sum(fv) / len(fv), sum(wv) / len(wv)
        rb, wb = fk * 1024 * f_fetch, wk * 1024 * f_write
        lines.append(f"| {_short(name)} | {fk:.0f} | {wk:.0f} | {rb:.0f} | {wb:.0f} |")
        if dom is None and not _is_probe(name):
            dom = (name, float(r["AverageNs"]), rb + wb)
    lines += ["", "Values read by bench.py (dominant kernel; void once the kernel source changes):", "",
              "<!-- values -->",
              f"kernel: {_short(dom[0])}",
              f"kernel_hash: {kernel_hash(workload)}",
              f"avg_duration_us: {dom[1] / 1e3:.2f}",
              f"fetch_factor: {f_fetch:.5f}",
              f"write_factor: {f_write:.5f}",
              f"hbm_bytes_per_launch: {dom[2]:.0f}",
              "<!-- values -->", ""]
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines))
    return out_path


def summarize_counters(workload, dirs, out_path, commands):
    """Write the per-dispatch averages of the counters collected in `dirs` (one rocprofv3
    --pmc run each) for this library's kernels, with the L2 hit rate derived from TCC_HIT_sum
    and TCC_MISS_sum when both were collected."""
    import glob
    vals = {}   # kernel -> counter -> list of per-dispatch values
    for d in dirs:
        for r in _read_csv(glob.glob(os.path.join(d, "*counter_collection.csv"))[0]):
            if "kvattn::" not in r["Kernel_Name"]:
                continue
            vals.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    names = sorted({c for v in vals.values() for c in v})
    lines = [f"# rocprofv3 counters: {workload} ({DESCR[workload]})", "",
             "Commands (from the repository root; rocprofv3 runs were started from /tmp):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", "Per-dispatch averages. MfmaUtil: percent of SIMD cycles with the matrix cores busy. "
              "LdsBankConflict: bank-conflict cycles per LDS access cycle. MeanOccupancyPerCU: "
              "resident waves per CU. L2 hit: TCC_HIT / (TCC_HIT + TCC_MISS).", "",
              "| kernel | dispatches | " + " | ".join(names) + " | L2 hit |",
              "|---|---|" + "---|" * len(names) + "---|"]
    for k in sorted(vals, key=lambda k: -len(vals[k])):
        v = vals[k]
        n = max(len(x) for x in v.values())
        avg = {c: sum(v[c]) / len(v[c]) for c in v}
        cells = [f"{avg[c]:.4g}" if c in avg else "" for c in names]
        hit = ""
        if "TCC_HIT_sum" in avg and "TCC_MISS_sum" in avg and avg["TCC_HIT_sum"] + avg["TCC_MISS_sum"] > 0:
            hit = f"{100 * avg['TCC_HIT_sum'] / (avg['TCC_HIT_sum'] + avg['TCC_MISS_sum']):.1f}%"
        lines.append(f"| {_short(k)} | {n} | " + " | ".join(cells) + f" | {hit} |")
    lines += ["", "Source these readings were taken on (void once the kernel source changes):", "",
              "<!-- values -->", f"kernel_hash: {kernel_hash(workload)}", "<!-- values -->", ""]
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines))
    return out_path


class HipTimer:
    """HIP timing events on an explicit stream, through the HIP runtime torch itself loaded,
    created with hipEventDisableSystemFence: recording them neither writes back nor
    invalidates the caches, so they do not perturb the kernels they bracket."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        path = None
        with open("/proc/self/maps") as fh:
            for line in fh:
                f = line.split()[-1]
                if os.path.basename(f).startswith("libamdhip64"):
                    path = f
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        self._c = ctypes
        self.hip = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [vp, vp]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        self.events = []

    def event(self):
        e = self._c.c_void_p()
        if self.hip.hipEventCreateWithFlags(self._c.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.events.append(e)
        return e

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ev, self._c.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        f = self._c.c_float()
        if self.hip.hipEventElapsedTime(self._c.byref(f), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value


def copy_bandwidth(torch, nbytes=2 << 30, reps=10):
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1.0)
    for _ in range(2):
        b.copy_(a)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del a, b
    return 2 * nbytes / (ms * 1e-3) / 1e9


def cpu_baseline(case, budget_s=10.0):
    """The float64 oracle on a bounded sample of the same workload: whole sequences (all
    heads), cycling over the batch until ~budget_s of CPU time has been spent."""
    import numpy as np
    import oracle
    lay = oracle.Layout(case.block_size, case.num_kv_heads, case.head_dim_k, case.head_dim_v,
                        case.dtype, case.latent)
    t0 = time.perf_counter()
    done_tokens = 0
    n_seq = 0
    while True:
        b = n_seq % case.batch
        oracle.decode_reference(lay, case.regions, case.region_blocks, case.table, case.ctx_lens,
                                case.q, case.scale, tok_begin=case.tok_begin, seqs=[b])
        beg = 0 if case.tok_begin is None else int(case.tok_begin[b])
        done_tokens += int(case.ctx_lens[b]) - beg
        n_seq += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    nbytes = done_tokens * case.kv_bytes_per_token()
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=None)
    except Exception:
        pass
    cores = len(os.sched_getaffinity(0))
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads or cores,
            "host_cpus": cores, "kind": "oracle",
            "sample": f"{n_seq} sequence passes over the {case.batch} sequences (all heads), "
                      f"{done_tokens} tokens, {nbytes} KV bytes, float64 numpy, {dt:.1f} s"}


def oracle_host_share(case):
    """cpu_baseline leg of the split workload: the host share [0, tok_begin) of every sequence,
    computed by the float64 oracle on this host's cores, timed.  Its (o, lse) is the external
    partial the timed steps merge."""
    import numpy as np
    import oracle
    lay = oracle.Layout(case.block_size, case.num_kv_heads, case.head_dim_k, case.head_dim_v,
                        case.dtype, case.latent)
    qf = oracle.bf16_bits_to_f64(case.q) if case.dtype == "bf16" else case.q.astype(np.float64)
    o = np.zeros((case.batch, case.num_q_heads, case.head_dim_v))
    lse = np.full((case.batch, case.num_q_heads), -np.inf)
    t0 = time.perf_counter()
    tokens = 0
    for b in range(case.batch):
        beg = int(case.tok_begin[b])
        k, v = oracle.gather_sequence(lay, case.ext_regions, case.ext_region_blocks,
                                      case.ext_table[b], 0, beg)
        o[b], lse[b] = oracle.attend(qf[b], k, v, case.scale)
        tokens += beg
    return o, lse, time.perf_counter() - t0, tokens


def kv_token_slots(case):
    """(logical, unique) K/V token slots one step reads: every sequence's tokens
    [tok_begin, L), and the distinct (physical block, slot) pairs among them -- a block shared
    by several sequences (prefix sharing) holds its tokens once."""
    import numpy as np
    bs = case.block_size
    keys = []
    for b in range(case.batch):
        beg = 0 if case.tok_begin is None else int(case.tok_begin[b])
        t = np.arange(beg, int(case.ctx_lens[b]), dtype=np.int64)
        keys.append(case.table[b][t // bs].astype(np.int64) * bs + t % bs)
    allk = np.concatenate(keys) if keys else np.zeros(0, np.int64)
    return int(allk.size), int(np.unique(allk).size)


def _time_steps(torch, fn, steps, warmup):
    """Wall-clock ms per call of fn() run back to back, bracketed by device synchronisation."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def host_share_bench(args):
    """The sequence split of the Mixtral-shaped 4 x 128K workload with a native CPU share,
    sized by the share policy: calibrate the per-position costs and fixed overheads of both
    sides (least-squares lines over several token counts), take r from the balance of the
    two step latencies, then time overlapped steps (device share on the GPU, host share on
    the CPU at the same time, merged on the GPU) at that r and around it."""
    import numpy as np
    import torch

    from paged_kv_cache_mla_amd import _lib
    from paged_kv_cache_mla_amd.api import DecodeStep, HostShare, share_fit, share_optimum
    from paged_kv_cache_mla_amd.session import DeviceCase, SplitStep
    from synth import make_case

    _lib.load()
    torch.cuda.set_device(0)
    # one CPU is left to the HIP runtime's own threads
    threads = args.host_threads or max(1, min(16, len(os.sched_getaffinity(0))) - 1)
    log("[share] generating split_128k (full) with every block on the device")
    # r = 0: the device pool holds every block; the same blocks in host memory (case.regions,
    # case.table) serve the host share, so any split point can be timed on one upload
    case = make_case("split_128k", "full", r=0.0)
    dc = DeviceCase(case)
    L, bs, B = int(case.ctx_lens[0]), case.block_size, case.batch

    def dstep(begin):
        return DecodeStep(dc.pool, dc.table, case.ctx_lens, case.part_tokens, case.num_q_heads,
                          case.head_dim_v, tok_begin=[begin] * B)

    def hshare(end):
        return HostShare(bs, case.num_kv_heads, case.head_dim_k, case.head_dim_v, case.dtype,
                         case.latent, case.regions, case.num_q_heads, case.scale, case.table,
                         [end] * B, n_threads=threads)

    def median(xs):
        return float(np.median(np.asarray(xs)))

    # Eq. 1's GPU component: the device partial's latency from its enqueue, over device
    # shares of 1/4 .. all of the context (the range where it is linear in the positions)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gpu_pts = []
    for m in (L // 4, L // 2, 3 * L // 4, L):
        st = dstep(L - m)
        vals = []
        for i in range(args.warmup + 10):
            ev0.record()
            st.partial(dc.q, dc.q_dtype, case.scale)
            ev1.record()
            torch.cuda.synchronize()
            if i >= args.warmup:
                vals.append(ev0.elapsed_time(ev1))
        gpu_pts.append((m, median(vals)))
        log(f"[share] gpu partial over {m} positions: {gpu_pts[-1][1] * 1e3:.1f} us")
    B_cost, C_gpu = share_fit([p[0] for p in gpu_pts], [p[1] for p in gpu_pts])
    # Eq. 1's CPU component, measured inside split steps: from the device partial's enqueue
    # until the merge of the host partial is enqueued (q out, host compute, launch)
    def cpu_points(ns):
        pts = []
        for n in ns:
            ss = SplitStep(dstep(n), dc.q, dc.q_dtype, case.scale, hshare(n), timing=True)
            vals, host = [], []
            for i in range(args.warmup + 10):
                ss.run()
                torch.cuda.synchronize()
                if i >= args.warmup:
                    vals.append(ss.component_ms()[1])
                    host.append(ss.host_ms)
            pts.append((n, median(vals), median(host)))
            log(f"[share] cpu share of {n} positions: component {pts[-1][1] * 1e3:.1f} us "
                f"(host compute {pts[-1][2] * 1e3:.1f} us)")
        return pts

    # a wide scan first, then a local one around the first estimate: the host's cost per
    # position is not constant over two decades of share sizes, and Eq. 2 needs the slope
    # and intercept where the balance falls
    cpu_wide = cpu_points((256, 1024, 4096, 8192))
    A_cost, C_cpu = share_fit([p[0] for p in cpu_wide], [p[1] for p in cpu_wide])
    r_wide = share_optimum(A_cost, B_cost, C_cpu, C_gpu, L)
    n0 = max(2 * bs, int(round(r_wide * L / bs)) * bs)
    local = sorted({max(bs, int(round(n0 * m / bs)) * bs) for m in (0.5, 0.75, 1.0, 1.5, 2.0)})
    cpu_pts = cpu_points(local)
    A_cost, C_cpu = share_fit([p[0] for p in cpu_pts], [p[1] for p in cpu_pts])
    r_pol = share_optimum(A_cost, B_cost, C_cpu, C_gpu, L)
    begin_pol = int(round(r_pol * L / bs)) * bs
    log(f"[share] wide fit r={r_wide:.5f}; local A={A_cost * 1e6:.2f} ns/pos C_cpu={C_cpu * 1e3:.1f} us  "
        f"B={B_cost * 1e6:.3f} ns/pos C_gpu={C_gpu * 1e3:.1f} us  r={r_pol:.5f} -> {begin_pol}")

    gpu_only = _time_steps(torch, lambda: dc.step.run(dc.q, dc.q_dtype, case.scale),
                           args.steps, args.warmup)
    cands = {0, begin_pol, 256, 512, 768, 1024, 1536, 2048, 4096}
    for m in (0.5, 0.75, 1.25, 1.5, 2):
        cands.add(int(round(begin_pol * m / bs)) * bs)
    sweep = []
    for begin, q_first in [(b, qf) for b in sorted(cands) for qf in (False, True)]:
        ss = SplitStep(dstep(begin), dc.q, dc.q_dtype, case.scale, hshare(begin), q_first=q_first)
        host = []

        def one():
            ss.run()
            host.append(ss.host_ms)
        ms = _time_steps(torch, one, args.steps, args.warmup)
        o, l = ss.step.o_out, ss.step.lse_out
        if not (torch.isfinite(o).all() and torch.isfinite(l).all()):
            raise RuntimeError("non-finite output")
        # the two components of the step in place (synchronised steps, so the timed loop
        # above is not perturbed by the timing events)
        sst = SplitStep(dstep(begin), dc.q, dc.q_dtype, case.scale, hshare(begin), timing=True,
                        q_first=q_first)
        comp = []
        for i in range(8):
            sst.run()
            torch.cuda.synchronize()
            if i >= 3:
                comp.append(sst.component_ms())
        sweep.append({"cpu_positions": begin, "r": round(begin / L, 6), "q_first": q_first,
                      "ms_per_step": round(ms, 5),
                      "host_ms": round(float(np.mean(host[-args.steps:])), 5),
                      "t_gpu_us": round(median([c[0] for c in comp]) * 1e3, 1),
                      "t_cpu_us": round(median([c[1] for c in comp]) * 1e3, 1)})
        log(f"[share] split at {begin}{' q_first' if q_first else ''}: {ms * 1e3:.1f} us/step "
            f"(host {sweep[-1]['host_ms'] * 1e3:.1f} us)")
    best = min(sweep, key=lambda e: e["ms_per_step"])
    per_pos = case.kv_bytes_per_token() * B
    out = {
        "mode": "host_share",
        "workload": "split_128k: " + DESCR["split_128k"].split(",")[0] + ", B4 x 128K, CPU share by policy",
        "host_threads": threads,
        "calibration": {
            "gpu": {"B_ns_per_position": round(B_cost * 1e6, 4), "C_gpu_us": round(C_gpu * 1e3, 2),
                    "points_us": [[n, round(ms * 1e3, 2)] for n, ms in gpu_pts]},
            "cpu": {"A_ns_per_position": round(A_cost * 1e6, 3), "C_cpu_us": round(C_cpu * 1e3, 2),
                    "points_us": [[n, round(ms * 1e3, 2)] for n, ms, _ in cpu_pts],
                    "host_compute_us": [[n, round(h * 1e3, 2)] for n, _, h in cpu_pts],
                    "wide_points_us": [[n, round(ms * 1e3, 2)] for n, ms, _ in cpu_wide],
                    "wide_r": round(r_wide, 6),
                    "host_GBps_at_largest": round(cpu_pts[-1][0] * per_pos / (cpu_pts[-1][2] * 1e-3) / 1e9, 2)},
        },
        "policy": {"r": round(r_pol, 6), "p": round(B_cost / (A_cost + B_cost), 6),
                   "cpu_positions": begin_pol},
        "gpu_only_ms_per_step": round(gpu_only, 5),
        "sweep": sweep,
        "measured_best": best,
    }
    print(json.dumps(out), flush=True)


def write_side_bench(args):
    """The write side on the Qwen3-30B-A3B-shaped layer (16 sequences, 4 KV heads, head dim 128,
    bf16, 16-token blocks): 32K-token prefills are appended and placed, then 2 * D decode steps
    each append one token per sequence through the GPU view and flush the staging window
    (D = 256).  Two routings: every batch to the GPU share (what the share policy picks on
    MI355X, where a GPU position costs ~1/100 of a host one) and every batch to the CPU share
    (device-to-host block copies, the most a flush can cost)."""
    import numpy as np
    import torch

    from paged_kv_cache_mla_amd import _lib
    from paged_kv_cache_mla_amd.api import (KVStore, Pool, ShareController, append_kv,
                                            block_bytes)

    _lib.load()
    torch.cuda.set_device(0)
    B, bs, hkv, d, D = 16, 16, 4, 128, 256
    warm = 64
    L0 = 32768 - D - warm
    steps = 2 * D
    bb = block_bytes(bs, hkv, d, d, "bf16", False)
    per_seq = (L0 + steps + warm) // bs + 2 * (D // bs) + 2
    timer = HipTimer()
    out = {"mode": "write_side",
           "workload": "Qwen3-30B-A3B-shaped layer: 16 x 32K, 4 KV heads, d 128, bf16, bs 16, D 256",
           "append_bytes_per_step": B * hkv * 2 * d * 2}
    # a first, unreported pass takes the process's one-time costs (measured: the first pass of
    # this loop runs 4-6x slower on the host than any later one, whatever its routing)
    for routing in ("warm-up", "gpu", "cpu"):
        dev_region = torch.empty(B * per_seq * bb // 2, dtype=torch.int16, device="cuda")
        host_blocks = B * ((steps + warm) // bs + 2 * (D // bs)) + 8
        host_region = torch.empty(host_blocks * bb // 2, dtype=torch.int16, pin_memory=True)
        lay = (bs, hkv, d, d, "bf16", False)
        dev_pool = Pool(*lay, [(dev_region.data_ptr(), B * per_seq)], seed=1)
        host_pool = Pool(*lay, [(host_region.data_ptr(), host_blocks)], seed=2)
        # the prefill stays on the GPU share in both cases; decode batches go where the
        # routing under test sends them.  B = 0 gives r = 0 at every length (all GPU).
        # A = 0 with C_CPU = L0 + 8 gives r(L0) = 0 but r(L) L = L - L0 - 8 afterwards, so
        # every D-token batch after the prefill goes to the CPU.
        if routing == "cpu":
            ctls = [ShareController(0.0, 1.0, float(L0 + 8), 0.0) for _ in range(B)]
        else:
            ctls = [ShareController(1.0, 0.0, 0.0, 0.0) for _ in range(B)]
        store = KVStore(dev_pool, host_pool, B, D, per_seq, ctls)
        store.reserve([L0] * B)
        gt, gl, _, _ = store.views()
        table_dev = torch.from_numpy(gt).cuda()
        log(f"[write] {routing}: appending {B} x {L0} prefill tokens")
        sp0 = torch.cuda.current_stream().cuda_stream
        pre_ms = 0.0
        pos = torch.zeros(1, dtype=torch.int32, device="cuda")
        for b in range(B):
            k = torch.randn(1, L0, hkv, d, device="cuda", dtype=torch.bfloat16).view(torch.int16)
            v = torch.randn(1, L0, hkv, d, device="cuda", dtype=torch.bfloat16).view(torch.int16)
            e0, e1 = timer.event(), timer.event()
            timer.record(e0, sp0)
            append_kv(dev_pool, k, v, _lib.BF16, table_dev[b:b + 1], per_seq, pos)
            timer.record(e1, sp0)
            torch.cuda.synchronize()
            pre_ms += timer.elapsed_ms(e0, e1)
        store.commit([L0] * B)
        store.place_prefill()
        torch.cuda.synchronize()
        gt, gl, _, _ = store.views()
        table_dev.copy_(torch.from_numpy(gt))
        pos_dev = torch.from_numpy(gl.copy()).cuda()
        k1 = torch.randn(B, 1, hkv, d, device="cuda", dtype=torch.bfloat16).view(torch.int16)
        v1 = torch.randn(B, 1, hkv, d, device="cuda", dtype=torch.bfloat16).view(torch.int16)
        ones = np.ones(B, np.int32)
        evs = [(timer.event(), timer.event()) for _ in range(steps + warm)]
        sp = torch.cuda.current_stream().cuda_stream
        host_s, store_s, flush_s, n_flush = 0.0, 0.0, [], 0
        torch.cuda.synchronize()
        for i in range(steps + warm):
            if i == warm:   # the first steps are warm-up (first launches, page faults)
                torch.cuda.synchronize()
                host_s, store_s, flush_s, n_flush = 0.0, 0.0, [], 0
                t_all = time.perf_counter()
            # a serving loop's driving of the store: views are read and uploaded only when
            # they change; otherwise the device positions advance on the device
            t0 = time.perf_counter()
            changed = store.reserve(ones)
            store_s += time.perf_counter() - t0
            if changed:
                gt, gl, _, _ = store.views()
                table_dev.copy_(torch.from_numpy(gt))
            timer.record(evs[i][0], sp)
            append_kv(dev_pool, k1, v1, _lib.BF16, table_dev, per_seq, pos_dev)
            timer.record(evs[i][1], sp)
            ts = time.perf_counter()
            store.commit(ones)
            changed = store.flush()
            store_s += time.perf_counter() - ts
            if changed:
                torch.cuda.synchronize()   # the copies of this flush, timed with it
                flush_s.append(time.perf_counter() - ts)
                n_flush += 1
                gt, gl, _, _ = store.views()
                table_dev.copy_(torch.from_numpy(gt))
                pos_dev.copy_(torch.from_numpy(gl))
            else:
                pos_dev += 1
            host_s += time.perf_counter() - t0
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_all
        app_us = [timer.elapsed_ms(a, b_) * 1e3 for a, b_ in evs[warm:]]
        gt, gl, ct, cl = store.views()
        pre_bytes = B * L0 * hkv * 2 * d * 2
        res = {"prefill_append_us_per_seq": round(pre_ms * 1e3 / B, 1),
               "prefill_append_GBps": round(pre_bytes / (pre_ms * 1e-3) / 1e9, 1),
               "steps": steps, "append_us": round(float(np.mean(app_us)), 2),
               "wall_us_per_step": round(wall / steps * 1e6, 2),
               "host_us_per_step": round(host_s / steps * 1e6, 2),
               "store_calls_us_per_step": round(store_s / steps * 1e6, 2),
               "gpu_view_tokens": int(gl.sum()), "cpu_view_tokens": int(cl.sum())}
        if flush_s:
            copied = B * D * hkv * 2 * d * 2
            fl = float(np.median(flush_s))
            res.update({"flushes_to_cpu": n_flush, "flush_us": round(fl * 1e6, 1),
                        "flush_bytes": copied, "flush_GBps": round(copied / fl / 1e9, 2),
                        "flush_us_amortized_per_step": round(fl * 1e6 / D, 2)})
        if routing != "warm-up":
            out[routing + "_routing"] = res
        log(f"[write] {routing}: {res}")
        store.close()
        del dev_region, host_region
    print(json.dumps(out), flush=True)


def sparse_bench(args):
    """Block-level sparse decode on the Qwen3-30B-A3B-shaped layer (16 x 32K, 4 KV heads, d 128,
    bf16): every sequence selects a seeded random `density` share of its 16-token blocks;
    kvattn_select_blocks builds the sub-tables on the device, then decode_partial and the merge
    run on them.  Reported against the selected KV bytes and next to the dense step."""
    import numpy as np
    import torch

    from paged_kv_cache_mla_amd import _lib
    from paged_kv_cache_mla_amd.api import choose_group_parts, decode_partial, merge_lse, select_blocks
    from paged_kv_cache_mla_amd.session import DeviceCase
    from synth import make_case

    _lib.load()
    torch.cuda.set_device(0)
    density = args.sparse
    case = make_case("gqa_32k", "full")
    dc = DeviceCase(case)
    B, bs = case.batch, case.block_size
    nb = -(-int(case.ctx_lens.max()) // bs)
    k = max(1, int(round(nb * density)))
    rng = np.random.default_rng(3)
    sel = np.stack([rng.choice(nb, k, replace=False) for _ in range(B)]).astype(np.int32)
    dev = "cuda"
    sel_dev = torch.from_numpy(sel).to(dev)
    sub_table = torch.empty((B, k), dtype=torch.int32, device=dev)
    seq_sub = torch.zeros((3, B), dtype=torch.int32, device=dev)
    seq_sub[2] = int(case.part_tokens[0])
    bound = np.full(B, k * bs, np.int32)
    parts = -(-(k * bs) // int(case.part_tokens[0]))
    # grouping saves partial writes but costs parallelism: the library's choice for the
    # selection's bounds (with a few partitions per (sequence, KV head) it does not group)
    g = args.group_parts or choose_group_parts(dc.pool, case.num_q_heads, bound, None,
                                               case.part_tokens)
    max_parts = -(-parts // g)
    o_part = torch.empty((B, case.num_q_heads, max_parts, case.head_dim_v), dtype=torch.float32, device=dev)
    lse_part = torch.empty((B, case.num_q_heads, max_parts), dtype=torch.float32, device=dev)
    nparts = torch.empty(B, dtype=torch.int32, device=dev)
    o = torch.empty((B, case.num_q_heads, case.head_dim_v), dtype=torch.float32, device=dev)
    lse = torch.empty((B, case.num_q_heads), dtype=torch.float32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)

    def step(evs=None):
        sp = torch.cuda.current_stream().cuda_stream
        if evs:
            timer.record(evs[0], sp)
        select_blocks(dc.step.table_dev, case.max_blocks, dc.step.seq_dev[0], bs, sel_dev,
                      sub_table, seq_sub[0], err)
        if evs:
            timer.record(evs[1], sp)
        decode_partial(dc.pool, dc.q, dc.q_dtype, case.num_q_heads, case.scale, sub_table, k,
                       bound, None, case.part_tokens, seq_sub, max_parts, o_part, lse_part,
                       nparts, err, None, g)
        if evs:
            timer.record(evs[2], sp)
        merge_lse(o_part, lse_part, nparts, B, case.num_q_heads, max_parts, case.head_dim_v, o,
                  None, None, lse)

    timer = HipTimer()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        raise RuntimeError(f"error flag {int(err.item())}")
    evs = [(timer.event(), timer.event(), timer.event()) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    t_sel = float(np.mean([timer.elapsed_ms(a, b_) for a, b_, _ in evs])) * 1e3
    t_dec = float(np.mean([timer.elapsed_ms(b_, c) for _, b_, c in evs])) * 1e3
    kv = B * k * bs * case.kv_bytes_per_token()
    dense = _time_steps(torch, lambda: dc.step.run(dc.q, dc.q_dtype, case.scale), args.steps,
                        args.warmup)
    out = {"mode": "sparse", "workload": "Qwen3-30B-A3B-shaped layer: 16 x 32K, 4 KV heads, d 128, bf16, bs 16",
           "density": density, "selected_blocks_per_seq": k, "selected_kv_bytes": kv,
           "group_parts": g, "ms_per_step": round(ms, 5), "select_us": round(t_sel, 2),
           "decode_partial_us": round(t_dec, 2),
           "selected_kv_GBps": round(kv / (t_dec * 1e-6) / 1e9, 1),
           "dense_ms_per_step": round(dense, 5),
           "speedup_vs_dense": round(dense / ms, 2)}
    print(json.dumps(out), flush=True)


def growth_bench(args):
    """Run-time pool growth over HIP virtual memory: time to back a range with new pages, to
    move pages from an "expert weights" range into the KV range (with and without the device
    synchronisation that guards pages still in use), and to grow the pool over them; at the
    step size of the pages' own controller (4 expert groups of 6 MiB) and at 1 GiB, in 2 MiB
    chunks, on the layout of the 16 x 32K layer."""
    import numpy as np
    import torch

    from paged_kv_cache_mla_amd import _lib
    from paged_kv_cache_mla_amd.api import Pool, VMMRange, block_bytes

    _lib.load()
    torch.cuda.set_device(0)
    torch.zeros(1, device="cuda")
    chunk = 2 << 20
    bb = block_bytes(16, 4, 128, 128, "bf16", False)
    out = {"mode": "growth", "chunk_bytes": chunk, "block_bytes": bb, "steps": []}
    for size in (24 << 20, 1 << 30):
        res = {"bytes": size}
        for trial in range(4):   # the first trial takes one-time costs; the last three are kept
            expert = VMMRange(2 * size, chunk)
            kv = VMMRange(2 * size, chunk)
            torch.cuda.synchronize()
            t = time.perf_counter()
            expert.map_new(0, size)
            t_map = time.perf_counter() - t
            t = time.perf_counter()
            expert.move_to(0, kv, 0, size, sync_device=True)
            t_move = time.perf_counter() - t
            t = time.perf_counter()
            kv.move_to(0, expert, size, size, sync_device=False)   # idle device: no guard needed
            t_move_ns = time.perf_counter() - t
            base = torch.empty(bb // 2, dtype=torch.int16, device="cuda")
            pool = Pool(16, 4, 128, 128, "bf16", False, [(base.data_ptr(), 1)])
            expert.move_to(size, kv, 0, size, sync_device=False)
            t = time.perf_counter()
            pool.add_region(kv.base, size // bb)
            st, _, _ = pool.block_table([16 * (size // bb)], size // bb)
            t_pool = time.perf_counter() - t
            assert st == _lib.OK
            pool.close()
            kv.close()
            expert.close()
            if trial:
                for k_, v_ in (("map_new_us", t_map), ("move_sync_us", t_move),
                               ("move_nosync_us", t_move_ns), ("pool_grow_and_claim_us", t_pool)):
                    res.setdefault(k_, []).append(v_ * 1e6)
        for k_ in list(res):
            if isinstance(res[k_], list):
                res[k_] = round(float(np.median(res[k_])), 1)
        res["blocks"] = size // bb
        res["move_us_per_chunk"] = round(res["move_nosync_us"] / (size // chunk), 2)
        out["steps"].append(res)
        log(f"[growth] {res}")
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa_32k", choices=sorted(DESCR))
    ap.add_argument("--r", type=float, default=0.5, help="host share of split_128k")
    ap.add_argument("--group-parts", type=int, default=0,
                    help="partitions merged on chip per written partial (default 0: the library's choice)")
    ap.add_argument("--span-parts", type=int, default=0,
                    help="pools with shared blocks: partitions per wave item of the decode plan "
                         "(default 0: the library's choice)")
    ap.add_argument("--plan", action="store_true",
                    help="run the step from a decode plan even when the pool holds no shared blocks")
    ap.add_argument("--claim", action="store_true",
                    help="pools with shared blocks: run the plan with work counters (workgroups "
                         "take the next unit when done) instead of one unit per workgroup")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--host-share", choices=["off", "policy"], default="off",
                    help="policy: time the split workload with a native CPU share sized by the "
                         "share policy (prints its own JSON line instead of the bench line)")
    ap.add_argument("--write-side", action="store_true",
                    help="time appends and staging-window flushes on the 16 x 32K layer "
                         "(prints its own JSON line instead of the bench line)")
    ap.add_argument("--sparse", type=float, default=0.0, metavar="DENSITY",
                    help="time block-level sparse decode of the 16 x 32K layer at this block "
                         "density (prints its own JSON line instead of the bench line)")
    ap.add_argument("--growth", action="store_true",
                    help="time run-time pool growth over moved virtual-memory pages (prints its own "
                         "JSON line instead of the bench line)")
    ap.add_argument("--host-threads", type=int, default=0,
                    help="host threads for --host-share (default: min(16, usable CPUs) - 1)")
    ap.add_argument("--summarize", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "STATS_DIR"),
                    help="write profiles/decode_partial_and_merge.<workload>.md from rocprofv3 "
                         "output directories (no GPU needed) and exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="PMC_DIR",
                    help="write profiles/counters.<workload>.md from rocprofv3 --pmc output "
                         "directories (no GPU needed) and exit")
    ap.add_argument("--command", action="append", default=[],
                    help="with --summarize / --summarize-counters: a command line to record")
    args = ap.parse_args()
    if args.summarize_counters:
        print(summarize_counters(args.workload, args.summarize_counters,
                                 os.path.join(ROOT, "profiles", f"counters.{args.workload}.md"),
                                 args.command))
        return
    if args.summarize:
        print(summarize_profile(args.workload, *args.summarize, profile_path(args.workload),
                                args.command))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this library has "
              "no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    if args.host_share == "policy":
        host_share_bench(args)
        return
    if args.write_side:
        write_side_bench(args)
        return
    if args.sparse > 0:
        sparse_bench(args)
        return
    if args.growth:
        growth_bench(args)
        return

    import numpy as np
    import torch

    from paged_kv_cache_mla_amd import _lib
    from paged_kv_cache_mla_amd.session import DeviceCase
    from synth import make_case

    _lib.load()
    torch.cuda.set_device(0)
    log(f"[bench] generating {args.workload} (full)")
    kw = {"r": args.r} if args.workload == "split_128k" else {}
    case = make_case(args.workload, "full" if args.workload != "tiny_fp32" else "small", **kw)
    dc = DeviceCase(case, group_parts=args.group_parts, span_parts=args.span_parts,
                    claim=args.claim, plan=True if args.plan else None)
    group_parts = dc.step.group_parts
    log(f"[bench] uploaded (group_parts {group_parts}{', the library choice' if dc.step.auto else ''})")
    o_ext = lse_ext = None
    cpu_share = None
    if case.ext_regions is not None:
        if not args.no_cpu_baseline:
            log("[bench] the host share [0, r L) of every sequence, by the oracle on the host")
            o_np, l_np, secs, toks = oracle_host_share(case)
            cpu_share = {"kind": "oracle", "tokens": toks, "seconds": round(secs, 3),
                         "kv_bytes": toks * case.kv_bytes_per_token(),
                         "GBps": round(toks * case.kv_bytes_per_token() / secs / 1e9, 3),
                         "cores": len(os.sched_getaffinity(0)),
                         "note": "the host share's partial merged by the timed steps"}
        else:
            # without the oracle leg the partial's values are a seeded stand-in: they do not
            # change the work of the step
            rng = np.random.default_rng(0)
            o_np = rng.standard_normal((case.batch, case.num_q_heads, case.head_dim_v))
            l_np = rng.standard_normal((case.batch, case.num_q_heads))
        o_ext = torch.from_numpy(o_np.astype(np.float32)).cuda()
        lse_ext = torch.from_numpy(l_np.astype(np.float32)).cuda()

    for _ in range(args.warmup):
        dc.run(o_ext, lse_ext)
    torch.cuda.synchronize()
    if int(dc.step.err.item()) != 0:
        raise RuntimeError(f"kernel error flag {int(dc.step.err.item())}")

    # The dominant kernel's duration: HIP events recorded on the launch stream around every
    # decode_partial of the timed loop.  They are created without the system-scope fence, so
    # recording one does not write back and invalidate the caches (torch's timing events do,
    # which adds ~3 us per event to the step on MI355X).
    timer = HipTimer()
    sp = torch.cuda.current_stream().cuda_stream
    evs = [(timer.event(), timer.event()) for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        timer.record(evs[i][0], sp)
        dc.partial()
        timer.record(evs[i][1], sp)
        dc.merge(o_ext, lse_ext)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_part = [timer.elapsed_ms(a, b) for a, b in evs]
    # a step's device time: from one decode_partial's start to the next one's (the steps are
    # enqueued back to back, so this spans the partial, the merge and the gaps between them)
    t_steps_ev = [timer.elapsed_ms(evs[i][0], evs[i + 1][0]) for i in range(args.steps - 1)] or [0.0]
    ms_step = wall * 1e3 / args.steps

    # The access pattern's own ceiling, outside the timed region: the gather probe issues the
    # decode kernel's loads (same grid, waves, table lookups and cache hints) with no arithmetic.
    gather = None
    try:
        if dc.step.plan is not None:
            raise NotImplementedError("the gather probe mirrors the per-sequence launch, not a plan")
        xsum = torch.zeros(case.batch * case.num_kv_heads, dtype=torch.int32, device="cuda")
        for _ in range(2):
            dc.step.probe(xsum)
        pevs = [(timer.event(), timer.event()) for _ in range(args.steps)]
        for i in range(args.steps):
            timer.record(pevs[i][0], sp)
            dc.step.probe(xsum)
            timer.record(pevs[i][1], sp)
        torch.cuda.synchronize()
        gather = float(np.mean([timer.elapsed_ms(a, b) for a, b in pevs]))
    except (_lib.KvattnError, NotImplementedError) as e:  # layouts the probe does not serve
        log(f"[bench] no gather probe for this layout: {e}")

    bpt = case.kv_bytes_per_token()
    slots_logical, slots_unique = kv_token_slots(case)
    kv_bytes = slots_logical * bpt          # every sequence's K/V range, as it attends to it
    kv_unique = slots_unique * bpt          # what must cross HBM: shared blocks once
    n_parts_total = int(dc.step.nparts.sum().item())
    q_bytes = case.q.nbytes
    table_bytes = int(sum(-(-(int(c) - (0 if case.tok_begin is None else int(case.tok_begin[b]))) //
                            case.block_size) for b, c in enumerate(case.ctx_lens))) * 4
    part_bytes = n_parts_total * case.num_q_heads * (case.head_dim_v + 1) * 4
    out_bytes = case.batch * case.num_q_heads * (case.head_dim_v + 1) * 4
    ext_bytes = out_bytes if o_ext is not None else 0
    # decode_partial: K/V once, q, table, partials written; the step adds the merge's reads of
    # the partials (and of the external partial) and its output
    kernel_bytes = kv_unique + q_bytes + table_bytes + part_bytes
    alg_bytes = kernel_bytes + part_bytes + ext_bytes + out_bytes
    flops = slots_logical * case.num_q_heads * 2 * (case.head_dim_k + case.head_dim_v)
    avg_part_ms = float(np.mean(t_part))
    achieved = kernel_bytes / (avg_part_ms * 1e-3) / 1e9
    value = kv_bytes / (ms_step * 1e-3) / 1e9
    layers = LAYERS.get(args.workload)
    copy_gbps = copy_bandwidth(torch)

    out = {
        "metric": "decode-attn KV GB/s (% of 8 TB/s HBM) + tokens/s, 30B-A3B shape bs16x32K",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if case.dtype == "bf16" else "f32",
        "data": "synthetic",
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(case.batch / (ms_step * 1e-3), 1),
        "attn_only_model_tokens_per_s": (round(case.batch / (layers * ms_step * 1e-3), 1)
                                         if layers else None),
        "t_partial_us": round(avg_part_ms * 1e3, 2),
        # the rest of the step: the merge kernel plus the launch gaps around it
        "t_merge_and_gaps_us": round((ms_step - avg_part_ms) * 1e3, 2),
        "t_step_median_us": round(float(np.median(t_steps_ev)) * 1e3, 2),
        "t_partial_median_us": round(float(np.median(t_part)) * 1e3, 2),
        "kv_bytes": kv_bytes,
        "alg_bytes": alg_bytes,
        "flops": flops,
        "copy_GBps": round(copy_gbps, 1),
        "config": {
            "workload": args.workload + ": " + DESCR[args.workload],
            "batch": case.batch,
            "ctx_len": int(case.ctx_lens.max()),
            "q_heads": case.num_q_heads,
            "kv_heads": case.num_kv_heads,
            "head_dim_k": case.head_dim_k,
            "head_dim_v": case.head_dim_v,
            "block_size": case.block_size,
            "part_tokens": int(case.part_tokens[0]),
            # the plan decomposes by its own wave items: no group_parts
            "group_parts": group_parts if dc.step.plan is None else None,
            "group_parts_auto": dc.step.auto,
            **({"plan_workgroups": dc.step.n_groups, "plan_max_parts": dc.step.max_parts,
                "span_parts": args.span_parts, "claim": args.claim}
               if dc.step.plan is not None else {}),
            "kv_dtype": case.dtype,
            "device_tokens": case.device_tokens(),
            **({"r": args.r} if args.workload == "split_128k" else {}),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_partial",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": stored_traffic(args.workload),
            "alg_bytes_per_launch": kernel_bytes,
            "avg_launch_us": round(avg_part_ms * 1e3, 2),
        },
    }
    if slots_unique != slots_logical:
        traffic = out["roofline"]["traffic"]
        out["shared_kv"] = {
            "kv_bytes_logical": kv_bytes,
            "kv_bytes_unique": kv_unique,
            "hbm_bytes_counter": traffic,
            "token_slots_logical": slots_logical,
            "token_slots_unique": slots_unique,
            "unique_fraction": round(slots_unique / slots_logical, 4),
            "unique_KV_GBps": round(kv_unique / (ms_step * 1e-3) / 1e9, 1),
            "note": "value counts every sequence's K/V (logical); the roofline counts each "
                    "shared block once (unique); hbm_bytes_counter is the rocprofv3 FETCH+WRITE "
                    "of decode_partial (null when taken on other kernel source)",
        }
    if cpu_share is not None:
        out["cpu_share"] = cpu_share
    if gather is not None:
        out["gather_ceiling"] = {
            "kernel": "gather probe: the decode kernel's loads, no arithmetic",
            "avg_launch_us": round(gather * 1e3, 2),
            "kv_GBps": round(kv_bytes / (gather * 1e-3) / 1e9, 1),
            "decode_frac_of_probe": round(gather / avg_part_ms, 4),
        }
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
