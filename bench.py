"""Benchmark: causal shared-latent MLA prefill on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-rows]

Headline workload: DeepSeek-V3-shaped absorbed MLA prefill, B=1, 128 query
heads over one shared latent KV head, N=8192 causal, dk=576 (512 latent + 64
RoPE), dv=512, bf16 inputs ~N(0,1) (seed 0), scale 1/sqrt(192).  A step is one
mla_fwd call over that batch, inputs resident in HBM.  Throughput counts only
algorithmic flops: visible (query, head, key) triples x (2*dk + 2*dv).

Rank 0 prints ONE JSON line with the headline, its roofline against the
dense bf16 MFMA peak, the fp64 CPU oracle timed on a bounded sample of the
same workload, and measured lines for the other steps of the path (one-device
ring with LSE folds, split varlen ring step, sparse top-k, standalone merge,
token-generation decode, V-up projection, and the headline shape in FP8).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 MFMA: 256 CU x 8192 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "causal MLA prefill TFLOP/s and % of bf16 MFMA peak on 1 MI355X"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_latent_dsv3_prefill_hbm_traffic.json")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "attn_fwd_latent_dsv3_prefill_counters.md")
COUNTER_CLOCK_KERNEL = "LatentCfg, 0"   # the headline kernel's name in the counter runs
N_XCD = 8
KERNEL_SRCS = [os.path.join(ROOT, "ring_chunk_attention_amd", "csrc", f)
               for f in ("mla_attn.hip", "mla_attn_kernels.inc", "mla_attn_body.inc", "mla_qk_chain.inc")]


def causal_pairs(n_q: int, n_kv: int, q_offset: int = 0, kv_offset: int = 0) -> int:
    """Visible (query, key) pairs of one head under the causal mask."""
    i = np.arange(n_q, dtype=np.int64)
    vis = np.clip(q_offset + i - kv_offset + 1, 0, n_kv)
    return int(vis.sum())


def _strip_comments(src: str) -> str:
    """C++ source without its comments and trailing blanks (string literals
    in these files hold no comment markers)."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(l.rstrip() for l in src.splitlines() if l.strip())


def kernel_hash() -> str:
    """Hash of the attention kernel's code (the launcher file, the kernel
    template and body it includes, and the generated Q.K chain), comments
    left out: a change of wording is not a change of the kernel."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path) as f:
            h.update(_strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


_HOLD = {}


def hold_stream():
    """Enqueue about 1 ms of unrelated GPU work (a 8192^3 bf16 matmul) on
    the current stream, so that the calls enqueued behind it while it runs
    reach the GPU back to back: a call shorter than the Python binding's
    marshalling would otherwise be timed with that host latency in it."""
    import torch
    if "a" not in _HOLD:
        _HOLD["a"] = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
        _HOLD["c"] = torch.empty_like(_HOLD["a"])
    torch.mm(_HOLD["a"], _HOLD["a"], out=_HOLD["c"])


def time_launches(fn, steps: int, warmup: int, hold: bool = False, per_launch: bool = True):
    """Warm up, then time `steps` calls with HIP events on the current stream;
    returns (ms per step over the whole region, mean ms per launch, min ms per
    launch, median ms per launch).  ``per_launch`` False: only the region is bracketed by events
    (each event record is a packet of its own on the queue, a few
    microseconds beside short calls) and the per-launch figures are the
    region's mean.  ``hold``: the calls also queue up behind hold_stream()
    first, so that a call shorter than its own host-side marshalling is timed
    on the GPU alone (the standalone merge)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    if hold:
        hold_stream()
    t0.record(stream)
    for k in range(steps):
        if per_launch:
            starts[k].record(stream)
        fn()
        if per_launch:
            ends[k].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    region = t0.elapsed_time(t1) / steps
    if not per_launch:
        return region, region, region, region
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return region, float(np.mean(per)), float(np.min(per)), float(np.median(per))


SCLK_FILES = ("/sys/class/drm/card0/device/pp_dpm_sclk",)


class ClockSampler:
    """Samples the GPU engine clock while work runs: the driver's
    pp_dpm_sclk lists the clock levels and marks the current one with '*'
    (the current engine clock in MHz).  Used as a context manager around a
    timed region; `mhz` is the list of samples."""

    def __init__(self, period_s: float = 0.002):
        import threading
        self.period = period_s
        self.mhz = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)
        self.path = next((p for p in SCLK_FILES if os.path.exists(p)), None)

    def _read(self):
        with open(self.path) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    m = re.search(r"(\d+)\s*[Mm]hz", line)
                    if m:
                        return int(m.group(1))
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read()
            except OSError:
                return
            if v:
                self.mhz.append(v)
            time.sleep(self.period)

    def __enter__(self):
        if self.path:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.path:
            self._thread.join()

    def summary(self):
        """Median of the samples taken above idle (a busy engine runs above
        1 GHz; idle gaps between launches read a few hundred MHz)."""
        busy = sorted(v for v in self.mhz if v >= 1000)
        if not busy:
            return None
        return {"median_mhz": busy[len(busy) // 2], "min_mhz": busy[0], "max_mhz": busy[-1],
                "samples": len(busy), "source": self.path}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, budget_s: float = 12.0):
    """The fp64 oracle on whole heads of the same workload until the budget is
    spent; throughput on the same algorithmic flop count."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    B, H, N, dk = case.q.shape
    flops = 0
    heads = 0
    t0 = time.perf_counter()
    while heads < H and time.perf_counter() - t0 < budget_s:
        oracle.dense_mla(case.q[:, heads:heads + 1], case.kv, 512, case.scale)
        flops += causal_pairs(N, N) * (2 * 576 + 2 * 512)
        heads += 1
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(), "logical_cpus_visible": len(os.sched_getaffinity(0)),
            "sample": f"fp64 NumPy oracle on heads 0..{heads - 1} of {H} (all {N} causal rows each), "
                      f"{dt:.1f} s wall, same flop count per head as the GPU"}


ROW_TRAFFIC = {   # row -> (kernel name substring, committed traffic summary)
    "sparse": ("LatentCfg, 3>", os.path.join(ROOT, "profiles", "attn_fwd_sparse_topk_s4096_k2048_hbm_traffic.json")),
    "decode": ("LatentCfg, 3>", os.path.join(ROOT, "profiles", "attn_fwd_decode_b64_kv8192_hbm_traffic.json")),
}


def counter_clock(path=COUNTERS_FILE):
    """The headline kernel's shader clock (MHz) from its committed counter
    summary (GRBM_GUI_ACTIVE per XCD over the dispatch), or None when the
    summary was taken on other kernel code."""
    try:
        text = open(path).read()
    except OSError:
        return None
    h = re.search(r"Kernel code hash: `([0-9a-f]+)`", text)
    m = re.search(r"\| shader clock over the dispatch \(MHz\) \| ([0-9.]+) \|", text)
    if not h or not m or h.group(1) != kernel_hash():
        return None
    return float(m.group(1))


def measured_traffic(path=TRAFFIC_FILE, full=False):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel source (``full``: the whole summary)."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha256_16") != kernel_hash():
        return None
    return t if full else t.get("bytes_per_launch")


ATTN_KERNEL = "attn_fwd_kernel<mla::(anonymous namespace)::LatentCfg"
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 30


def _csvs(folder, suffix):
    import glob
    return sorted(glob.glob(os.path.join(folder, "**", "*" + suffix), recursive=True))


def _short_kernel(name):
    name = name.replace("(anonymous namespace)::", "").replace("mla::", "")
    if name.startswith("void "):
        name = name[5:]
    depth = 0
    for k, ch in enumerate(name):  # drop the argument list
        depth += ch == "<"
        depth -= ch == ">"
        if ch == "(" and depth == 0:
            name = name[:k]
            break
    return name if len(name) <= 90 else name[:87] + "..."


def summarize_stats(folder, out_path, cmd):
    """Short markdown summary of a `rocprofv3 --kernel-trace --stats
    --output-format csv` run: launches grouped by kernel and grid size, with the
    mean duration over all launches and over all but the first (warm-up) one."""
    import csv
    files = _csvs(folder, "kernel_trace.csv")
    if not files:
        sys.exit(f"no *kernel_trace.csv under {folder}")
    groups = {}
    for r in csv.DictReader(open(files[0])):
        key = (_short_kernel(r["Kernel_Name"]), int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(v) for v in groups.values())
    lines = ["# Kernel durations: " + os.path.basename(out_path).rsplit(".", 1)[0], "",
             "Command (from the repository root, on one MI355X):", "", "    " + cmd, "",
             "Launches grouped by kernel and grid (workgroups); durations in microseconds "
             "from the kernel trace; `steady` leaves out the first launch of the group.", "",
             "| kernel | workgroups | calls | mean | steady mean | min | max | share |",
             "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for (name, wgs), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        steady = d[1:] if len(d) > 1 else d
        lines.append(f"| `{name}` | {wgs} | {len(d)} | {sum(d) / len(d):.1f} | "
                     f"{sum(steady) / len(steady):.1f} | {min(d):.1f} | {max(d):.1f} | "
                     f"{100 * sum(d) / total:.1f}% |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_counters(folders, kernel, out_path, cmds):
    """Markdown summary of `rocprofv3 --pmc` csv runs (one folder per pass):
    each counter's value summed over the dispatch's sampled units, for the last
    dispatch of the kernel whose name contains `kernel`, and the ratios the
    design cites (SIMD and CU busy fractions use the per-XCD GRBM_GUI_ACTIVE
    as the clock count)."""
    import csv
    vals = {}
    clock_mhz = None
    for folder in folders:
        files = _csvs(folder, "counter_collection.csv")
        if not files:
            sys.exit(f"no *counter_collection.csv under {folder}")
        per, dur = {}, {}
        for r in csv.DictReader(open(files[0])):
            if kernel not in r["Kernel_Name"]:
                continue
            d = per.setdefault(int(r["Dispatch_Id"]), {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            if r.get("End_Timestamp") and r.get("Start_Timestamp"):
                dur[int(r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        if not per:
            sys.exit(f"no dispatch of a kernel named like {kernel!r} in {folder}")
        last = max(per)
        vals.update(per[last])
        if clock_mhz is None and "GRBM_GUI_ACTIVE" in per[last] and dur.get(last, 0) > 0:
            # GRBM_GUI_ACTIVE counts shader-clock cycles per XCD (summed over the 8)
            clock_mhz = per[last]["GRBM_GUI_ACTIVE"] / N_XCD / dur[last] * 1e3
    lines = ["# Counters: " + os.path.basename(out_path).rsplit(".", 1)[0], "",
             "Commands (from the repository root, on one MI355X; one pass each):", ""]
    lines += ["    " + c for c in cmds]
    lines += ["", f"Last dispatch of the kernel named like `{kernel}`; values summed over the units "
              "rocprofv3 reports.", "", "| counter | value |", "|---|---:|"]
    lines += [f"| `{k}` | {v:.4g} |" for k, v in sorted(vals.items())]
    clk = vals.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD   # per XCD
    derived = []
    if clock_mhz:
        derived.append(("shader clock over the dispatch (MHz)", clock_mhz))
    if clk:
        if "SQ_VALU_MFMA_BUSY_CYCLES" in vals:
            derived.append(("MFMA busy (per SIMD)", vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (clk * 1024)))
        if "SQ_ACTIVE_INST_VALU" in vals:
            derived.append(("VALU busy (per CU, 4-cycle issue)", vals["SQ_ACTIVE_INST_VALU"] / (clk * 256)))
    if vals.get("SQ_WAVE_CYCLES"):
        for k, label in (("SQ_WAIT_ANY", "waves waiting on a memory counter"),
                         ("SQ_WAIT_INST_ANY", "waves waiting to issue")):
            if k in vals:
                derived.append((label, vals[k] / vals["SQ_WAVE_CYCLES"]))
    if vals.get("TCC_HIT_sum") is not None and vals.get("TCC_MISS_sum"):
        derived.append(("L2 hit rate", vals["TCC_HIT_sum"] / (vals["TCC_HIT_sum"] + vals["TCC_MISS_sum"])))
    if vals.get("SQ_WAVE_CYCLES") and "SQ_WAIT_INST_LDS" in vals:
        derived.append(("waves waiting on an LDS instruction", vals["SQ_WAIT_INST_LDS"] / vals["SQ_WAVE_CYCLES"]))
    if vals.get("SQ_INSTS_MFMA"):
        for k in ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS"):
            if k in vals:
                derived.append((f"{k} per MFMA", vals[k] / vals["SQ_INSTS_MFMA"]))
    if derived:
        lines += ["", "| derived | value |", "|---|---:|"]
        lines += [f"| {k} | {v:.4g} |" if "MHz" in k else f"| {k} | {v:.3g} |" for k, v in derived]
    if kernel == COUNTER_CLOCK_KERNEL:
        lines += ["", f"Kernel code hash: `{kernel_hash()}`"]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter_means(folder, counter, reduce=None):
    """Mean value of `counter` per dispatch of each kernel (rocprofv3 csv), or
    another reduction over the dispatches (``reduce``, e.g. max)."""
    import csv
    files = _csvs(folder, "counter_collection.csv")
    if not files:
        sys.exit(f"no *counter_collection.csv under {folder}")
    per = {}
    for r in csv.DictReader(open(files[0])):
        if r["Counter_Name"] != counter:
            continue
        key = (r["Kernel_Name"], r.get("Dispatch_Id") or r.get("Correlation_Id"))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    means = {}
    for (name, _), v in per.items():
        means.setdefault(name, []).append(v)
    return {k: (reduce(v) if reduce else sum(v) / len(v)) for k, v in means.items()}


def summarize_traffic(fetch_dir, write_dir, cmd_fetch, cmd_write, kernel=ATTN_KERNEL, out=TRAFFIC_FILE,
                      label="attn_fwd_kernel<LatentCfg, LATENT>",
                      workload="DeepSeek-V3-shaped absorbed MLA prefill, causal, B=1 H=128 N=8192"):
    """HBM bytes per launch of a kernel: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch, averaged over its dispatches) scaled by what they read for a
    plain 1 GiB device copy in the same run; written with the hash of the
    kernel source it was taken on, so that a later kernel change makes
    bench.py report null."""
    def pick(means, key):
        hits = [v for k, v in means.items() if key in k]
        if not hits:
            sys.exit(f"kernel {key!r} not found; kernels: {list(means)}")
        return hits[0]
    fm, wm = _counter_means(fetch_dir, "FETCH_SIZE"), _counter_means(write_dir, "WRITE_SIZE")
    f_attn, w_attn = pick(fm, kernel), pick(wm, kernel)
    # the calibration copy is the largest copy dispatch (small blits of the
    # inputs' upload may share the kernel)
    f_copy = pick(_counter_means(fetch_dir, "FETCH_SIZE", max), COPY_KERNEL)
    w_copy = pick(_counter_means(write_dir, "WRITE_SIZE", max), COPY_KERNEL)
    f_scale = COPY_BYTES / (f_copy * 1024.0)   # the copy reads COPY_BYTES
    w_scale = COPY_BYTES / (w_copy * 1024.0)   # and writes COPY_BYTES
    fetch_b = f_attn * 1024.0 * f_scale
    write_b = w_attn * 1024.0 * w_scale
    res = {"kernel": label,
           "workload": workload,
           "kernel_sha256_16": kernel_hash(),
           "fetch_kib_raw": round(f_attn, 1), "write_kib_raw": round(w_attn, 1),
           "copy_1GiB_fetch_kib_raw": round(f_copy, 1), "copy_1GiB_write_kib_raw": round(w_copy, 1),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "fetch_bytes": int(fetch_b), "write_bytes": int(write_b),
           "bytes_per_launch": int(fetch_b + write_b),
           "cmd_fetch": cmd_fetch, "cmd_write": cmd_write}
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res, indent=1))


def copy_calibration():
    """One plain device copy of 1 GiB: the HBM counters' calibration."""
    import torch
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-rows", action="store_true", help="headline only")
    ap.add_argument("--only-row", choices=["ring", "merge", "split", "sparse", "decode", "vup", "fp8"],
                    help="time this one row alone (no headline, no CPU baseline): for profiling a kernel")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run one plain device copy of 1 GiB (HBM counter calibration)")
    ap.add_argument("--summarize-stats", metavar="DIR",
                    help="write a markdown summary of a rocprofv3 --stats csv run to --out, then exit")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the HBM traffic summary from FETCH_SIZE / WRITE_SIZE csv runs, then exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="write a summary of rocprofv3 --pmc csv runs (one folder per pass) to --out, then exit")
    ap.add_argument("--kernel", default="attn_fwd", help="kernel name substring for --summarize-counters")
    ap.add_argument("--traffic-row", choices=sorted(ROW_TRAFFIC),
                    help="--summarize-traffic for this row's kernel (written to the row's summary file)")
    ap.add_argument("--out", help="output file of --summarize-stats / --summarize-counters")
    ap.add_argument("--cmd", nargs="*", default=[],
                    help="the profiling command(s) the summary came from, recorded in it")
    args = ap.parse_args()
    if args.summarize_stats:
        summarize_stats(args.summarize_stats, args.out, " ".join(args.cmd))
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.kernel, args.out, args.cmd)
        return
    if args.summarize_traffic:
        cf, cw = (args.cmd + ["", ""])[:2]
        if args.traffic_row:
            kern, path = ROW_TRAFFIC[args.traffic_row]
            wl = {"sparse": "sparse top-k latent MLA, S=4096 S_kv=16384 H=128 K=2048 (drawn, unsorted lists)",
                  "decode": "MLA decode, B=64 sequences x 8192 cache rows, H=128 (4 key ranges of 2048)"}
            summarize_traffic(*args.summarize_traffic, cf, cw, kernel=kern, out=path,
                              label="attn_fwd_kernel<LatentCfg, SPARSE_PIPE>", workload=wl[args.traffic_row])
        else:
            summarize_traffic(*args.summarize_traffic, cf, cw)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this build has no "
              f"multi-GPU path; the ring across GPUs is design-only.", file=sys.stderr)
        sys.exit(2)

    import torch
    import ring_chunk_attention_amd as mla
    import workloads as W

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    if args.only_row:
        rows = measure_rows(mla, W, to_dev, args.steps, args.warmup, only=args.only_row)
        if args.copy_calib:
            copy_calibration()
        print(json.dumps({"row": args.only_row, **rows}), flush=True)
        return

    print("bench: generating the DeepSeek-V3 prefill inputs", file=sys.stderr, flush=True)
    case = W.dsv3_prefill(0)
    B, H, N, dk = case.q.shape
    q, kv = to_dev(case.q), to_dev(case.kv)
    out = torch.empty((B, H, N, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")

    def step():
        mla.fwd(q, kv, scale=case.scale, head_dim_v=512, causal=True, out=out, lse=lse)

    print("bench: timing", file=sys.stderr, flush=True)
    with ClockSampler() as clk:
        region_ms, launch_ms, launch_min_ms, launch_med_ms = time_launches(step, args.steps, args.warmup)
    flops = B * H * causal_pairs(N, N) * (2 * dk + 2 * 512)
    value = flops / (region_ms * 1e-3) / 1e12
    achieved = flops / (launch_ms * 1e-3) / 1e12
    traffic = measured_traffic()
    clock = clk.summary()

    if args.copy_calib:
        copy_calibration()

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(region_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": "DeepSeek-V3-shaped absorbed MLA prefill, causal",
                   "batch": B, "q_heads": H, "kv_heads": 1, "seq_len": N, "dk": dk, "dv": 512,
                   "scale": "1/sqrt(192)", "inputs": "bf16 N(0,1), seed 0",
                   "flop_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": "attn_fwd_kernel<LatentCfg, LATENT>",
                     "launch_ms_mean": round(launch_ms, 4), "launch_ms_min": round(launch_min_ms, 4),
                     "launch_ms_median": round(launch_med_ms, 4)},
        "engine_clock": clock,
    }
    # The same achieved rate against the peak at the shader clock the kernel
    # ran at.  The driver's DPM level (pp_dpm_sclk, sampled above) reads well
    # below that clock under this load, so the fraction takes the clock the
    # kernel's own cycle counter gives over a dispatch in its committed
    # counter summary, and falls back to the DPM median without one.
    shader = counter_clock()
    if clock or shader:
        mhz = shader if shader else clock["median_mhz"]
        peak_at = PEAK_BF16_TFLOPS * mhz / 2400.0
        result["roofline"]["frac_at_measured_clock"] = round(achieved / peak_at, 4)
        result["roofline"]["peak_at_measured_clock"] = round(peak_at, 1)
        result["roofline"]["clock_mhz"] = round(mhz, 1)
        result["roofline"]["clock_source"] = (
            "GRBM_GUI_ACTIVE per XCD over a dispatch of this kernel code (profiles/"
            + os.path.basename(COUNTERS_FILE) + ")" if shader else "pp_dpm_sclk median during the timed region")
    if clock:
        clock["note"] = "driver DPM level; reads below the shader clock under MFMA load"
    del q, kv, out, lse
    torch.cuda.empty_cache()

    if not args.no_rows:
        result["rows"] = measure_rows(mla, W, to_dev, args.steps, args.warmup)
    if not args.no_cpu:
        print("bench: CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(result), flush=True)


def measure_rows(mla, W, to_dev, steps, warmup, per_launch=False, only=None):
    """Time the other steps of the path at their workload shapes."""
    import torch
    rows = {}
    steps = max(3, min(steps, 10))

    if only in (None, "ring"):
        # one-device ring: 16 heads, N = 4096 as 4 chunks of 1024, folds in place
        print("bench: ring workload", file=sys.stderr, flush=True)
        c = W.ring4(0)
        q, kv = to_dev(c.q), to_dev(c.kv)
        o = torch.empty((1, 16, 4096, 512), dtype=torch.bfloat16, device="cuda")
        l = torch.empty((1, 16, 4096), dtype=torch.float32, device="cuda")
        # 10 calls (4 diagonal, 6 full) in one launch, 6 of them folding into a
        # float32 running result; each chunk's calls fold in ring order (the
        # default: the diagonal first) or in the balanced steps' order (full
        # calls first, the diagonal last)
        # (each timed behind a hold, so that the ring driver's host-side
        # validation of its 10 calls is not timed as GPU idle time)
        # The two schedules and the same workload unchunked (for the cost of
        # chunking) are timed in turn, five rounds with the order rotated (each
        # variant takes each place in a round), after all three have run
        # untimed; each is reported as its median.  Short runs on a GPU whose
        # clock moves with load and heat vary by several percent from one run
        # to the next, and the first runs after the long headline read slow.
        carry = torch.empty(mla.ring_workspace_size(1, 16, 4096, 4), dtype=torch.uint8, device="cuda")
        variants = {
            "balanced": lambda: mla.ring_fwd(q, kv, 4, scale=c.scale, out=o, lse=l, carry=carry, order="balanced"),
            "ring": lambda: mla.ring_fwd(q, kv, 4, scale=c.scale, out=o, lse=l, carry=carry, order="ring"),
            "unchunked": lambda: mla.fwd(q, kv, scale=c.scale, out=o, lse=l)}
        times = {k: [] for k in variants}
        order = ("ring", "balanced", "unchunked")
        for k in order:
            for _ in range(steps):
                variants[k]()
        for rnd in range(5):
            for k in order[rnd % 3:] + order[:rnd % 3]:
                times[k].append(time_launches(variants[k], steps, warmup, hold=True, per_launch=False)[0])
        ms, ms_bal, ms1 = (float(np.median(times[k])) for k in ("ring", "balanced", "unchunked"))
        fl = 16 * causal_pairs(4096, 4096) * 2176
        rows["ring_4x1024_h16"] = {"ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 2),
                                   "pct_of_peak": round(100 * fl / ms / 1e9 / PEAK_BF16_TFLOPS, 2),
                                   "calls": 10, "launches": 1, "folds": 6, "schedule": "ring order",
                                   "balanced_ms": round(ms_bal, 4), "unchunked_ms": round(ms1, 4),
                                   "vs_unchunked": round(ms / ms1, 3), "balanced_vs_unchunked": round(ms_bal / ms1, 3),
                                   "timing": "median of 5 interleaved rounds of %d steps each" % steps}
        del q, kv, o, l
    if only in (None, "merge"):
        # standalone merge of two [1, 16, 1024, 512] partials (HBM-bound): two
        # chunks of the ring workload's result
        c = W.ring4(0)
        q, kv = to_dev(c.q), to_dev(c.kv)
        o, l = mla.fwd(q, kv, scale=c.scale)
        a, b = o[:, :, :1024].contiguous(), o[:, :, 1024:2048].contiguous()
        la, lb = l[:, :, :1024].contiguous(), l[:, :, 1024:2048].contiguous()
        mo, ml = torch.empty_like(a), torch.empty_like(la)
        ms = time_launches(lambda: mla.merge(a, la, b, lb, out=mo, lse=ml), steps, warmup, hold=True,
                                 per_launch=False)[0]
        nbytes = 3 * a.numel() * 2 + 3 * la.numel() * 4
        rows["merge_h16_1024x512"] = {"ms": round(ms, 4), "GBps": round(nbytes / ms / 1e6, 1),
                                      "hbm_frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4)}
        del q, kv, o, l, a, b, la, lb, mo, ml

    if only in (None, "split"):
        # split q/k varlen ring step: 8 sequences, 32 heads, prev fold
        print("bench: split varlen workload", file=sys.stderr, flush=True)
        c = W.split_ring_step(0)
        args = [to_dev(x) for x in (c.q1, c.q2, c.k1, c.k2, c.v)]
        sl = torch.from_numpy(c.seq_lens).cuda()
        prev = (to_dev(c.prev_out), torch.from_numpy(c.prev_lse).cuda())
        T = int(c.seq_lens.sum())
        so = torch.empty((T, 32, 128), dtype=torch.bfloat16, device="cuda")
        sL = torch.empty((32, T), dtype=torch.float32, device="cuda")
        ms = time_launches(lambda: mla.split_fwd(*args, scale=c.scale, seq_lens=sl, prev=prev,
                                                       out=so, lse=sL), steps, warmup, per_launch=False)[0]
        fl = 32 * sum(causal_pairs(int(L), int(L)) for L in c.seq_lens) * (2 * 192 + 2 * 128)
        rows["split_varlen_8seq_h32"] = {"ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 2),
                                         "pct_of_peak": round(100 * fl / ms / 1e9 / PEAK_BF16_TFLOPS, 2),
                                         "tokens": T}
        del args, sl, prev, so, sL

    if only in (None, "sparse"):
        # sparse top-k: 4096 queries x 128 heads x 2048 gathered rows
        print("bench: sparse workload", file=sys.stderr, flush=True)
        c = W.sparse_topk(0)
        t = [to_dev(x) for x in (c.q_lift, c.q_pe, c.c_kv, c.k_pe)]
        idx = torch.from_numpy(c.idx).cuda()
        so = torch.empty((1, 4096, 128 * 512), dtype=torch.bfloat16, device="cuda")
        sL = torch.empty((1, 4096, 128), dtype=torch.float32, device="cuda")
        ms = time_launches(lambda: mla.sparse_fwd(*t, idx, scale=c.scale, out=so, lse=sL), steps, warmup, per_launch=False)[0]
        fl = 4096 * 128 * 2048 * 2176
        gathered = 4096 * 2048 * 1152
        rows["sparse_topk_s4096_k2048_h128"] = {
            "ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 2),
            "pct_of_peak": round(100 * fl / ms / 1e9 / PEAK_BF16_TFLOPS, 2),
            "gather_GBps": round(gathered / ms / 1e6, 1),
            "compulsory_bytes": sum(x.numel() * x.element_size() for x in (*t, idx, so, sL)),
            "gathered_bytes": gathered}
        tr = measured_traffic(ROW_TRAFFIC["sparse"][1], full=True)
        if tr:
            rows["sparse_topk_s4096_k2048_h128"].update(
                hbm_bytes_measured=tr["bytes_per_launch"], hbm_fetch_bytes=tr["fetch_bytes"],
                hbm_GBps_measured=round(tr["bytes_per_launch"] / ms / 1e6, 1))
        del t, idx, so, sL

    if only in (None, "decode"):
        # token generation: 64 sequences x 128 heads, 8192 cache rows each, the
        # keys split across workgroups (4 ranges of 2048) and reduced through LSE
        print("bench: decode workload", file=sys.stderr, flush=True)
        c = W.dsv3_decode(0)
        q, kv, lens = to_dev(c.q), to_dev(c.kv), torch.from_numpy(c.kv_lens).cuda()
        B, H = c.q.shape[:2]
        do = torch.empty((B, H, 512), dtype=torch.bfloat16, device="cuda")
        dl = torch.empty((B, H), dtype=torch.float32, device="cuda")
        ms = time_launches(lambda: mla.decode_fwd(q, kv, scale=c.scale, kv_lens=lens, out=do, lse=dl),
                                 steps, warmup, per_launch=False)[0]
        keys = int(c.kv_lens.astype(np.int64).sum())
        fl = H * keys * 2176
        # algorithmic HBM bytes: each cache row once, the queries, outputs and LSEs
        nbytes = keys * 576 * 2 + B * H * 576 * 2 + B * H * 512 * 2 + B * H * 4
        rows["decode_b64_kv8192_h128"] = {
            "ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 2),
            "pct_of_peak": round(100 * fl / ms / 1e9 / PEAK_BF16_TFLOPS, 2),
            "GBps": round(nbytes / ms / 1e6, 1), "hbm_frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4),
            "bytes": nbytes}
        tr = measured_traffic(ROW_TRAFFIC["decode"][1], full=True)
        if tr:
            rows["decode_b64_kv8192_h128"].update(
                hbm_bytes_measured_attention_kernel=tr["bytes_per_launch"], hbm_fetch_bytes=tr["fetch_bytes"])
        del q, kv, lens, do, dl

    if only in (None, "vup"):
        # V-up projection of a prefill's latent output: [1, 128, 8192, 512] x
        # per-head [128, 512] weights -> [8192, 128 * 128]; HBM-bound
        print("bench: V-up workload", file=sys.stderr, flush=True)
        c = W.dsv3_vup(0)
        o, w = to_dev(c.o), to_dev(c.w_uv)
        B, H, T, L = c.o.shape
        vo = torch.empty((B, T, H, 128), dtype=torch.bfloat16, device="cuda")
        ms = time_launches(lambda: mla.vup(o, w, out=vo), steps, warmup, per_launch=False)[0]
        fl = B * H * T * L * 128 * 2
        nbytes = o.numel() * 2 + w.numel() * 2 + vo.numel() * 2   # each operand once
        rows["vup_h128_t8192"] = {
            "ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 2),
            "GBps": round(nbytes / ms / 1e6, 1), "hbm_frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4),
            "bytes": nbytes}
        del o, w, vo

    if only in (None, "fp8"):
        # the headline workload with FP8 e4m3 Q and KV (unit scales), both
        # products on 8-bit MFMA, bf16 output and fp32 LSE
        print("bench: FP8 prefill workload", file=sys.stderr, flush=True)
        c = W.dsv3_prefill_fp8(0)
        q8 = torch.from_numpy(c.q8).cuda().view(torch.float8_e4m3fn)
        kv8 = torch.from_numpy(c.kv8).cuda().view(torch.float8_e4m3fn)
        B, H, N, _ = c.q8.shape
        fo = torch.empty((B, H, N, 512), dtype=torch.bfloat16, device="cuda")
        fl_ = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        ms = time_launches(lambda: mla.fwd_fp8(q8, kv8, scale=c.scale, out=fo, lse=fl_), steps, warmup,
                                 per_launch=False)[0]
        fl = B * H * causal_pairs(N, N) * 2176
        rows["prefill_fp8_dsv3_h128_n8192"] = {
            "ms": round(ms, 4), "tflops": round(fl / ms / 1e9, 2),
            "pct_of_fp8_peak": round(100 * fl / ms / 1e9 / PEAK_FP8_TFLOPS, 2),
            "peak_tflops": PEAK_FP8_TFLOPS, "dtype": "e4m3 inputs and P, fp32 accumulation, bf16 out"}
        del q8, kv8, fo, fl_
    return rows


if __name__ == "__main__":
    main()
