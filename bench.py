"""Segmented top-k benchmark on one MI355X.

One step = one batched_topk call over one batch of synthetic input (all of the
hot path: pass-0 streaming, radix passes, tie selection, sort, output).  The
headline workload is 4096 segments x 4096 float32 keys ~ N(0,1) with uint32
index values, k = 64, MaxPairs, gpu_to_gpu + prefer_smaller_index,
stable_sorted.  Its inputs (128 MiB) would fit the 256 MiB Infinity Cache, so
steps rotate over enough copies of the input that each step reads its keys
from HBM.  The other workloads are measured the same way and reported under
"workloads".

Prints one JSON line.  Usage:  python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
HEADLINE = "normal_f32_4096x4096_k64"
KEY_BYTES = {"f32": 4, "bf16": 2, "f16": 2, "u32": 4, "i32": 4}
CACHE_BYTES = 256 << 20  # Infinity Cache


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model():
    """CPU model name from /proc/cpuinfo (plus family/model numbers when the
    name is generic), read on the machine the benchmark runs on."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" in line:
                    k, v = line.split(":", 1)
                    info.setdefault(k.strip(), v.strip())
    except OSError:
        pass
    name = info.get("model name") or platform.processor() or "unknown"
    if "cpu family" in info and "model" in info:
        name += f" (family {info['cpu family']}, model {info['model']})"
    return name


def host_cpus():
    """CPUs this process may run on (its affinity mask)."""
    try:
        return len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        return os.cpu_count() or 1


def workload_sizes(off_np, k):
    import numpy as np
    n = np.maximum(off_np[1:] - off_np[:-1], 0)
    return int(n.sum()), int(np.minimum(n, k).sum())


def measure(name, steps, warmup, stream_rotate=True, min_timed_ms=0.0):
    """Times `steps` back-to-back calls (after `warmup`) with HIP events on the
    stream the library launches on.  Returns a dict of figures.  With
    `min_timed_ms`, calls far shorter than that get more steps (and warmup
    calls), so that the timed region is not a handful of calls on a cold host
    path."""
    import numpy as np
    import torch

    import segmented_top_selection_amd as st
    import workloads

    w = workloads.WORKLOADS[name]
    keys, vals, off = w["gen"](device="cuda", **w["args"])
    if not w["pairs"]:
        vals = None
    off_np = off.cpu().numpy()
    N, KK = workload_sizes(off_np, w["k"])
    sk = KEY_BYTES[w["key_type"]]
    sv = 4 if vals is not None else 0
    in_bytes = keys.numel() * sk + (vals.numel() * 4 if vals is not None else 0)
    # Copies so that every step reads inputs that are not cache-resident.
    copies = 1
    if stream_rotate and in_bytes < 4 * CACHE_BYTES:
        copies = max(2, int(np.ceil(4 * CACHE_BYTES / in_bytes)))
    ins = [(keys, vals)] + [(keys.clone(), vals.clone() if vals is not None else None)
                            for _ in range(copies - 1)]
    s = off.numel() - 1
    out_k = torch.empty((s, w["k"]), dtype=keys.dtype, device="cuda")
    out_v = torch.empty((s, w["k"]), dtype=torch.int32, device="cuda") if vals is not None else None

    def step(i):
        kk, vv = ins[i % copies]
        st.batched_topk(kk, off, w["k"], values=vv, largest=w["largest"],
                        determinism=w["determinism"], tie_break=w["tie_break"],
                        ordering=w["ordering"], key_type=w["key_type"], out_keys=out_k,
                        out_values=out_v, max_segment_size=w.get("max_segment_size"))

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    if min_timed_ms > 0:
        t0 = time.perf_counter()
        for i in range(3):
            step(warmup + i)
        torch.cuda.synchronize()
        est_ms = (time.perf_counter() - t0) / 3 * 1e3
        if steps * est_ms < min_timed_ms:
            steps = min(2000, int(np.ceil(min_timed_ms / est_ms)))
            for i in range(20):
                step(warmup + 3 + i)
            warmup += 23
            torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    # Whole-job rate: `steps` back-to-back calls between two events.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(warmup + i)
    e1.record(stream)
    enqueue_s = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = e0.elapsed_time(e1)
    ms = total_ms / steps
    t = ms / 1e3
    # Launch duration: events right before and after each call, same stream.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record(stream)
        step(warmup + steps + i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in evs]  # ms
    bytes_roof = N * (sk + sv) + KK * (sk + sv)          # metric's single-read roofline
    bytes_alg = N * sk + KK * sv + KK * (sk + sv)         # what the method must move
    res = dict(
        workload=name, segments=s, keys=N, k=w["k"], key_type=w["key_type"], steps=steps,
        warmup=warmup,
        mode=f"{'Max' if w['largest'] else 'Min'}{'Pairs' if vals is not None else 'Keys'} "
             f"{w['determinism']}/{w['tie_break']}/{w['ordering']}",
        ms_per_step=ms, launch_ms_mean=float(np.mean(per)), launch_ms_min=min(per),
        launch_ms_median=float(np.median(per)), host_enqueue_us_per_call=enqueue_s / steps * 1e6,
        wall_s=wall,
        keys_per_s=N / t, input_copies=copies,
        bytes_roof=bytes_roof, hbm_roof_frac=(bytes_roof / (HBM_PEAK_GBS * 1e9)) / t,
        bytes_alg=bytes_alg, alg_gbs=bytes_alg / t / 1e9,
    )
    del ins, keys, vals, out_k, out_v
    torch.cuda.empty_cache()
    return res


COPY_PROBE_REPS = 5


def copy_probe(mib=256, reps=COPY_PROBE_REPS):
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters (FETCH_SIZE / WRITE_SIZE) of a profiled run."""
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy probe: {reps} copies of {mib} MiB")


PROBE_LIB = os.path.join(ROOT, "segmented_top_selection_amd", "probe", "libsegtopk_probe.so")


def stream_read_probe(gib=2, reps=10):
    """GB/s of a plain streaming read (16-byte non-temporal loads, the load the
    top-k kernels stream their keys with) of a `gib` GiB buffer, far beyond
    the Infinity Cache: best over a few grid sizes of the median of `reps`
    timed launches.  The reference point for each workload's probe_frac."""
    import ctypes

    import numpy as np
    import torch
    lib = ctypes.CDLL(PROBE_LIB)
    lib.segtopk_probe_stream_read.restype = ctypes.c_int
    lib.segtopk_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32,
                                              ctypes.c_void_p, ctypes.c_void_p]
    nbytes = gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(3)
    stream = torch.cuda.current_stream()
    best = None
    for wgs in (768, 2048, 4096):
        sink = torch.empty(wgs * 256, dtype=torch.int32, device="cuda")
        times = []
        for r in range(reps + 2):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            rc = lib.segtopk_probe_stream_read(buf.data_ptr(), nbytes, wgs, sink.data_ptr(),
                                               stream.cuda_stream)
            b.record(stream)
            if rc != 0:
                raise RuntimeError(f"stream-read probe failed: {rc}")
            torch.cuda.synchronize()
            if r >= 2:
                times.append(a.elapsed_time(b))
        gbs = nbytes / (float(np.median(times)) / 1e3) / 1e9
        log(f"stream-read probe: {gib} GiB, {wgs} workgroups: {gbs:.0f} GB/s")
        if best is None or gbs > best["gbs"]:
            best = dict(gbs=gbs, workgroups=wgs, gib=gib, median_ms=float(np.median(times)))
        del sink
    del buf
    torch.cuda.empty_cache()
    return best


KERNEL_SRC_DIR = os.path.join(ROOT, "segmented_top_selection_amd", "csrc")


def kernel_hash():
    """SHA-256 over every library source (names and contents, sorted)."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(KERNEL_SRC_DIR)):
        with open(os.path.join(KERNEL_SRC_DIR, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(name):
    """HBM bytes per launch from the last rocprofv3 FETCH_SIZE / WRITE_SIZE
    runs (profiles/traffic_<workload>.json), or None when the kernel source
    has changed since they were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_hash():
        return None
    return t.get("traffic_bytes_per_launch")


def traffic_from(fetch_csv, write_csv, name):
    """Turns two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, then
    WRITE_SIZE; KiB per dispatch) of `--copy-probe` runs into HBM bytes per
    topk_kernel launch, each counter scaled by what it reads for the 256 MiB
    plain copy, and writes profiles/traffic_<workload>.json."""
    import csv

    def per_kernel(path, counter):
        topk, copies = [], []
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                v = float(row["Counter_Value"])
                if "topk_kernel" in row["Kernel_Name"]:
                    topk.append(v)
                elif "copyBuffer" in row["Kernel_Name"]:
                    copies.append((int(row["Dispatch_Id"]), v))
        if not topk or not copies:
            raise SystemExit(f"{path}: no topk_kernel or copy dispatches with {counter}")
        # The probe's copies are the run's first ones (input generation may
        # copy other buffers later).
        probe = [v for _, v in sorted(copies)[:COPY_PROBE_REPS]]
        return sum(topk) / len(topk), max(probe), len(topk)

    copy_bytes = 256 << 20
    f_kib, f_copy, n_f = per_kernel(fetch_csv, "FETCH_SIZE")
    w_kib, w_copy, n_w = per_kernel(write_csv, "WRITE_SIZE")
    f_scale = copy_bytes / (f_copy * 1024)
    w_scale = copy_bytes / (w_copy * 1024)
    run = ("cd /tmp && rocprofv3 --pmc {c} --output-format csv -d <out dir>/{w}/{c} -o p -- "
           "python3 /root/repo/bench.py --workload {w} --only-headline --no-cpu-baseline --no-probe "
           "--copy-probe --steps 5 --warmup 2")
    out = {
        "workload": name,
        "commands": [run.format(c=c, w=name) for c in ("FETCH_SIZE", "WRITE_SIZE")] + [
            f"python3 bench.py --workload {name} --traffic-from <FETCH_SIZE csv> <WRITE_SIZE csv>"],
        "kernel_source_sha256": kernel_hash(),
        "dispatches": [n_f, n_w],
        "fetch_kib_per_launch": f_kib, "write_kib_per_launch": w_kib,
        "copy_probe_fetch_kib": f_copy, "copy_probe_write_kib": w_copy,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "traffic_bytes_per_launch": f_kib * 1024 * f_scale + w_kib * 1024 * w_scale,
    }
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def cpu_baseline(name, budget_s=2.0, max_sample_keys=1 << 23):
    """The oracle, as it stands, on a bounded sample of the workload (whole
    segments taken from the start; a single segment longer than
    `max_sample_keys` is cut to its first `max_sample_keys` keys, taken as one
    segment), on the host cores.  The sample grows until one run takes about a
    quarter of `budget_s`, then runs are repeated for about `budget_s`."""
    import numpy as np
    import torch

    import oracle
    import workloads

    w = workloads.WORKLOADS[name]
    args = dict(w["args"])
    keys, vals, off = w["gen"](device="cuda", **args)
    s = off.numel() - 1
    threads = oracle.default_threads()
    off_h = off.cpu().numpy()
    rows = min(s, 64)
    while True:
        b, e = int(off_h[0]), int(off_h[rows])
        cut = False
        if rows == 1 and e - b > max_sample_keys:
            e, cut = b + max_sample_keys, True
        kb = keys[b:e].cpu()
        kb = kb.view(torch.int16).numpy().view(np.uint16) if kb.element_size() == 2 else \
            kb.view(torch.int32).numpy().view(np.uint32)
        kb = kb.view(np.float32) if w["key_type"] == "f32" else kb
        vb = vals[b:e].cpu().numpy().view(np.uint32) if w["pairs"] else None
        o = np.array([0, e - b], np.int64) if cut else off_h[:rows + 1] - b

        def run():
            t0 = time.perf_counter()
            oracle.batched_topk(kb, o, w["k"], key_type=w["key_type"], values=vb,
                                largest=w["largest"],
                                prefer_larger=w["tie_break"] == "prefer_larger_index",
                                threads=threads)
            return time.perf_counter() - t0
        elapsed = run()
        if rows >= s or elapsed > budget_s / 4:
            break
        rows = min(s, rows * 4)
    times = [elapsed]
    while sum(times) < budget_s:
        times.append(run())
    t = float(np.median(times))
    n = int(o[-1])
    used = min(threads, rows)  # the oracle's threads work on whole segments
    what = (f"the first {n} keys of segment 0 of {name}, as one segment" if cut else
            f"{rows} of {s} segments ({n} keys) of {name}")
    del keys, vals, off
    torch.cuda.empty_cache()
    return dict(value=n / t, unit="keys/s", cores=used, kind="oracle",
                sample=f"{what}, median of {len(times)} runs, {t:.3f} s each",
                threads_requested=threads, host_cpus=host_cpus(), cpu=cpu_model())


def combined_pair(others):
    """The two 32 x 4 Mi calls (uint32 and float32 halves) as one 64 x 4 Mi
    workload: keys over the summed step times."""
    a, b = others.get("uniform_u32_32x4Mi_k2048"), others.get("normal10_f32_32x4Mi_k2048")
    if not a or not b:
        return None
    t = (a["ms_per_step"] + b["ms_per_step"]) / 1e3
    alg = a["bytes_alg"] + b["bytes_alg"]
    roof = a["bytes_roof"] + b["bytes_roof"]
    return dict(keys_per_s=(a["keys"] + b["keys"]) / t, ms_per_step=t * 1e3,
                alg_gbs=alg / t / 1e9, alg_frac=alg / t / 1e9 / HBM_PEAK_GBS,
                hbm_roof_frac=roof / (HBM_PEAK_GBS * 1e9) / t)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--only-headline", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the stream-read probe")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 256 MiB device copy (counter calibration)")
    ap.add_argument("--size-hint", type=int, default=None,
                    help="pass this max_segment_size with the --workload calls (for "
                         "instance its segment length, which selects the small-segment "
                         "kernel at 4096 keys or fewer); the default passes none")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json from two rocprofv3 --pmc "
                         "runs of this script with --copy-probe, then exit")
    a = ap.parse_args()
    if a.traffic_from:
        traffic_from(a.traffic_from[0], a.traffic_from[1], a.workload)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {a.gpus}); segments are "
              f"independent, so N GPUs would each run this call on their own shard.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    if a.copy_probe:
        copy_probe()
    probe = None if a.no_probe else stream_read_probe()
    if a.size_hint is not None:
        workloads.WORKLOADS[a.workload]["max_segment_size"] = a.size_hint
    head = measure(a.workload, a.steps, a.warmup)
    if probe:
        head["probe_frac"] = head["alg_gbs"] / probe["gbs"]
    log("headline", json.dumps(head))
    others = {}
    if not a.only_headline:
        for name in workloads.WORKLOADS:
            if name == a.workload:
                continue
            others[name] = measure(name, max(5, a.steps // 2), 2, min_timed_ms=5.0)
            if probe:
                others[name]["probe_frac"] = others[name]["alg_gbs"] / probe["gbs"]
            log(name, json.dumps(others[name]))
    cpu = None if a.no_cpu_baseline else cpu_baseline(a.workload)
    if not a.no_cpu_baseline and not a.only_headline:
        for name in others:
            others[name]["cpu_baseline"] = cpu_baseline(name)
            log(name, "cpu_baseline", json.dumps(others[name]["cpu_baseline"]))

    # The headline plan is one kernel launch per call, so the average over
    # the K back-to-back calls is that kernel's launch duration (an event pair
    # around each call also times the dispatch of the next packet: the
    # per-call figures launch_ms_* run 2-3 us above a kernel trace).
    kernel_ms = head["ms_per_step"]
    line = {
        "metric": "segmented top-k keys/sec + % of single-read HBM roofline (fp32, k=64)",
        "value": head["keys_per_s"],
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["key_type"],
        "data": "synthetic",
        "config": {"workload": a.workload, "size_hint": a.size_hint, "segments": head["segments"],
                   "segment_len": head["keys"] // max(1, head["segments"]), "k": head["k"],
                   "mode": head["mode"]},
        "hbm_single_read_roofline_frac": head["hbm_roof_frac"],
        "roofline": {"bound": "hbm", "achieved": head["bytes_alg"] / (kernel_ms / 1e3) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": head["bytes_alg"] / (kernel_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                     "launch_us": kernel_ms * 1e3,
                     "launch_us_event_pair": head["launch_ms_mean"] * 1e3,
                     "bytes_per_launch": head["bytes_alg"],
                     "traffic": measured_traffic(a.workload),
                     "probe_gbs": probe["gbs"] if probe else None,
                     "probe_frac": head.get("probe_frac")},
        "stream_read_probe": probe,
        "cpu_baseline": cpu,
        "workloads": {n: {kk: (round(v, 6) if isinstance(v, float) else v)
                          for kk, v in r.items()} for n, r in others.items()},
        "combined_32x4Mi_pair": combined_pair(others),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
