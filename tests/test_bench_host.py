"""Host logic of bench.py that needs no GPU: turning two rocprofv3 counter
files into HBM bytes per launch, with the counters scaled by the plain-copy
probe of the same run, and the refusal of more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import bench

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def write_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for d, name, v in rows:
            w.writerow(dict(Dispatch_Id=d, Kernel_Name=name, Counter_Name=counter,
                            Counter_Value=v))


def test_traffic_from_scales_by_the_probe_copies(tmp_path, monkeypatch):
    os.makedirs(tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    copy = "void copyBuffer(...)"
    topk = "void segtopk_impl::topk_kernel<0, true, 4, false>(Params)"
    # Five probe copies of 256 MiB come first; FETCH_SIZE reads half of the
    # copied KiB, WRITE_SIZE all of them.  A larger copy later in the run
    # (input generation) must not be taken for the probe.
    fetch = [(i, copy, 131072.0) for i in range(5)] + [(9, copy, 524288.0)]
    fetch += [(20 + i, topk, 1000.0 + 10 * i) for i in range(3)]
    write = [(i, copy, 262144.0) for i in range(5)] + [(9, copy, 1048576.0)]
    write += [(20 + i, topk, 100.0) for i in range(3)]
    fcsv, wcsv = tmp_path / "f.csv", tmp_path / "w.csv"
    write_csv(fcsv, "FETCH_SIZE", fetch)
    write_csv(wcsv, "WRITE_SIZE", write)
    bench.traffic_from(str(fcsv), str(wcsv), "some_workload")
    out = json.load(open(tmp_path / "profiles" / "traffic_some_workload.json"))
    assert abs(out["fetch_scale"] - 2.0) < 1e-12 and abs(out["write_scale"] - 1.0) < 1e-12
    assert out["dispatches"] == [3, 3]
    expect = 1010.0 * 1024 * 2.0 + 100.0 * 1024 * 1.0
    assert abs(out["traffic_bytes_per_launch"] - expect) < 1e-6
    assert out["kernel_source_sha256"] == bench.kernel_hash()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
