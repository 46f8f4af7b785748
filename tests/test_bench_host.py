"""Host logic of bench.py: the counter ingest (rocprofv3 counter-collection
CSV + the counter pass's dispatch manifest -> per-problem HBM bytes) and the
launch-weighted traffic the roofline reports.  Synthetic CSVs, no GPU."""
import csv
import json
import subprocess
import sys
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(...)>"


class Cfg:
    def __init__(self, **kw):
        self.kw = kw

    def as_dict(self):
        return dict(self.kw)


class P:
    def __init__(self, fmt, M, N, K, packed, cfg, R):
        self.fmt, self.M, self.N, self.K, self.packed, self.cfg, self.R = fmt, M, N, K, packed, cfg, R
        self.layout_name = {0: "row", 1: "packed", 2: "seg2", 4: "seg4", 8: "seg8"}[int(packed)]


def write_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            r = {k: 0 for k in FIELDS}
            r.update(Correlation_Id=i + 1, Dispatch_Id=i + 1, Kernel_Name=name,
                     Counter_Name=counter, Counter_Value=value)
            w.writerow(r)


def make_run(tmp_path, fetch_rows, write_rows, order):
    cfg_a = dict(tile_n=16, waves_k=2, unroll=4, split_k=4, swap_ab=1)
    cfg_b = dict(tile_n=32, waves_k=1, unroll=1, split_k=1, swap_ab=0)
    man = {"problems": [{"fmt": "FP8_Dynamic", "M": 1, "N": 512, "K": 7168, "layout": "packed",
                         "cfg": cfg_a, "kernel": "gemm_kernel<0, 1, 1, 2, 4, 1, 1>"},
                        {"fmt": "W8A8_INT8", "M": 8, "N": 896, "K": 5120, "layout": "row",
                         "cfg": cfg_b, "kernel": "gemm_kernel<0, 1, 1, 2, 4, 1, 1>"}],
           "gemm_dispatch_order": order, "copy_bytes_read": 1 << 20,
           "copy_bytes_written": 1 << 20, "copies": 3, "source_hash": bench.kernel_source_hash()}
    mp = tmp_path / "manifest.json"
    mp.write_text(json.dumps(man))
    fc, wc = tmp_path / "fetch.csv", tmp_path / "write.csv"
    write_csv(fc, "FETCH_SIZE", fetch_rows)
    write_csv(wc, "WRITE_SIZE", write_rows)
    return mp, fc, wc, cfg_a, cfg_b


def test_ingest_and_weighted_traffic(tmp_path, monkeypatch):
    g0 = "void w8::gemm_kernel<0, 1, 1, 2, 4, 1, 1>(w8::GemmArgs)"
    g1 = g0   # two problems served by one kernel instance
    # the copy reads 1 MiB but FETCH_SIZE reports half of it: fetch scale 2
    fetch = [("__amd_rocclr_copyBuffer", 5.0), (g0, 100.0), (g0, 110.0), (g1, 400.0), (g1, 400.0),
             (COPY, 512.0), (COPY, 512.0), (COPY, 512.0)]
    write = [("__amd_rocclr_copyBuffer", 1.0), (g0, 10.0), (g0, 10.0), (g1, 4.0), (g1, 6.0),
             (COPY, 1024.0), (COPY, 1024.0), (COPY, 1024.0)]
    mp, fc, wc, cfg_a, cfg_b = make_run(tmp_path, fetch, write, [0, 0, 1, 1])
    out = tmp_path / "counters.json"
    bench.ingest_counters(str(mp), str(fc), str(wc), str(out), "cmd")
    d = json.loads(out.read_text())
    assert d["fetch_scale"] == pytest.approx(2.0) and d["write_scale"] == pytest.approx(1.0)
    assert [r["fetch_kib"] for r in d["problems"]] == [105.0, 400.0]
    assert [r["write_kib"] for r in d["problems"]] == [10.0, 5.0]
    monkeypatch.setattr(bench, "PMC_FILE", str(out))
    pa = P("FP8_Dynamic", 1, 512, 7168, True, Cfg(**cfg_a), R=3)
    pb = P("W8A8_INT8", 8, 896, 5120, False, Cfg(**cfg_b), R=1)
    ta = (105.0 * 2 + 10.0) * 1024
    tb = (400.0 * 2 + 5.0) * 1024
    assert bench.measured_traffic("gemm_kernel<0, 1, 1, 2, 4, 1, 1>", [pa]) == round(ta)
    # each problem is weighted by its launches, like the achieved rate
    assert bench.measured_traffic("gemm_kernel<0, 1, 1, 2, 4, 1, 1>", [pa, pb]) == \
        round((3 * ta + tb) / 4)
    # another kernel name, config or layout: no measured traffic
    assert bench.measured_traffic("gemm_kernel<1, 1, 2, 1, 1, 0, 0>", [pb]) is None
    pc = P("FP8_Dynamic", 1, 512, 7168, False, Cfg(**cfg_a), R=3)
    assert bench.measured_traffic("gemm_kernel<0, 1, 1, 2, 4, 1, 1>", [pc]) is None
    pd = P("FP8_Dynamic", 1, 512, 7168, True, Cfg(**dict(cfg_a, split_k=8)), R=3)
    assert bench.measured_traffic("gemm_kernel<0, 1, 1, 2, 4, 1, 1>", [pd]) is None
    # counters taken from other kernel sources are stale
    d["source_hash"] = "0" * 16
    out.write_text(json.dumps(d))
    assert bench.measured_traffic("gemm_kernel<0, 1, 1, 2, 4, 1, 1>", [pa]) is None


def test_ingest_rejects_dispatch_mismatch(tmp_path):
    g0 = "void w8::gemm_kernel<0, 1, 1, 2, 4, 1, 1>(w8::GemmArgs)"
    fetch = [(g0, 1.0), (COPY, 1.0), (COPY, 1.0), (COPY, 1.0)]
    mp, fc, wc, _, _ = make_run(tmp_path, fetch, fetch, [0, 0, 1, 1])
    with pytest.raises(SystemExit):
        bench.ingest_counters(str(mp), str(fc), str(wc), str(tmp_path / "o.json"), "cmd")


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
