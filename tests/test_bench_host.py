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


def test_summarize_counters(tmp_path):
    """The counter summary averages each problem's dispatches (matched to the
    manifest's dispatch order) and derives TA busy % over the dispatch time at
    2.4 GHz and the L2 hit rate."""
    def full_manifest(order):
        mp, _, _, _, _ = make_run(tmp_path, [], [], order)
        man = json.loads(mp.read_text())
        for pr in man["problems"]:
            for k in ("waves_n", "x_lds", "grid"):
                pr["cfg"].setdefault(k, 1 if k == "waves_n" else 0)
        mp.write_text(json.dumps(man))
        return mp

    mp = full_manifest([0, 1, 0, 1])
    gemm = "void w8::gemm_kernel<0, 1, 1, 1, 1, 4, 0, 8, 0, 0>(w8::GemmArgs)"
    vals = [  # dispatch: (ns, TA_BUSY_avr, TCC_HIT_sum, TCC_MISS_sum, SQ_WAVES, SQ_INSTS_VMEM_RD)
        (4000, 2400, 60, 40, 256, 1000), (2000, 960, 30, 70, 448, 500),
        (4000, 4800, 20, 80, 256, 3000), (2000, 960, 50, 50, 448, 700)]
    path = tmp_path / "pmc.csv"
    names = ("TA_BUSY_avr", "TCC_HIT_sum", "TCC_MISS_sum", "SQ_WAVES", "SQ_INSTS_VMEM_RD")
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        # a copy kernel first: not a GEMM, ignored
        r = {k: 0 for k in FIELDS}
        r.update(Dispatch_Id=1, Kernel_Name=COPY, Counter_Name="TA_BUSY_avr", Counter_Value=5)
        w.writerow(r)
        for d, (ns, *cs) in enumerate(vals):
            for name, v in zip(names, cs):
                r = {k: 0 for k in FIELDS}
                r.update(Dispatch_Id=d + 2, Kernel_Name=gemm, Counter_Name=name, Counter_Value=v,
                         Start_Timestamp=1000, End_Timestamp=1000 + ns)
                w.writerow(r)
    out = tmp_path / "out.md"
    bench.summarize_counters(str(mp), str(path), str(out), "cmd")
    rows = [l.split("|")[1:-1] for l in out.read_text().splitlines()
            if l.startswith("| FP8") or l.startswith("| W8A8")]
    rows = [[c.strip() for c in r] for r in rows]
    # problem 0: dispatches 0 and 2; ns 4000, TA (2400 + 4800) / 2 = 3600 cycles of 9600
    assert rows[0][6] == "4.00" and rows[0][9] == "3,600" and rows[0][10] == "37.5"
    assert rows[0][11] == "40.0"  # hits 40 of 100 on average
    assert rows[0][8] == "2,000" and rows[0][7] == "256"
    # problem 1: TA 960 of 4800 cycles, hits 40 of 100
    assert rows[1][10] == "20.0" and rows[1][11] == "40.0" and rows[1][8] == "600"
    # a dispatch count that does not match the manifest is refused
    mp2 = full_manifest([0, 1, 0])
    with pytest.raises(SystemExit):
        bench.summarize_counters(str(mp2), str(path), str(out), "cmd")
