"""Benchmark: geomean us per GEMM and achieved HBM GB/s over the small-M 8-bit
GEMM sweep on one MI355X.

Workload: the 24 (M, N, K) shapes of synthetic.SWEEP (M <= 32) in each of the
three formats (FP8_Dynamic, W8A8_INT8, Block_FP8): 72 GEMM problems, each
with the config the library resolves from its per-shape table (the tuned
table shipped with the package; default config on a miss).

Per problem, three HIP graphs are captured once:
  gemm   R back-to-back GEMMs, each reading its own copy of the weights;
  path   R back-to-back (activation quantization + GEMM) pairs;
  linear R back-to-back linear layers through the single entry point
         w8_linear with its own table entry: the fused kernel (quantization
         inside the GEMM, one launch) or, where the tuner found it faster,
         the quantize kernel and the GEMM (quant_launch = 1).
The R weight copies span at least --rotate-mib MiB (default 1024), more than
the last-level cache, so every weight byte read in the timed region comes
from HBM.  One step replays the three graphs of every problem once; W warmup steps
are untimed, then K steps are timed, bracketed by device synchronization.

Per problem: us per GEMM = median over steps of (graph time / R).  The
headline value is the geometric mean over the 72 problems of the achieved
GB/s of the GEMM, algorithmic bytes (weights + activations + scales + bf16
output) / us per GEMM; geomean us per GEMM is reported beside it, and so is
the same pair for the whole path (quantize + GEMM, two calls) and the time
of the linear layer through w8_linear (with the count of problems whose
table entry is the fused kernel).

roofline: the dominant GEMM kernel instance -- the largest sum, over the
problems that use it, of one GEMM's time per problem (the headline weighs
every problem once; the graphs' launch counts only follow from rotating
1 GiB of weight copies, so they would favour the smallest shapes) --
achieved = its algorithmic bytes per launch / its average launch time from
the HIP events, against the 8 TB/s HBM peak.

cpu_baseline: the oracle (oracle/, plain C, fp64/int64) run on the host on a
bounded sample of the same problems (quantize + GEMM), in the same unit.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synthetic  # noqa: E402

HBM_PEAK_GBPS = 8000.0
PMC_FILE = os.path.join(ROOT, "profiles", "gemm_sweep72_hbm_counters.json")
KERNEL_SOURCES = ("w8_gemm.hpp", "w8_device.hpp", "w8_gemm_inst.hip", "w8_launch.hpp")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bit_quantized_gemm_token_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, problems):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    runs (FETCH_SIZE and WRITE_SIZE in KiB per dispatch, each scaled by what
    the same counter reads for a plain copy of known size), weighted over
    `problems` like the achieved rate.  None when the counter file is missing,
    was taken from other kernel sources, or lacks any of these problems with
    the same config and layout."""
    try:
        with open(PMC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != kernel_source_hash():
        return None
    rows = {(r["fmt"], r["M"], r["N"], r["K"], r["layout"], json.dumps(r["cfg"], sort_keys=True)): r
            for r in d.get("problems", [])}
    total = launches = 0.0
    for p in problems:
        r = rows.get((p.fmt, p.M, p.N, p.K, p.layout_name,
                      json.dumps(p.cfg.as_dict(), sort_keys=True)))
        if r is None or r.get("kernel") != kernel:
            return None
        total += (r["fetch_kib"] * d["fetch_scale"] + r["write_kib"] * d["write_scale"]) * 1024 * p.R
        launches += p.R
    return round(total / launches) if launches else None


def counter_pass(problems, w8, manifest_path, copy_mib, launches=2):
    """Launches for a rocprofv3 --pmc run: each problem's GEMM `launches` times,
    each on another weight copy, then a plain device copy of `copy_mib` MiB
    (float32 negation: it reads and writes exactly that many bytes) three
    times; every launch is followed by a device synchronization, so dispatches
    never queue up under the profiler.  The dispatch order is written to
    `manifest_path` for ingest_counters()."""
    order = []
    for i, p in enumerate(problems):
        for r in range(launches):
            w8.gemm_w8a8(p.fmt, p.xq, p.sx, p.weights[r % p.R], p.sw, cfg=p.cfg, y=p.y_gemm,
                         workspace=p.ws)
            torch.cuda.synchronize()
            order.append(i)
    n = (copy_mib << 20) // 4
    src = torch.zeros(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
    manifest = {"problems": [{"fmt": p.fmt, "M": p.M, "N": p.N, "K": p.K,
                              "layout": p.layout_name, "cfg": p.cfg.as_dict(),
                              "kernel": p.kernel} for p in problems],
                "gemm_dispatch_order": order, "copy_bytes_read": n * 4, "copy_bytes_written": n * 4,
                "copies": 3, "source_hash": kernel_source_hash()}
    with open(manifest_path, "w") as f:
        json.dump(manifest, f)
    log(f"[bench] counter pass: {len(order)} GEMM dispatches, 3 copies of {copy_mib} MiB; "
        f"manifest {manifest_path}")


def _read_counter_csv(path, counter):
    """Per-dispatch values of `counter` from a rocprofv3 counter-collection
    CSV, in dispatch order: [(kernel_name, value)]."""
    import csv
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") != counter:
                continue
            rows.append((int(r.get("Dispatch_Id") or r.get("Correlation_Id") or 0),
                         r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort(key=lambda t: t[0])
    return [(k, v) for _, k, v in rows]


def ingest_counters(manifest_path, fetch_csv, write_csv, out_path, command):
    """Turns the two counter runs into the per-problem HBM traffic file read
    by measured_traffic()."""
    with open(manifest_path) as f:
        man = json.load(f)
    res = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _read_counter_csv(path, counter)
        gemm = [v for k, v in rows if "gemm_kernel<" in k]
        copy = [v for k, v in rows if "neg" in k]
        if len(gemm) != len(man["gemm_dispatch_order"]) or len(copy) != man["copies"]:
            raise SystemExit(f"{path}: {len(gemm)} GEMM and {len(copy)} copy dispatches, expected "
                             f"{len(man['gemm_dispatch_order'])} and {man['copies']}")
        per = {}
        for i, v in zip(man["gemm_dispatch_order"], gemm):
            per.setdefault(i, []).append(v)
        nbytes = man["copy_bytes_read"] if counter == "FETCH_SIZE" else man["copy_bytes_written"]
        copy_kib = sorted(copy)[len(copy) // 2]
        res[counter] = (per, nbytes / (copy_kib * 1024), copy_kib)
    fetch, fscale, fcopy = res["FETCH_SIZE"]
    write, wscale, wcopy = res["WRITE_SIZE"]
    probs = []
    for i, p in enumerate(man["problems"]):
        row = dict(p)
        row["fetch_kib"] = round(sum(fetch[i]) / len(fetch[i]), 3)
        row["write_kib"] = round(sum(write[i]) / len(write[i]), 3)
        probs.append(row)
    out = {"source_hash": man["source_hash"], "fetch_scale": round(fscale, 5),
           "write_scale": round(wscale, 5), "copy_fetch_kib": fcopy, "copy_write_kib": wcopy,
           "copy_bytes": man["copy_bytes_read"], "command": command, "problems": probs}
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    log(f"[bench] wrote {out_path}: fetch scale {fscale:.4f}, write scale {wscale:.4f}, "
        f"{len(probs)} problems")


def _cfg_str(c):
    return (f"tn{c['tile_n']} wk{c['waves_k']} wn{c['waves_n']} u{c['unroll']} s{c['split_k']} "
            f"sw{c['swap_ab']} xl{c['x_lds']}" + (f" g{c['grid']}" if c.get("grid") else ""))


def summarize_trace(stats_csv, out_md, command, bench_json=None):
    """profiles/*.md from a rocprofv3 kernel_stats.csv: per kernel, calls,
    total, average, min and max duration and share of the kernel time; with
    the JSON line of an unprofiled bench run, its dominant kernel's trace
    figures beside the bench's own average launch time."""
    import csv
    rows = []
    with open(stats_csv, newline="") as f:
        for r in csv.DictReader(f):
            ns = lambda k: float(r.get(k) or 0)
            rows.append((r["Name"], int(r["Calls"]), ns("TotalDurationNs"), ns("AverageNs"),
                         ns("MinNs"), ns("MaxNs"), float(r.get("Percentage") or 0)))
    rows.sort(key=lambda t: -t[2])
    lines = ["# rocprofv3 kernel trace: " + os.path.basename(out_md)[:-3].replace("_", " "), "",
             "Command (run from /tmp on the MI355X box, repository at $R):", "", "```", command,
             "```", "",
             "Kernel durations in microseconds, start to end of each dispatch, over every call "
             "in the run.  Under the kernel trace the dispatches of a graph are serialized, so "
             "averages include no overlap of consecutive launches.", "",
             "| kernel | calls | total ms | avg us | min us | max us | % |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for name, calls, tot, avg, mn, mx, pct in rows[:40]:
        short = name if len(name) <= 90 else name[:87] + "..."
        lines.append(f"| `{short}` | {calls} | {tot / 1e6:.2f} | {avg / 1e3:.3f} | "
                     f"{mn / 1e3:.3f} | {mx / 1e3:.3f} | {pct:.2f} |")
    if bench_json:
        with open(bench_json) as f:
            line = json.loads(f.read().strip().splitlines()[-1])
        rf = line["roofline"]
        # rocprofv3 names it "void w8::gemm_kernel<...>(w8::GemmArgs)"
        hit = [r for r in rows if "::" + rf["kernel"] + "(" in r[0]]
        lines += ["", f"Dominant kernel of the bench line (`{rf['kernel']}`, "
                  f"{len(rf['problems'])} problems: {', '.join(rf['problems'])}): "]
        if hit:
            name, calls, tot, avg, mn, mx, pct = hit[0]
            lines[-1] += (f"rocprofv3 average {avg / 1e3:.3f} us over {calls} calls (min "
                          f"{mn / 1e3:.3f}, max {mx / 1e3:.3f}); the unprofiled bench reports "
                          f"avg_launch_us = {rf['avg_launch_us']} for it (graph replay, where "
                          f"consecutive launches overlap head and tail).")
        else:
            lines[-1] += "not in this trace."
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    log(f"[bench] wrote {out_md} ({len(rows)} kernels)")


PHASE_PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                           "bit_quantized_gemm_token_amd", "w8_phase_probe")


def phase_study(out_md, command, only=None):
    """profiles/*.md from the phase probe (built beside the library from
    csrc/w8_phase_probe.hip): per configuration, the per-launch time of a
    graph replay and where it goes, from s_memrealtime stamps the probe's
    build of the kernel records at its phase boundaries."""
    import subprocess
    if not os.path.exists(PHASE_PROBE):
        raise SystemExit(f"{PHASE_PROBE} is missing: build the package first")
    cmd = [PHASE_PROBE] + ([only] if only else [])
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        raise SystemExit(f"phase probe failed ({r.returncode}):\n{r.stderr}")
    rows = [json.loads(l) for l in r.stdout.splitlines() if l.startswith("{")]
    lines = ["# Where one GEMM launch's time goes (phase probe)", "",
             "Command (on the MI355X box, repository at $R):", "", "```", command, "```", "",
             "`w8_phase_probe` replays each configuration from a HIP graph as the benchmark does "
             "(R launches on R weight copies spanning >= 1 GiB) and times the graph with HIP "
             "events (`us/launch`).  Its build of the GEMM kernel records `s_memrealtime` "
             "(100 MHz, common to the whole device) at the phase boundaries of every workgroup "
             "(`W8_PHASE_STAMPS`, see `csrc/w8_gemm.hpp`); from one more replay, averaged over "
             "the launches:", "",
             "- `gap`: from the previous launch's last workgroup finishing to this launch's "
             "first workgroup starting (the launch cost under graph replay);",
             "- `in-kernel`: first workgroup start to last workgroup end; `start spread`: first "
             "to last workgroup start;",
             "- `loop w0` / `loop max`: K loop of wave 0 / of the workgroup's slowest wave, from "
             "the workgroup's start; `K-sum`: summing the K-waves through LDS after the slowest "
             "wave (workgroups whose waves split K);",
             "- shared tiles (split-K): `ack` the partial stores acknowledged, `count` the "
             "arrival counter's round trip, `last` the last arriver's partial reads, epilogue "
             "and stores;",
             "- owned tiles: `epilogue` from the K-sum to the stores completed.", "",
             "Stamps of the phases that end in a wait (`last`, `epilogue`) are taken after the "
             "wave's outstanding memory operations complete; the kernels of the library have "
             "no stamps.", "",
             "| configuration | grid | block | us/launch | gap | in-kernel | start spread | "
             "loop w0 | loop max | K-sum | ack | count | last | epilogue |",
             "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for q in rows:
        split = q["ack_us"] > 0
        f = lambda k, on=True: f"{q[k]:.2f}" if on else "-"
        lines.append(f"| {q['name']} | {q['grid']} | {q['block']} | {q['us_per_launch']:.2f} | "
                     f"{f('gap_us')} | {f('in_kernel_us')} | {f('start_spread_us')} | "
                     f"{f('loop_wave0_us')} | {f('loop_slowest_wave_us')} | "
                     f"{f('kwave_sum_us', q['waves_k'] > 1)} | "
                     f"{f('ack_us', split)} | {f('count_us', split)} | "
                     f"{f('last_arriver_us', split)} | {f('epilogue_us', not split)} |")
    with open(out_md, "w") as fo:
        fo.write("\n".join(lines) + "\n")
    log(f"[bench] wrote {out_md} ({len(rows)} configurations)")


def summarize_traffic(out_md):
    """The HBM-traffic table from the counter file that measured_traffic() reads."""
    import bit_quantized_gemm_token_amd as w8
    with open(PMC_FILE) as f:
        d = json.load(f)
    lines = ["# HBM traffic per GEMM launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
             "Two counter runs of `bench.py --counter-pass` (each problem's GEMM launched twice, "
             "one weight copy each, synchronized after every launch; then a plain float32 "
             "negation copy three times).  FETCH_SIZE counts the L2's requests to the fabric "
             "(reads served by the last-level cache included), so it bounds HBM reads from "
             "above.  Both counters are scaled by what they read for the copy of known size: "
             f"FETCH_SIZE x {d['fetch_scale']}, WRITE_SIZE x {d['write_scale']} "
             f"(the copy moves {d['copy_bytes'] // 1024} KiB each way).  Kernel sources hash "
             f"{d['source_hash']}.", "", "Commands (from /tmp on the MI355X box, repository at "
             "$R):", "", "```", d.get("command", ""), "```", "",
             "| format | M | N | K | layout | config | HBM bytes (scaled) | algorithmic bytes | "
             "ratio |", "|---|---:|---:|---:|---|---|---:|---:|---:|"]
    ratios = []
    for r in d["problems"]:
        hbm = r["fetch_kib"] * d["fetch_scale"] * 1024 + r["write_kib"] * d["write_scale"] * 1024
        alg = w8.algorithmic_bytes(r["fmt"], r["M"], r["N"], r["K"])
        ratios.append(hbm / alg)
        lines.append(f"| {r['fmt']} | {r['M']} | {r['N']} | {r['K']} | {r['layout']} | "
                     f"{_cfg_str(r['cfg'])} | {hbm:,.0f} | {alg:,} | {hbm / alg:.3f} |")
    lines += ["", f"Geomean ratio {geomean(ratios):.3f} over {len(ratios)} problems."]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    log(f"[bench] wrote {out_md}")


def summarize_mfma(manifest_path, counter_csv, out_md, command):
    """MFMA utilisation per problem from one counter pass: busy cycles over the
    dispatch time, executed MFMA ops against the algorithmic 2MNK."""
    import csv
    with open(manifest_path) as f:
        man = json.load(f)
    per = {}
    with open(counter_csv, newline="") as f:
        for r in csv.DictReader(f):
            if "gemm_kernel<" not in r["Kernel_Name"]:
                continue
            key = int(r.get("Dispatch_Id") or r.get("Correlation_Id") or 0)
            e = per.setdefault(key, {})
            e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                e["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    disp = [per[k] for k in sorted(per)]
    if len(disp) != len(man["gemm_dispatch_order"]):
        raise SystemExit(f"{counter_csv}: {len(disp)} GEMM dispatches, expected "
                         f"{len(man['gemm_dispatch_order'])}")
    acc = {}
    for i, e in zip(man["gemm_dispatch_order"], disp):
        acc.setdefault(i, []).append(e)
    lines = ["# MFMA utilisation per GEMM launch (rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES, "
             "SQ_INSTS_VALU_MFMA_MOPS_F8/_I8)", "",
             "One counter run of `bench.py --counter-pass` (each problem's GEMM launched twice, "
             "synchronized after every launch).  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES (summed over "
             "the SIMDs) / (dispatch duration x 2.4 GHz x 1024 SIMDs).  Executed MFMA ops = MOPS "
             "x 512 against the algorithmic 2MNK: one MFMA serves a group of token rows (16, "
             "or 16/T on the K-segmented layout segT, whose MFMA keeps only T diagonal blocks of "
             "its products), so executed / 2MNK = 16 x (token groups) / M, 16 at M = 1 on any "
             "layout, more where a stage's first steps run masked; and their rate against the "
             "dense fp8 / int8 MFMA peak (5.0 POP/s).", "",
             "Command (from /tmp on the MI355X box, repository at $R):", "", "```", command, "```",
             "", "| format | M | N | K | layout | config | dispatch us | MFMA busy % | "
             "executed MFMA ops | 2MNK | executed / 2MNK | TOP/s | % of peak |",
             "|---|---:|---:|---:|---|---|---:|---:|---:|---:|---:|---:|---:|"]
    for i, pr in enumerate(man["problems"]):
        es = acc.get(i, [])
        if not es:
            continue
        ns = sum(e.get("ns", 0.0) for e in es) / len(es)
        busy = sum(e.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for e in es) / len(es)
        mops = sum(e.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0) + e.get("SQ_INSTS_VALU_MFMA_MOPS_I8", 0.0)
                   for e in es) / len(es) * 512
        alg = 2 * pr["M"] * pr["N"] * pr["K"]
        busy_pct = 100 * busy / (ns * 2.4 * 1024) if ns else 0.0
        tops = mops / ns / 1e3 if ns else 0.0
        lines.append(f"| {pr['fmt']} | {pr['M']} | {pr['N']} | {pr['K']} | "
                     f"{pr.get('layout', '')} | {_cfg_str(pr['cfg'])} | "
                     f"{ns / 1e3:.2f} | {busy_pct:.2f} | {mops:,.0f} | {alg:,} | {mops / alg:.2f} | "
                     f"{tops:.1f} | {100 * tops / 5000:.2f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    log(f"[bench] wrote {out_md}")


def summarize_counters(manifest_path, counter_csv, out_md, command):
    """Per-problem memory-pipeline counters from one counter pass (rocprofv3
    --pmc with TA_BUSY_avr, TCC_HIT_sum, TCC_MISS_sum, SQ_WAVES,
    SQ_INSTS_VMEM_RD): how busy the vector-memory path of a compute unit is
    during a launch, and how many L2 requests hit."""
    import csv
    with open(manifest_path) as f:
        man = json.load(f)
    per = {}
    with open(counter_csv, newline="") as f:
        for r in csv.DictReader(f):
            if "gemm_kernel<" not in r["Kernel_Name"]:
                continue
            key = int(r.get("Dispatch_Id") or r.get("Correlation_Id") or 0)
            e = per.setdefault(key, {})
            e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            if r.get("Start_Timestamp") and r.get("End_Timestamp"):
                e["ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    disp = [per[k] for k in sorted(per)]
    if len(disp) != len(man["gemm_dispatch_order"]):
        raise SystemExit(f"{counter_csv}: {len(disp)} GEMM dispatches, expected "
                         f"{len(man['gemm_dispatch_order'])}")
    acc = {}
    for i, e in zip(man["gemm_dispatch_order"], disp):
        acc.setdefault(i, []).append(e)

    def mean(es, c):
        return sum(e.get(c, 0.0) for e in es) / len(es)

    lines = ["# Vector-memory path and L2 per GEMM launch (rocprofv3 TA_BUSY, TCC_HIT/MISS, "
             "SQ_WAVES, SQ_INSTS_VMEM_RD)", "",
             "One counter run of `bench.py --counter-pass` (each problem's GEMM launched twice on "
             "two weight copies, synchronized after every launch; averages of the two).  "
             "Dispatch us: the counter run's dispatch time (the profiler serializes and "
             "instruments each launch, so it is longer than under graph replay).  TA busy = "
             "TA_BUSY_avr, the busy cycles of the texture-address unit (one per compute unit) "
             "averaged over the units; TA busy % = that over the dispatch time at 2.4 GHz, the "
             "share of the launch in which an average compute unit's vector-memory path is "
             "issuing addresses.  VMEM rd = vector-memory read instructions issued in the whole "
             "launch (SQ_INSTS_VMEM_RD), waves = SQ_WAVES.  L2 hit % = TCC_HIT / (TCC_HIT + "
             "TCC_MISS) over all L2 requests of the launch (weights stream past the L2 and miss; "
             "activations, scales and split-K partials re-read by many workgroups hit).", "",
             "Command (from /tmp on the MI355X box, repository at $R):", "", "```", command, "```",
             "", "| format | M | N | K | layout | config | dispatch us | waves | VMEM rd | "
             "TA busy cycles | TA busy % | L2 hit % |",
             "|---|---:|---:|---:|---|---|---:|---:|---:|---:|---:|---:|"]
    for i, pr in enumerate(man["problems"]):
        es = acc.get(i, [])
        if not es:
            continue
        ns = mean(es, "ns")
        ta = mean(es, "TA_BUSY_avr")
        hit, miss = mean(es, "TCC_HIT_sum"), mean(es, "TCC_MISS_sum")
        lines.append(
            f"| {pr['fmt']} | {pr['M']} | {pr['N']} | {pr['K']} | {pr.get('layout', '')} | "
            f"{_cfg_str(pr['cfg'])} | {ns / 1e3:.2f} | {mean(es, 'SQ_WAVES'):,.0f} | "
            f"{mean(es, 'SQ_INSTS_VMEM_RD'):,.0f} | {ta:,.0f} | "
            f"{100 * ta / (ns * 2.4) if ns else 0:.1f} | "
            f"{100 * hit / (hit + miss) if hit + miss else 0:.1f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    log(f"[bench] wrote {out_md}")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--rotate-mib", type=int, default=1024)
    p.add_argument("--formats", default="FP8_Dynamic,W8A8_INT8,Block_FP8")
    p.add_argument("--cpu-budget-s", type=float, default=20.0)
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--table", default=None, help="config table to load instead of the shipped one")
    p.add_argument("--layout", choices=("table", "row", "packed", "seg2", "seg4", "seg8"),
                   default="table",
                   help="weight layout: the fastest one per the table (default), or forced")
    p.add_argument("--report", default=None, help="write per-problem results (JSON) here")
    p.add_argument("--no-moe", action="store_true", help="skip the MoE grouped GEMM measurement")
    p.add_argument("--counter-pass", default=None, metavar="MANIFEST",
                   help="instead of timing, make the launches for a rocprofv3 --pmc run and "
                        "write their order to MANIFEST")
    p.add_argument("--copy-calibration-mib", type=int, default=256,
                   help="size of the plain device copy in a counter pass")
    p.add_argument("--ingest-counters", nargs=3, default=None,
                   metavar=("MANIFEST", "FETCH_CSV", "WRITE_CSV"),
                   help="write the HBM counter file from a counter pass's manifest and the "
                        "FETCH_SIZE and WRITE_SIZE counter-collection CSVs, then exit")
    p.add_argument("--ingest-command", default="",
                   help="the commands that made the counter runs, recorded with them")
    p.add_argument("--summarize-trace", nargs=2, default=None, metavar=("STATS_CSV", "OUT_MD"),
                   help="write the kernel-trace summary (profiles/*.md) from a rocprofv3 "
                        "--kernel-trace --stats kernel_stats.csv, then exit")
    p.add_argument("--summarize-traffic", default=None, metavar="OUT_MD",
                   help="write the HBM-traffic summary from the counter file, then exit")
    p.add_argument("--summarize-mfma", nargs=3, default=None,
                   metavar=("MANIFEST", "COUNTER_CSV", "OUT_MD"),
                   help="write the MFMA-utilisation summary from a counter pass with "
                        "SQ_VALU_MFMA_BUSY_CYCLES and SQ_INSTS_VALU_MFMA_MOPS_F8/_I8, then exit")
    p.add_argument("--summarize-counters", nargs=3, default=None,
                   metavar=("MANIFEST", "COUNTER_CSV", "OUT_MD"),
                   help="write the vector-memory and L2 counter summary from a counter pass with "
                        "TA_BUSY_avr, TCC_HIT_sum, TCC_MISS_sum, SQ_WAVES, SQ_INSTS_VMEM_RD, "
                        "then exit")
    p.add_argument("--phases", default=None, metavar="OUT_MD",
                   help="run the phase probe (w8_phase_probe) and write its summary, then exit")
    p.add_argument("--bench-line", default=None, metavar="JSON",
                   help="with --summarize-trace: an unprofiled bench run's output line, whose "
                        "dominant kernel the summary reports")
    p.add_argument("--summary-command", default="",
                   help="the command that made the profile, recorded in the summary")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Problem:
    def __init__(self, w8, fmt, M, N, K, rotate_bytes, dev, layout="table"):
        self.fmt, self.M, self.N, self.K = fmt, M, N, K
        # the weight layout the table times best for this shape (row-major if
        # none): 0 row-major, 1 packed, 2/4/8 K-segmented packed
        self.packed = w8.best_layout(fmt, M, N, K) if layout == "table" else w8.LAYOUTS[layout]
        self.layout_name = w8.LAYOUT_NAMES[self.packed]
        self.cfg, self.from_table = w8.resolve_config(fmt, M, N, K, packed=self.packed)
        self.bytes = w8.algorithmic_bytes(fmt, M, N, K)
        x_bits = synthetic.activations(fmt, M, N, K)
        self.x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        if fmt == "W8A8_INT8":
            wq_np, sw_np = synthetic.int8_weights(fmt, M, N, K)
            wq = torch.from_numpy(wq_np).to(dev)
            self.sw = torch.from_numpy(sw_np).to(dev)
        else:
            w = torch.from_numpy(synthetic.fp32_weights(fmt, M, N, K)).to(dev)
            wq, self.sw = w8.quantize_weight(fmt, w)
            del w
        self.R = max(2, math.ceil(rotate_bytes / (N * K)))
        self.wbytes = w8.packed_weight_size(fmt, N, K, self.packed) if self.packed else N * K
        if self.packed:
            pk = w8.pack_weight(fmt, wq, layout=self.packed)
            self.pool = torch.empty((self.R, pk.data.numel()), dtype=torch.uint8, device=dev)
            self.pool.copy_(pk.data.unsqueeze(0).expand(self.R, -1))
            self.weights = [w8.PackedWeight(fmt, N, K, self.pool[r], self.packed)
                            for r in range(self.R)]
        else:
            self.pool = torch.empty((self.R, N, K), dtype=wq.dtype, device=dev)
            self.pool.copy_(wq.unsqueeze(0).expand(self.R, N, K))
            self.weights = [self.pool[r] for r in range(self.R)]
        self.wq = self.weights[0]
        self.xq, self.sx = w8.quantize_act(fmt, self.x)
        # one output per graph, so each graph's replayed result can be checked
        self.y_gemm = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        self.y_path = torch.empty_like(self.y_gemm)
        self.y_linear = torch.empty_like(self.y_gemm)
        self.ws = w8.Workspace(dev, max(w8.workspace_size(fmt, M, N, K, self.cfg,
                                                          packed=self.packed), 256))
        # the linear layer through w8_linear, with its own table entry for the
        # same weight layout (fused kernel or quantize launch + GEMM)
        self.cfg_l, self.from_table_l = w8.resolve_config(fmt, M, N, K, packed=self.packed,
                                                          op="linear")
        self.ws_l = w8.Workspace(dev, max(w8.workspace_size(fmt, M, N, K, self.cfg_l,
                                                            packed=self.packed, op="linear"), 256))
        # the kernel instance (its name in a rocprofv3 trace): token blocks of
        # 16 rows, or of 16/T on the K-segmented layouts (one launch's)
        rows = 16 // max(self.packed, 1)
        mb = min(2, -(-M // rows))
        c = self.cfg
        self.kernel = (f"gemm_kernel<{w8.FORMATS[fmt]}, {mb}, {c.tile_n // rows}, {c.waves_k}, "
                       f"{c.waves_n}, {c.unroll}, {c.swap_ab}, {self.packed}, {c.x_lds}, "
                       f"{1 if c.grid > 0 else 0}>")

    def run_gemm(self, w8):
        for r in range(self.R):
            w8.gemm_w8a8(self.fmt, self.xq, self.sx, self.weights[r], self.sw, cfg=self.cfg,
                         y=self.y_gemm, workspace=self.ws)

    def run_path(self, w8):
        for r in range(self.R):
            xq, sx = w8.quantize_act(self.fmt, self.x, xq=self.xq, sx=self.sx)
            w8.gemm_w8a8(self.fmt, xq, sx, self.weights[r], self.sw, cfg=self.cfg, y=self.y_path,
                         workspace=self.ws)

    def run_linear(self, w8):
        for r in range(self.R):
            w8.linear(self.fmt, self.x, self.weights[r], self.sw, cfg=self.cfg_l, y=self.y_linear,
                      workspace=self.ws_l, fused=True)

    def capture(self, w8, stream):
        self.g_gemm = torch.cuda.CUDAGraph()
        self.g_path = torch.cuda.CUDAGraph()
        self.g_linear = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g_gemm, stream=stream):
            self.run_gemm(w8)
        with torch.cuda.graph(self.g_path, stream=stream):
            self.run_path(w8)
        with torch.cuda.graph(self.g_linear, stream=stream):
            self.run_linear(w8)


# ------------------------------------------------------------------ MoE --
# The MoE layers of synthetic.MOE_SHAPES (128 experts, top-8) at the token
# counts synthetic.MOE_TOKENS.  Synthetic: random codes and scales, seeded
# routing.
MOE_E, MOE_TOPK = synthetic.MOE_E, synthetic.MOE_TOPK
MOE_SHAPES, MOE_TOKENS = synthetic.MOE_SHAPES, synthetic.MOE_TOKENS


def _random_codes(fmt, shape, dev, gen):
    c = torch.randint(0, 256, shape, dtype=torch.int32, device=dev, generator=gen).to(torch.uint8)
    if fmt == "W8A8_INT8":
        c[c == 0x80] = 0x81
    else:
        c[(c & 0x7F) == 0x7F] = 0x38
    return c


def moe_bench(w8, dev, rotate_bytes, warmup, reps):
    """Per (format, projection, token count): one graph of G grouped-GEMM calls,
    call j on weight copy j % R with routing seed j, so the distinct expert
    weights a graph reads exceed the last-level cache; beside it the same
    calls as one dense GEMM launch per active expert (rows gathered
    beforehand), and from the bf16 tokens: moe_linear (quantization fused)
    and quantize_act + moe_gemm.  us per call = median graph time / G."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    rows_out = []
    for fmt in ("FP8_Dynamic", "W8A8_INT8", "Block_FP8"):
        for name, N, K in MOE_SHAPES:
            pbytes = w8.packed_weight_size(fmt, N, K)
            set_bytes = MOE_E * pbytes
            R = max(2, math.ceil(rotate_bytes / set_bytes))
            weights = [w8.PackedExperts(fmt, N, K, _random_codes(fmt, (MOE_E, pbytes), dev, gen))
                       for _ in range(R)]
            nsw = N if fmt != "Block_FP8" else ((N + 127) // 128) * (K // 128)
            sw = (torch.rand((MOE_E, nsw), device=dev, generator=gen) * 0.01 + 0.001)
            for T in MOE_TOKENS:
                active = min(MOE_E, MOE_TOPK * T)
                G = max(R, min(64, math.ceil(rotate_bytes / (active * pbytes))))
                bits = synthetic.activations(fmt, T, N, K)
                x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
                xq, sx = w8.quantize_act(fmt, x)
                calls = []
                for j in range(G):
                    off, rows = synthetic.moe_routing(T, MOE_E, MOE_TOPK, seed=1000 * T + j)
                    calls.append((weights[j % R], torch.from_numpy(off).to(dev),
                                  torch.from_numpy(rows).to(dev), off, rows))
                # an expert holds at most T rows (top-k picks distinct experts)
                cfg, from_table = w8.moe_config(fmt, MOE_E, T, N, K, T, packed=True)
                cfg_l, from_table_l = w8.moe_linear_config(fmt, MOE_E, T, N, K, T, packed=True)
                ws = w8.Workspace(dev, max(256, w8.moe_workspace_size(fmt, MOE_E, T, N, K, T, cfg,
                                                                      packed=True),
                                           w8.moe_workspace_size(fmt, MOE_E, T, N, K, T, cfg_l,
                                                                 packed=True)))
                y = torch.empty((T * MOE_TOPK, N), dtype=torch.bfloat16, device=dev)
                # per-expert dense launches: gathered rows and configs prepared up front
                dense = []
                for wt, _, _, off, rows in calls:
                    for e in range(MOE_E):
                        a, b = int(off[e]), int(off[e + 1])
                        if b > a:
                            r = torch.from_numpy(rows[a:b].astype(np.int64)).to(dev)
                            dense.append((xq[r].contiguous(), sx[r].contiguous(),
                                          w8.PackedWeight(fmt, N, K, wt.data[e]), sw[e],
                                          y[a:b], w8.resolve_config(fmt, b - a, N, K,
                                                                    packed=True)[0]))
                wsd = w8.Workspace(dev, max([256] + [w8.workspace_size(fmt, d[0].shape[0], N, K,
                                                                       d[5], packed=True)
                                                     for d in dense]))
                stream = torch.cuda.Stream(dev)
                stream.wait_stream(torch.cuda.current_stream(dev))
                g_moe, g_dense = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
                g_lin, g_qm = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
                with torch.cuda.graph(g_moe, stream=stream):
                    for wt, offt, rowst, _, _ in calls:
                        w8.moe_gemm(fmt, xq, sx, offt, rowst, wt, sw, max_m=T, cfg=cfg, y=y,
                                    workspace=ws)
                # from bf16 tokens: fused (moe_linear), and quantize_act + moe_gemm
                with torch.cuda.graph(g_lin, stream=stream):
                    for wt, offt, rowst, _, _ in calls:
                        w8.moe_linear(fmt, x, offt, rowst, wt, sw, max_m=T, cfg=cfg_l, y=y,
                                      workspace=ws)
                with torch.cuda.graph(g_qm, stream=stream):
                    for wt, offt, rowst, _, _ in calls:
                        xq2, sx2 = w8.quantize_act(fmt, x)
                        w8.moe_gemm(fmt, xq2, sx2, offt, rowst, wt, sw, max_m=T, cfg=cfg, y=y,
                                    workspace=ws)
                with torch.cuda.graph(g_dense, stream=stream):
                    for d in dense:
                        w8.gemm_w8a8(fmt, d[0], d[1], d[2], d[3], cfg=d[5], y=d[4], workspace=wsd)
                t = {"moe": [], "dense": [], "linear": [], "quant_moe": []}
                with torch.cuda.stream(stream):
                    for i in range(warmup + reps):
                        for key, gr in (("moe", g_moe), ("dense", g_dense), ("linear", g_lin),
                                        ("quant_moe", g_qm)):
                            e0 = torch.cuda.Event(enable_timing=True)
                            e1 = torch.cuda.Event(enable_timing=True)
                            e0.record(stream)
                            gr.replay()
                            e1.record(stream)
                            e1.synchronize()
                            if i >= warmup:
                                t[key].append(e0.elapsed_time(e1) * 1e3 / G)
                us, us_d, us_l, us_qm = (sorted(t[k])[len(t[k]) // 2]
                                         for k in ("moe", "dense", "linear", "quant_moe"))
                n_act = np.mean([int((np.diff(c[3]) > 0).sum()) for c in calls])
                byts = n_act * (N * K + 4 * nsw) + T * K + T * MOE_TOPK * N * 2
                rows_out.append({"fmt": fmt, "proj": name, "N": N, "K": K, "T": T,
                                 "active_experts": float(n_act), "calls": G, "copies": R,
                                 "cfg": cfg.as_dict(), "cfg_from_table": bool(from_table),
                                 "cfg_linear": cfg_l.as_dict(),
                                 "cfg_linear_from_table": bool(from_table_l),
                                 "us": round(us, 3), "us_linear": round(us_l, 3),
                                 "us_quant_plus_moe": round(us_qm, 3),
                                 "us_per_expert_launches": round(us_d, 3),
                                 "gbps": round(byts / (us * 1e3), 1)})
                log(f"[moe] {fmt} {name} T={T}: {us:.2f} us ({byts / (us * 1e3):.0f} GB/s), "
                    f"per-expert launches {us_d:.2f} us, {n_act:.0f} experts active; from bf16: "
                    f"fused {us_l:.2f} us, quantize + grouped {us_qm:.2f} us")
                del g_moe, g_dense, g_lin, g_qm, dense
            del weights
            torch.cuda.empty_cache()
    return {"workload": f"{MOE_E} experts, top-{MOE_TOPK}, gate_up 1536x2048 and down 2048x768, "
                        f"T in {list(MOE_TOKENS)}, 3 formats, packed weights",
            "problems": len(rows_out),
            "geomean_us": round(geomean([r["us"] for r in rows_out]), 3),
            "geomean_gbps": round(geomean([r["gbps"] for r in rows_out]), 1),
            "geomean_speedup_vs_per_expert_launches": round(
                geomean([r["us_per_expert_launches"] / r["us"] for r in rows_out]), 3),
            "geomean_us_linear_fused": round(geomean([r["us_linear"] for r in rows_out]), 3),
            "geomean_us_quant_plus_moe": round(
                geomean([r["us_quant_plus_moe"] for r in rows_out]), 3),
            "rows": rows_out}


# Launch shapes tried for the read floor (grid, waves per workgroup, chunks
# in flight per wave); the fastest counts.
FLOOR_SHAPES = ((128, 8, 2), (256, 4, 2), (256, 8, 2), (512, 4, 2), (512, 4, 4), (512, 8, 2),
                (1024, 4, 2), (1024, 4, 4))


def read_floors(w8, problems, stream, reps=7):
    """Per distinct weight size B: the time of one launch of the library's
    read-floor kernel (w8_read_floor) streaming B bytes, graph-replayed over
    the same rotating weight copies the GEMM reads (R launches per graph,
    launch r on copy r), median over replays, fastest of FLOOR_SHAPES."""
    sink = torch.empty(1024 * 16, dtype=torch.int32, device=problems[0].x.device)
    out = {}
    for p in problems:
        if p.wbytes in out:
            continue
        flat = p.pool.view(-1)
        best = None
        for grid, waves, depth in FLOOR_SHAPES:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for r in range(p.R):
                    w8.read_floor(flat[r * p.wbytes:(r + 1) * p.wbytes], p.wbytes, sink, grid,
                                  waves, depth)
            ts = []
            with torch.cuda.stream(stream):
                for i in range(reps + 2):
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    g.replay()
                    e1.record(stream)
                    e1.synchronize()
                    if i >= 2:
                        ts.append(e0.elapsed_time(e1) * 1e3 / p.R)
            us = sorted(ts)[len(ts) // 2]
            if best is None or us < best["us"]:
                best = {"us": us, "grid": grid, "waves": waves, "depth": depth}
            del g
        out[p.wbytes] = best
        log(f"[bench] read floor {p.wbytes} B: {best['us']:.3f} us "
            f"(grid {best['grid']}, {best['waves']} waves, depth {best['depth']})")
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def context_floors(dev, nbytes):
    """Two device figures the small-shape results are read against: the cost
    of one launch of a one-element kernel under graph replay, and the rate of
    a plain device copy of `nbytes` (torch's copy_, counting the bytes read
    and written)."""
    s = torch.cuda.Stream(dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    t = torch.zeros(1, device=dev)
    n = 1000
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(n):
            t.add_(1.0)
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)  # first call outside the timing
    launch, copy = [], []
    with torch.cuda.stream(s):
        for i in range(7):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(s)
            g.replay()
            e[1].record(s)
            dst.copy_(src)
            e[2].record(s)
            e[2].synchronize()
            if i >= 2:
                launch.append(e[0].elapsed_time(e[1]) * 1e3 / n)
                copy.append(2 * nbytes / (e[1].elapsed_time(e[2]) * 1e6))
    del g, src, dst
    return {"launch_floor_us": round(sorted(launch)[len(launch) // 2], 3),
            "copy_gbps": round(sorted(copy)[len(copy) // 2], 1),
            "copy_bytes": nbytes}


def geomean(v):
    v = [x for x in v if x > 0]
    return math.exp(sum(math.log(x) for x in v) / len(v)) if v else 0.0


def cpu_baseline(problems, budget_s, threads=None, refcheck=True):
    """The oracle, timed on the host: passes over the problems (quantize + GEMM
    of each) until `budget_s` seconds of oracle time are spent; per problem the
    fastest run counts.  threads: the oracle's OpenMP thread count (None: all
    it would use)."""
    import oracle
    oracle._load()
    if threads:
        oracle.set_threads(threads)
    inputs = []
    for p in problems:
        x_bits = synthetic.activations(p.fmt, p.M, p.N, p.K)
        if p.fmt == "W8A8_INT8":
            wq, sw = synthetic.int8_weights(p.fmt, p.M, p.N, p.K)
            wq = wq.view(np.uint8)
        else:
            wq, sw = oracle.quantize_weight(p.fmt, synthetic.fp32_weights(p.fmt, p.M, p.N, p.K))
        inputs.append((x_bits, wq, sw))
    best = [math.inf] * len(problems)
    done, t_total, passes = set(), 0.0, 0
    while t_total < budget_s and (passes == 0 or len(done) == len(problems)):
        for i, (p, (x_bits, wq, sw)) in enumerate(zip(problems, inputs)):
            if t_total >= budget_s and (passes > 0 or not refcheck):
                break
            t0 = time.perf_counter()
            Y, _, _ = oracle.forward(p.fmt, x_bits, wq, sw)
            dt = time.perf_counter() - t0
            t_total += dt
            best[i] = min(best[i], dt)
            if i not in done and refcheck:
                # refcheck: the GPU outputs of this problem's three replayed
                # graphs (GEMM, quantize + GEMM, linear layer) against the oracle
                ok = True
                for y in (p.y_gemm, p.y_path, p.y_linear):
                    got = y.float().cpu().numpy().astype(np.float64)
                    ok = ok and bool((np.abs(got - Y) <= 1e-2 + 1e-2 * np.abs(Y)).all())
                p.refcheck = ok
            done.add(i)
        passes += 1
    checked = [problems[i] for i in sorted(done)]
    gbps = [problems[i].bytes / (best[i] * 1e9) for i in sorted(done)]
    return {
        "value": round(geomean(gbps), 4),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"{len(checked)} of {len(problems)} problems "
                   f"({', '.join(sorted(set(p.fmt for p in checked)))}), quantize + GEMM, "
                   f"{passes} passes in {t_total:.1f} s of CPU work, fastest run per problem; "
                   f"geomean of algorithmic bytes / time"),
    }, checked


def main():
    args = parse()
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters, PMC_FILE, args.ingest_command)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, args.summary_command, args.bench_line)
        return
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma, args.summary_command)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.summary_command)
        return
    if args.phases:
        phase_study(args.phases, args.summary_command)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import bit_quantized_gemm_token_amd as w8
    if args.table:
        w8.clear_config_table()
        w8.load_config_table(args.table)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fmts = args.formats.split(",")
    rotate = args.rotate_mib << 20

    problems = []
    t0 = time.time()
    for fmt in fmts:
        for (M, N, K) in synthetic.SWEEP:
            problems.append(Problem(w8, fmt, M, N, K, rotate, dev, args.layout))
    torch.cuda.synchronize()
    log(f"[bench] {len(problems)} problems set up in {time.time() - t0:.1f} s "
        f"({sum(p.from_table == 1 for p in problems)} configs from the table)")
    if args.counter_pass:
        counter_pass(problems, w8, args.counter_pass, args.copy_calibration_mib)
        return
    stream = torch.cuda.Stream(dev)
    t0 = time.time()
    for p in problems:
        p.capture(w8, stream)
    torch.cuda.synchronize()
    log(f"[bench] graphs captured in {time.time() - t0:.1f} s "
        f"({sum(p.R for p in problems)} GEMMs per graph set)")

    def step(record):
        for p in problems:
            if record:
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
                ev[0].record(stream)
                p.g_gemm.replay()
                ev[1].record(stream)
                p.g_path.replay()
                ev[2].record(stream)
                p.g_linear.replay()
                ev[3].record(stream)
                p.events.append(ev)
            else:
                p.g_gemm.replay()
                p.g_path.replay()
                p.g_linear.replay()

    with torch.cuda.stream(stream):
        for p in problems:
            p.events = []
        for i in range(args.warmup):
            step(False)
        torch.cuda.synchronize()
        log(f"[bench] {args.warmup} warmup steps done")
        t_start = time.perf_counter()
        for i in range(args.steps):
            step(True)
        torch.cuda.synchronize()
        t_elapsed = time.perf_counter() - t_start
    log(f"[bench] {args.steps} timed steps in {t_elapsed:.2f} s")

    for p in problems:
        g = sorted(e[0].elapsed_time(e[1]) for e in p.events)
        a = sorted(e[1].elapsed_time(e[2]) for e in p.events)
        f = sorted(e[2].elapsed_time(e[3]) for e in p.events)
        p.us_gemm = g[len(g) // 2] * 1e3 / p.R
        p.us_path = a[len(a) // 2] * 1e3 / p.R
        p.us_linear = f[len(f) // 2] * 1e3 / p.R
        p.gbps = p.bytes / (p.us_gemm * 1e3)
        p.gbps_path = p.bytes / (p.us_path * 1e3)
        p.us_gemm_min = g[0] * 1e3 / p.R
        p.us_gemm_p90 = g[min(len(g) - 1, math.ceil(0.9 * len(g)) - 1)] * 1e3 / p.R
    torch.cuda.synchronize()

    # refcheck of the timed graphs themselves: each output cleared to NaN, each
    # graph replayed once, and its result compared bit for bit with an eager
    # call of the same config (and, below, with the oracle)
    graph_equal = 0
    with torch.cuda.stream(stream):
        for p in problems:
            for y in (p.y_gemm, p.y_path, p.y_linear):
                y.fill_(float("nan"))
            p.g_gemm.replay()
            p.g_path.replay()
            p.g_linear.replay()
    torch.cuda.synchronize()
    for p in problems:
        eager = w8.linear(p.fmt, p.x, p.wq, p.sw, cfg=p.cfg)
        eager_l = w8.linear(p.fmt, p.x, p.wq, p.sw, cfg=p.cfg_l, fused=True)
        torch.cuda.synchronize()
        same = lambda a, b: torch.equal(a.view(torch.int16), b.view(torch.int16))
        p.graph_equal = (same(p.y_gemm, eager) and same(p.y_path, eager) and
                         same(p.y_linear, eager_l))
        graph_equal += p.graph_equal
        if not p.graph_equal:
            log(f"[bench] graph replay differs from eager: {p.fmt} {p.M}x{p.N}x{p.K}")
    log(f"[bench] graph-replayed outputs equal to eager: {graph_equal}/{len(problems)}")

    floors = read_floors(w8, problems, stream)
    for p in problems:
        p.floor_us = floors[p.wbytes]["us"]
        p.frac_of_floor = p.floor_us / p.us_gemm

    # dominant kernel instance
    by_kernel = {}
    for p in problems:
        by_kernel.setdefault(p.kernel, []).append(p)
    # the instance with the largest summed time of one GEMM per problem
    dom = max(by_kernel, key=lambda k: sum(p.us_gemm for p in by_kernel[k]))
    dp = by_kernel[dom]
    launches = sum(p.R for p in dp)
    achieved = sum(p.bytes * p.R for p in dp) / sum(p.us_gemm * 1e3 * p.R for p in dp)
    roofline = {
        "kernel": dom,
        "problems": [f"{p.fmt} {p.M}x{p.N}x{p.K}" for p in dp],
        "bound": "hbm",
        "achieved": round(achieved, 2),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "avg_launch_us": round(sum(p.us_gemm * p.R for p in dp) / launches, 4),
        "bytes_per_launch": round(sum(p.bytes * p.R for p in dp) / launches),
        "traffic": measured_traffic(dom, dp),
    }

    floors = context_floors(dev, 1 << 30)
    log(f"[bench] launch floor {floors['launch_floor_us']} us, plain copy "
        f"{floors['copy_gbps']} GB/s")

    # the MoE grouped GEMM, measured after the sweep (not part of the headline)
    moe = None
    if not args.no_moe:
        for p in problems:  # free the sweep's graphs and weight copies first
            p.g_gemm = p.g_path = p.g_linear = None
            p.pool = p.weights = p.wq = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        t0 = time.time()
        moe = moe_bench(w8, dev, rotate, args.warmup, max(args.steps // 2, 3))
        log(f"[bench] MoE measured in {time.time() - t0:.1f} s")

    cpu = None
    refcheck = {"graph_replay_equals_eager": f"{graph_equal}/{len(problems)}"}
    if not args.no_cpu:
        import oracle
        cpu, checked = cpu_baseline(problems, args.cpu_budget_s)
        refcheck["graph_outputs_vs_oracle"] = f"{sum(p.refcheck for p in checked)}/{len(checked)} pass"
        # one thread, on the FP8_Dynamic problems (a third of the sweep)
        one, _ = cpu_baseline([p for p in problems if p.fmt == fmts[0]], args.cpu_budget_s / 2,
                              threads=1, refcheck=False)
        cpu["one_thread"] = {k: one[k] for k in ("value", "unit", "cores", "sample")}
    else:
        refcheck["graph_outputs_vs_oracle"] = "skipped"

    per_fmt = {}
    for fmt in fmts:
        ps = [p for p in problems if p.fmt == fmt]
        per_fmt[fmt] = {"geomean_us_per_gemm": round(geomean([p.us_gemm for p in ps]), 4),
                        "geomean_gbps": round(geomean([p.gbps for p in ps]), 2),
                        "geomean_frac_of_floor": round(geomean([p.frac_of_floor for p in ps]), 4),
                        "geomean_us_quant_plus_gemm": round(geomean([p.us_path for p in ps]), 4),
                        "geomean_us_linear": round(geomean([p.us_linear for p in ps]), 4)}
    value = geomean([p.gbps for p in problems])
    out = {
        "metric": "geomean us/GEMM + achieved HBM GB/s, 8-bit GEMM sweep M<=32 (1 GPU)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_elapsed * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3/int8 (fp32/int32 acc)",
        "data": "synthetic",
        "config": {"workload": "24-shape M<=32 sweep x {FP8_Dynamic, W8A8_INT8, Block_FP8} "
                               "= 72 GEMMs, per-shape table configs, HIP graph replay over "
                               f"{args.rotate_mib} MiB of rotating weights per problem",
                   "problems": len(problems),
                   "table_hits": sum(p.from_table == 1 for p in problems),
                   "bucket_hits": sum(p.from_table == 2 for p in problems),
                   "packed_layout": sum(bool(p.packed) for p in problems),
                   "layouts": {n: sum(p.layout_name == n for p in problems)
                               for n in ("row", "packed", "seg2", "seg4", "seg8")}},
        "geomean_us_per_gemm": round(geomean([p.us_gemm for p in problems]), 4),
        "geomean_us_per_gemm_min": round(geomean([p.us_gemm_min for p in problems]), 4),
        "geomean_us_per_gemm_p90": round(geomean([p.us_gemm_p90 for p in problems]), 4),
        "geomean_us_quant_plus_gemm": round(geomean([p.us_path for p in problems]), 4),
        "geomean_gbps_quant_plus_gemm": round(geomean([p.gbps_path for p in problems]), 2),
        "geomean_us_linear": round(geomean([p.us_linear for p in problems]), 4),
        "geomean_gbps_linear": round(geomean([p.bytes / (p.us_linear * 1e3)
                                              for p in problems]), 2),
        "linear_fused_problems": sum(p.cfg_l.quant_launch == 0 for p in problems),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "context": dict(floors, frac_of_copy_bw=round(value / floors["copy_gbps"], 4)),
        "read_floor": {
            "what": "w8_read_floor: one launch streaming the problem's weight bytes, graph-replayed "
                    "over the same rotating copies; fastest of the launch shapes tried",
            "geomean_us": round(geomean([p.floor_us for p in problems]), 4),
            "geomean_frac_of_floor": round(geomean([p.frac_of_floor for p in problems]), 4),
            "worst_frac_of_floor": round(min(p.frac_of_floor for p in problems), 4),
            "problems_within_1_25x": sum(p.frac_of_floor >= 0.8 for p in problems)},
        "per_format": per_fmt,
        "refcheck": refcheck,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if moe is not None:
        out["moe"] = {k: v for k, v in moe.items() if k != "rows"}
    if args.report:
        rows = [{"fmt": p.fmt, "M": p.M, "N": p.N, "K": p.K, "cfg": p.cfg.as_dict(),
                 "layout": p.layout_name,
                 "from_table": p.from_table, "R": p.R, "bytes": p.bytes,
                 "us_gemm": round(p.us_gemm, 4), "us_gemm_min": round(p.us_gemm_min, 4),
                 "us_gemm_p90": round(p.us_gemm_p90, 4), "us_quant_plus_gemm": round(p.us_path, 4),
                 "floor_us": round(p.floor_us, 4), "frac_of_floor": round(p.frac_of_floor, 4),
                 "graph_equal": bool(p.graph_equal),
                 "us_linear": round(p.us_linear, 4), "cfg_linear": p.cfg_l.as_dict(),
                 "linear_from_table": p.from_table_l,
                 "gbps": round(p.gbps, 1), "frac": round(p.gbps / HBM_PEAK_GBPS, 4),
                 "kernel": p.kernel} for p in problems]
        with open(args.report, "w") as f:
            json.dump({"summary": out, "problems": rows,
                       "moe": moe["rows"] if moe else []}, f, indent=1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
