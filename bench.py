"""Benchmark: geomean us per GEMM and achieved HBM GB/s over the small-M 8-bit
GEMM sweep on one MI355X.

Workload: the 24 (M, N, K) shapes of synthetic.SWEEP (M <= 32) in each of the
three formats (FP8_Dynamic, W8A8_INT8, Block_FP8): 72 GEMM problems, each
with the config the library resolves from its per-shape table (the tuned
table shipped with the package; default config on a miss).

Per problem, two HIP graphs are captured once:
  gemm  R back-to-back GEMMs, each reading its own copy of the weights;
  path  R back-to-back (activation quantization + GEMM) pairs.
The R weight copies span at least --rotate-mib MiB (default 1024), more than
the last-level cache, so every weight byte read in the timed region comes
from HBM.  One step replays both graphs of every problem once; W warmup steps
are untimed, then K steps are timed, bracketed by device synchronization.

Per problem: us per GEMM = median over steps of (graph time / R).  The
headline value is the geometric mean over the 72 problems of the achieved
GB/s of the GEMM, algorithmic bytes (weights + activations + scales + bf16
output) / us per GEMM; geomean us per GEMM is reported beside it, and so is
the same pair for the whole path (quantize + GEMM).

roofline: the dominant GEMM kernel instance (largest summed time over the
problems that use it), achieved = its algorithmic bytes per launch / its
average launch time from the HIP events, against the 8 TB/s HBM peak.

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
    p.add_argument("--report", default=None, help="write per-problem results (JSON) here")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Problem:
    def __init__(self, w8, fmt, M, N, K, rotate_bytes, dev):
        self.fmt, self.M, self.N, self.K = fmt, M, N, K
        # the weight layout the table times best for this shape (row-major if none)
        self.packed = w8.best_layout(fmt, M, N, K)
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
        if self.packed:
            pk = w8.pack_weight(fmt, wq)
            self.pool = torch.empty((self.R, pk.data.numel()), dtype=torch.uint8, device=dev)
            self.pool.copy_(pk.data.unsqueeze(0).expand(self.R, -1))
            self.weights = [w8.PackedWeight(fmt, N, K, self.pool[r]) for r in range(self.R)]
        else:
            self.pool = torch.empty((self.R, N, K), dtype=wq.dtype, device=dev)
            self.pool.copy_(wq.unsqueeze(0).expand(self.R, N, K))
            self.weights = [self.pool[r] for r in range(self.R)]
        self.wq = self.weights[0]
        self.xq, self.sx = w8.quantize_act(fmt, self.x)
        self.y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        self.ws = w8.Workspace(dev, max(w8.workspace_size(fmt, M, N, K, self.cfg), 256))
        mb = (M + 15) // 16
        c = self.cfg
        self.kernel = (f"gemm_kernel<{w8.FORMATS[fmt]}, {mb}, {c.tile_n // 16}, {c.waves_k}, "
                       f"{c.unroll}, {c.swap_ab}, {int(self.packed)}>")

    def capture(self, w8, stream):
        self.g_gemm = torch.cuda.CUDAGraph()
        self.g_path = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g_gemm, stream=stream):
            for r in range(self.R):
                w8.gemm_w8a8(self.fmt, self.xq, self.sx, self.weights[r], self.sw, cfg=self.cfg,
                             y=self.y, workspace=self.ws)
        with torch.cuda.graph(self.g_path, stream=stream):
            for r in range(self.R):
                xq, sx = w8.quantize_act(self.fmt, self.x, xq=self.xq, sx=self.sx)
                w8.gemm_w8a8(self.fmt, xq, sx, self.weights[r], self.sw, cfg=self.cfg, y=self.y,
                             workspace=self.ws)


def geomean(v):
    v = [x for x in v if x > 0]
    return math.exp(sum(math.log(x) for x in v) / len(v)) if v else 0.0


def cpu_baseline(problems, budget_s):
    """The oracle on a bounded sample of the problems, timed on the host."""
    import oracle
    oracle._load()
    gbps, done, t_total = [], [], 0.0
    for p in problems:
        if t_total >= budget_s:
            break
        x_bits = synthetic.activations(p.fmt, p.M, p.N, p.K)
        if p.fmt == "W8A8_INT8":
            wq, sw = synthetic.int8_weights(p.fmt, p.M, p.N, p.K)
            wq = wq.view(np.uint8)
        else:
            wq, sw = oracle.quantize_weight(p.fmt, synthetic.fp32_weights(p.fmt, p.M, p.N, p.K))
        t0 = time.perf_counter()
        Y, _, _ = oracle.forward(p.fmt, x_bits, wq, sw)
        dt = time.perf_counter() - t0
        t_total += dt
        gbps.append(p.bytes / (dt * 1e9))
        # refcheck: the GPU output of this problem against the oracle
        got = p.y_check.float().cpu().numpy().astype(np.float64)
        p.refcheck = bool((np.abs(got - Y) <= 1e-2 + 1e-2 * np.abs(Y)).all())
        done.append(p)
    return {
        "value": round(geomean(gbps), 4),
        "unit": "GB/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"{len(done)} of {len(problems)} problems in sweep order "
                   f"({', '.join(sorted(set(p.fmt for p in done)))}), quantize + GEMM, one run "
                   f"each, {t_total:.1f} s of CPU work; geomean of algorithmic bytes / time"),
    }, done


def main():
    args = parse()
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
            problems.append(Problem(w8, fmt, M, N, K, rotate, dev))
    torch.cuda.synchronize()
    log(f"[bench] {len(problems)} problems set up in {time.time() - t0:.1f} s "
        f"({sum(p.from_table for p in problems)} configs from the table)")
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
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
                ev[0].record(stream)
                p.g_gemm.replay()
                ev[1].record(stream)
                p.g_path.replay()
                ev[2].record(stream)
                p.events.append(ev)
            else:
                p.g_gemm.replay()
                p.g_path.replay()

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
        p.us_gemm = g[len(g) // 2] * 1e3 / p.R
        p.us_path = a[len(a) // 2] * 1e3 / p.R
        p.gbps = p.bytes / (p.us_gemm * 1e3)
        p.gbps_path = p.bytes / (p.us_path * 1e3)
        p.us_gemm_min = g[0] * 1e3 / p.R
        p.us_gemm_p90 = g[min(len(g) - 1, int(0.9 * len(g)))] * 1e3 / p.R
        # one eager run for the refcheck
        p.y_check = w8.linear(p.fmt, p.x, p.wq, p.sw, cfg=p.cfg)
    torch.cuda.synchronize()

    # dominant kernel instance
    by_kernel = {}
    for p in problems:
        by_kernel.setdefault(p.kernel, []).append(p)
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
        "traffic": None,
    }

    cpu = None
    if not args.no_cpu:
        cpu, checked = cpu_baseline(problems, args.cpu_budget_s)
        refcheck = f"{sum(p.refcheck for p in checked)}/{len(checked)} pass"
    else:
        refcheck = "skipped"

    per_fmt = {}
    for fmt in fmts:
        ps = [p for p in problems if p.fmt == fmt]
        per_fmt[fmt] = {"geomean_us_per_gemm": round(geomean([p.us_gemm for p in ps]), 4),
                        "geomean_gbps": round(geomean([p.gbps for p in ps]), 2),
                        "geomean_us_quant_plus_gemm": round(geomean([p.us_path for p in ps]), 4)}
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
                   "table_hits": sum(p.from_table for p in problems),
                   "packed_layout": sum(bool(p.packed) for p in problems)},
        "geomean_us_per_gemm": round(geomean([p.us_gemm for p in problems]), 4),
        "geomean_us_quant_plus_gemm": round(geomean([p.us_path for p in problems]), 4),
        "geomean_gbps_quant_plus_gemm": round(geomean([p.gbps_path for p in problems]), 2),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "per_format": per_fmt,
        "refcheck": refcheck,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if args.report:
        rows = [{"fmt": p.fmt, "M": p.M, "N": p.N, "K": p.K, "cfg": p.cfg.as_dict(),
                 "layout": "packed" if p.packed else "row",
                 "from_table": p.from_table, "R": p.R, "bytes": p.bytes,
                 "us_gemm": round(p.us_gemm, 4), "us_gemm_min": round(p.us_gemm_min, 4),
                 "us_gemm_p90": round(p.us_gemm_p90, 4), "us_quant_plus_gemm": round(p.us_path, 4),
                 "gbps": round(p.gbps, 1), "frac": round(p.gbps / HBM_PEAK_GBPS, 4),
                 "kernel": p.kernel} for p in problems]
        with open(args.report, "w") as f:
            json.dump({"summary": out, "problems": rows}, f, indent=1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
