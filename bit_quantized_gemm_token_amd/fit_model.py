"""Measured data for the config cost model, and the fit of its constants.

    python -m bit_quantized_gemm_token_amd.fit_model collect --out CSV
           [--formats ...] [--layouts packed] [--ops gemm] [--shapes M,N,K;...]
           [--replays 3] [--rotate-mib 256] [--time-budget-s 0]
    python -m bit_quantized_gemm_token_amd.fit_model fit CSV [--top-n 16] [--params a,b]
    python -m bit_quantized_gemm_token_amd.fit_model bucket-eval --shapes M,N,K;...

collect (GPU): for every shape, layout and op, times every candidate of the
tuner's feasible set with the tuner's own harness (w8_profile_configs: graph
replays over rotating weight copies) and appends one CSV row per candidate:
fmt, op, layout, M, N, K, the config fields, the measured us (empty when the
config failed validation) and the model's current prediction.

fit (CPU): fits the constants of the model in csrc/w8_model.cpp to those
timings (a ranking loss plus a weighted log-time error, Nelder-Mead over the
constants, which enter the model non-linearly) and reports how good the model's
top-1 and the best of its top-N are against the measured best -- the two
quantities the flashinfer-ai/flashinfer pull 3948 discussion weighs (top-1
geomean, and the loss of autotuning only a top-N ranked list).  Every
prediction comes from the library's own model (w8_predict_us, with the trial
constants passed in), so the fit tunes exactly the model the library ships;
the printed constants go into kParams in csrc/w8_model.cpp.

bucket-eval (GPU): for shapes whose M has no table entry but whose
floor(log2 M) bucket has one, times the bucket entry's config, the model's
pick and the tuned best (packed weights) and reports the ratios.
"""
import argparse
import csv
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CFG_KEYS = ("tile_n", "waves_k", "waves_n", "unroll", "split_k", "grid", "swap_ab", "x_lds",
            "quant_launch")
PARAM_NAMES = ("t0", "cu_bw", "latency", "hbm_bw", "slots", "sk_base", "sk_slot", "xl_stage",
               "wg_cost", "mfma", "reduce", "q_launch", "q_row_bw")


def collect(a):
    import bit_quantized_gemm_token_amd as w8
    from bit_quantized_gemm_token_amd.tune_sweep import default_shapes
    if a.shapes:
        shapes = [tuple(int(v) for v in s.split(",")) for s in a.shapes.split(";") if s]
    else:
        shapes = default_shapes()
    new = not os.path.exists(a.out)
    t0 = time.time()
    with open(a.out, "a", newline="") as f:
        wr = csv.writer(f)
        if new:
            wr.writerow(("fmt", "op", "layout", "M", "N", "K") + CFG_KEYS + ("us", "pred"))
        for op in a.ops.split(","):
            for fmt in a.formats.split(","):
                for packed in [w8.LAYOUTS[v] for v in a.layouts.split(",")]:
                    for (M, N, K) in shapes:
                        if a.time_budget_s and time.time() - t0 > a.time_budget_s:
                            print("[collect] time budget reached", flush=True)
                            return 0
                        ranked = w8.rank_configs(fmt, M, N, K, packed=packed, op=op)
                        cfgs = [c for _, c in ranked]
                        us = w8.profile_configs(fmt, M, N, K, cfgs, packed=packed, op=op,
                                                warmup=1, replays=a.replays,
                                                rotate_bytes=a.rotate_mib << 20)
                        layout = "packed" if packed else "row"
                        for (pred, c), u in zip(ranked, us):
                            d = c.as_dict()
                            wr.writerow((fmt, op, layout, M, N, K) + tuple(d[k] for k in CFG_KEYS)
                                        + ("" if u is None else f"{u:.4f}", f"{pred:.4f}"))
                        f.flush()
                        good = [u for u in us if u is not None]
                        print(f"[collect] {op} {fmt} {layout} {M}x{N}x{K}: {len(cfgs)} configs, "
                              f"best {min(good):.3f} us, model top-1 {us[0]} us", flush=True)
    return 0


# ------------------------------------------------------------------ model --
def _library():
    import bit_quantized_gemm_token_amd as w8
    return w8


def predict(p, fmt, op, M, N, K, c, layout=1):
    """The library model's prediction (us per call) with constants p."""
    w8 = _library()
    return w8.predict_us([(fmt, op, layout, M, N, K, c)], params=p)[0]


# the constants compiled into csrc/w8_model.cpp (kParams); the fit starts here
CURRENT = (1.6537, 56705.2, 1.0003, 4.54169e6, 2.608, 1.2018, 1.5197, 0.43, 0.1419, 0.0146,
           0.051, 0.225973, 20816.5)


def load(path):
    """Timed rows of a collect CSV as numpy arrays, grouped by problem, plus
    the rows packed once for the library's batch prediction."""
    import numpy as np
    w8 = _library()
    with open(path) as f:
        rows = [r for r in csv.DictReader(f) if r["us"]]
    d = {k: np.array([int(r[k]) for r in rows]) for k in ("M", "N", "K") + CFG_KEYS}
    d["fmt"] = np.array([r["fmt"] for r in rows])
    d["op"] = np.array([r["op"] for r in rows])
    d["us"] = np.array([float(r["us"]) for r in rows])
    key = np.array([f"{r['fmt']} {r['op']} {r['layout']} {r['M']}x{r['N']}x{r['K']}"
                    for r in rows])
    d["keys"], d["group"] = np.unique(key, return_inverse=True)
    d["batch"] = w8.PredictBatch([
        (r["fmt"], r["op"], w8.LAYOUTS[r["layout"]], int(r["M"]), int(r["N"]), int(r["K"]),
         {k: int(r[k]) for k in CFG_KEYS}) for r in rows])
    return d


def predict_arrays(p, d):
    """The library model's predictions for every row of load(), constants p."""
    return d["batch"].run(p)


def evaluate(p, d, top_n):
    """(geomean top-1 / best, geomean best-of-top-n / best, worst of the latter)."""
    import numpy as np
    pr = predict_arrays(p, d)
    l1 = ln = 0.0
    worst = 1.0
    for g in range(len(d["keys"])):
        ix = np.where(d["group"] == g)[0]
        best = d["us"][ix].min()
        o = ix[np.argsort(pr[ix], kind="stable")]
        l1 += math.log(d["us"][o[0]] / best)
        r = d["us"][o[:top_n]].min() / best
        ln += math.log(r)
        worst = max(worst, r)
    n = len(d["keys"])
    return math.exp(l1 / n), math.exp(ln / n), worst


def fit(a):
    """Nelder-Mead over the logs of the constants (all positive) from CURRENT,
    minimizing the ranking loss -- log(top-1 / best) plus half of
    log(best of the top 4 / best), averaged over problems -- plus 0.3 x the
    squared log error of the predictions, weighted by (best / us)^4 so the
    configs near the top of each problem count most."""
    import numpy as np
    from scipy.optimize import minimize
    d = load(a.csv)
    print(f"[fit] {len(d['keys'])} problems, {len(d['us'])} timed configs", flush=True)
    groups = [np.where(d["group"] == g)[0] for g in range(len(d["keys"]))]
    best = np.zeros(len(d["us"]))
    for ix in groups:
        best[ix] = d["us"][ix].min()
    wt = (best / d["us"]) ** 4
    free = [PARAM_NAMES.index(n) for n in (a.params.split(",") if a.params else PARAM_NAMES)]
    base = np.log(np.array(CURRENT, dtype=float))

    def unpack(x):
        v = base.copy()
        v[free] = x
        return np.exp(v)

    def objective(x):
        p = unpack(x)
        pr = predict_arrays(p, d)
        reg = np.sum(wt * (np.log(pr) - np.log(d["us"])) ** 2) / np.sum(wt)
        rank = 0.0
        for ix in groups:
            o = ix[np.argsort(pr[ix], kind="stable")[:4]]
            b = d["us"][ix].min()
            rank += math.log(d["us"][o[0]] / b) + 0.5 * math.log(d["us"][o].min() / b)
        return rank / len(groups) + 0.3 * reg

    x0 = base[free]
    print(f"[fit] start: objective {objective(x0):.4f}; top-1, top-{a.top_n}, worst: "
          f"{evaluate(unpack(x0), d, a.top_n)}", flush=True)
    res = minimize(objective, x0, method="Nelder-Mead",
                   options={"maxiter": a.maxiter, "xatol": 1e-4, "fatol": 1e-7})
    p = unpack(res.x)
    top1, topn, worst = evaluate(p, d, a.top_n)
    print(f"[fit] objective {res.fun:.4f} after {res.nit} iterations", flush=True)
    print(f"[fit] model top-1 vs measured best: geomean x{top1:.4f}; best of top-{a.top_n}: "
          f"geomean x{topn:.4f}, worst x{worst:.4f}", flush=True)
    print("constexpr ModelParams kParams = {" + ", ".join(f"{v:.6g}" for v in p) + "};",
          flush=True)
    return 0


def bucket_eval(a):
    """For shapes whose M has no table entry but whose floor(log2 M) bucket
    has one: time the bucket's config, the model's pick and the tuned best."""
    import bit_quantized_gemm_token_amd as w8
    shapes = [tuple(int(v) for v in s.split(",")) for s in a.shapes.split(";") if s]
    ratios = {"bucket": [], "model": []}
    for fmt in a.formats.split(","):
        for (M, N, K) in shapes:
            cfg_b, src = w8.resolve_config(fmt, M, N, K, packed=True)
            if src != 2:
                print(f"[bucket] {fmt} {M}x{N}x{K}: no bucket entry, skipped", flush=True)
                continue
            cfg_m = w8.model_config(fmt, M, N, K, packed=True)
            t_b, t_m = w8.profile_configs(fmt, M, N, K, [cfg_b, cfg_m], packed=True)
            best, st = w8.tune_shape(fmt, M, N, K, packed=True, insert=False)
            (t_t,) = w8.profile_configs(fmt, M, N, K, [best], packed=True)
            ratios["bucket"].append(t_b / t_t)
            ratios["model"].append(t_m / t_t)
            print(f"[bucket] {fmt} {M}x{N}x{K}: bucket {t_b:.3f} us, model {t_m:.3f} us, "
                  f"tuned {t_t:.3f} us", flush=True)
    for k, v in ratios.items():
        if v:
            print(f"[bucket] {k} / tuned: geomean x{math.exp(sum(map(math.log, v)) / len(v)):.4f}"
                  f", worst x{max(v):.4f} over {len(v)} shapes", flush=True)
    return 0


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("collect")
    c.add_argument("--out", required=True)
    c.add_argument("--formats", default="FP8_Dynamic,W8A8_INT8,Block_FP8")
    c.add_argument("--layouts", default="packed")
    c.add_argument("--ops", default="gemm")
    c.add_argument("--shapes", default=None)
    c.add_argument("--replays", type=int, default=3)
    c.add_argument("--rotate-mib", type=int, default=256)
    c.add_argument("--time-budget-s", type=float, default=0.0)
    f = sub.add_parser("fit")
    f.add_argument("csv")
    f.add_argument("--top-n", type=int, default=16)
    f.add_argument("--maxiter", type=int, default=3000)
    f.add_argument("--params", default=None,
                   help="comma-separated constants to fit (default: all)")
    b = sub.add_parser("bucket-eval")
    b.add_argument("--formats", default="FP8_Dynamic,W8A8_INT8,Block_FP8")
    b.add_argument("--shapes", required=True)
    a = p.parse_args(argv)
    if a.cmd == "collect":
        sys.path.insert(0, ROOT)
        return collect(a)
    if a.cmd == "bucket-eval":
        return bucket_eval(a)
    return fit(a)


if __name__ == "__main__":
    sys.exit(main())
