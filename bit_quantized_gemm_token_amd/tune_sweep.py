"""Ahead-of-time tuning of a list of shapes into a config table file.

    python -m bit_quantized_gemm_token_amd.tune_sweep --out TABLE [--formats ...]
           [--ops gemm,linear] [--layouts row,packed,seg2,seg4,seg8]
           [--shapes M,N,K;M,N,K...]
           [--no-resume] [--retune] [--max-split-k 256] [--top-n N]
           [--moe-shapes E,topk,T,N,K;...]

Default shapes: the 24-shape M <= 32 sweep of synthetic.SWEEP plus the shapes
the tests and benchmarks name (N=K=4096 at M in {1, 4, 16, 32}; N=4608,
K=7168 at M in {1, 8, 32}; N=512, K=7168 at M in {1, 2, 4, 8, 16, 32};
16 x 896 x 1024).  Ops "moe" and "moe_linear" tune the MoE grouped GEMM on
quantized tokens and on bf16 tokens with the quantization fused (moe_tune) on
their own shapes, packed layout only: by default the 128-expert top-8 layers
of synthetic.MOE_SHAPES at the token counts synthetic.MOE_TOKENS.  The
K-segmented layouts (seg2, seg4, seg8: 16/T-row blocks) are tuned only for
the M one launch covers, M <= 2 x 16/T (beyond it a call runs as several
launches and the plain packed layout is the better one), unless --all-m.

Tuning is the expensive offline step the page describes (ai-radar.it,
"Helion nel backend vLLM", paragraph 6: ahead-of-time tuning can take hours
and its config files must be managed), so this tool is resumable: entries
already in TABLE for this arch and ABI are kept and skipped, and the table is
rewritten (write-then-rename, by the library) after every tuned shape.
"""
import argparse
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

EXTRA_SHAPES = ((1, 4096, 4096), (4, 4096, 4096), (16, 4096, 4096), (32, 4096, 4096),
                (1, 4608, 7168), (8, 4608, 7168), (32, 4608, 7168),
                (1, 512, 7168), (2, 512, 7168), (4, 512, 7168), (8, 512, 7168),
                (16, 512, 7168), (32, 512, 7168), (16, 896, 1024))


def default_shapes():
    sys.path.insert(0, ROOT)
    from synthetic import SWEEP
    out = []
    for s in tuple(SWEEP) + EXTRA_SHAPES:
        if s not in out:
            out.append(s)
    return out


def default_moe_shapes():
    sys.path.insert(0, ROOT)
    import synthetic
    return [(synthetic.MOE_E, synthetic.MOE_TOPK, T, N, K)
            for _, N, K in synthetic.MOE_SHAPES for T in synthetic.MOE_TOKENS]


def main(argv=None):
    import bit_quantized_gemm_token_amd as w8
    p = argparse.ArgumentParser()
    p.add_argument("--out", required=True)
    p.add_argument("--formats", default="FP8_Dynamic,W8A8_INT8,Block_FP8")
    p.add_argument("--layouts", default="row,packed")
    p.add_argument("--all-m", action="store_true",
                   help="tune the K-segmented layouts at every M, not only M <= 32/T")
    p.add_argument("--ops", default="gemm", help="comma list of gemm, linear, moe, moe_linear")
    p.add_argument("--moe-shapes", default=None, help="E,topk,T,N,K;... for the MoE ops")
    p.add_argument("--shapes", default=None)
    p.add_argument("--no-resume", action="store_true")
    p.add_argument("--retune", action="store_true",
                   help="tune the selected ops, layouts and shapes again even where the table "
                        "has an entry (the other entries are kept)")
    p.add_argument("--max-split-k", type=int, default=w8.MAX_SPLIT_K)
    p.add_argument("--rotate-mib", type=int, default=512)
    p.add_argument("--replays", type=int, default=5)
    p.add_argument("--stream-k", action="store_true", help="also try stream-K grids")
    p.add_argument("--top-n", type=int, default=0,
                   help="time only the cost model's top N candidates (0 = all)")
    p.add_argument("--time-budget-s", type=float, default=0.0,
                   help="stop starting new shapes after this many seconds (0 = no limit)")
    a = p.parse_args(argv)
    if a.shapes:
        shapes = [tuple(int(v) for v in s.split(",")) for s in a.shapes.split(";") if s]
    else:
        shapes = default_shapes()
    w8.clear_config_table()
    if not a.no_resume and os.path.exists(a.out):
        w8.load_config_table(a.out)
    t0 = time.time()
    done = skipped = 0
    layouts = [w8.LAYOUTS[v] for v in a.layouts.split(",")]
    if a.moe_shapes:
        moe_shapes = [tuple(int(v) for v in s.split(",")) for s in a.moe_shapes.split(";") if s]
    else:
        moe_shapes = default_moe_shapes()
    jobs = []
    for op in a.ops.split(","):
        for fmt in a.formats.split(","):
            if op in ("moe", "moe_linear"):  # (T, N, K) keys the entry; E, topk: routing
                jobs += [(op, fmt, (T, N, K), True, (E, k)) for E, k, T, N, K in moe_shapes]
            else:
                jobs += [(op, fmt, s, packed, None) for s in shapes for packed in layouts
                         if a.all_m or packed < 2 or s[0] <= 32 // packed]
    for op, fmt, (M, N, K), packed, moe in jobs:
        if not a.retune and w8.lookup_config(fmt, M, N, K, packed=packed, op=op) is not None:
            skipped += 1
            continue
        if a.time_budget_s and time.time() - t0 > a.time_budget_s:
            print(f"[tune] time budget reached after {done} shapes", flush=True)
            print(f"[tune] tuned {done}, kept {skipped}, table {a.out}", flush=True)
            return 0
        if moe:
            best, st = w8.moe_tune(fmt, moe[0], M, N, K, moe[1], rotate_bytes=a.rotate_mib << 20,
                                   replays=a.replays, max_split_k=a.max_split_k, insert=True,
                                   packed=True, fused=op == "moe_linear")
        else:
            try:
                best, st = w8.tune_shape(fmt, M, N, K, rotate_bytes=a.rotate_mib << 20,
                                         replays=a.replays, max_split_k=a.max_split_k,
                                         insert=True, packed=packed, stream_k=a.stream_k, op=op,
                                         top_n=a.top_n)
            except w8.W8Error as e:          # e.g. no candidate of this layout fits the shape
                print(f"[tune] {op} {fmt} {w8.LAYOUT_NAMES[int(packed)]} {M}x{N}x{K}: "
                      f"not tuned ({e})", flush=True)
                continue
        w8.save_config_table(a.out)
        done += 1
        print(f"[tune] {op} {fmt} {w8.LAYOUT_NAMES[int(packed)]} {M}x{N}x{K}: {best} "
              f"{st['best_us_bank2']:.3f} us "
              f"({st['best_gbps']:.0f} GB/s; default {st['default_us_bank2']:.3f} us; "
              f"{st['validated']}/{st['candidates']} validated; {st['tune_seconds']:.1f} s)",
              flush=True)
    print(f"[tune] tuned {done}, kept {skipped}, table {a.out}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
