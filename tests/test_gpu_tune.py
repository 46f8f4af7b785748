"""The ahead-of-time tuner on the GPU: its winner is a valid, validated config
that is no slower than the default on the second timing bank, it lands in the
config table, survives a save/load round trip and is what the GEMM resolves;
an injected validation failure removes a candidate."""
import numpy as np
import pytest
import torch

from tests.gpu_cases import Case, assert_bf16_close

pytestmark = pytest.mark.gpu

SMALL = dict(warmup=1, replays=3, bank2_top=3, rotate_bytes=64 << 20, max_split_k=8)


@pytest.fixture(scope="module")
def w8():
    import bit_quantized_gemm_token_amd as mod
    return mod


@pytest.fixture(autouse=True)
def _restore_table(w8):
    yield
    w8.clear_config_table()
    w8.load_default_table()


@pytest.mark.parametrize("fmt,M,N,K,packed,stream_k,op", [
    ("W8A8_INT8", 16, 896, 1024, False, False, "gemm"),
    ("FP8_Dynamic", 4, 512, 2048, True, True, "gemm"),
    ("Block_FP8", 8, 512, 1024, False, False, "gemm"),
    ("Block_FP8", 32, 512, 1024, True, False, "gemm"),
    ("FP8_Dynamic", 8, 512, 2048, True, False, "linear"),
    ("W8A8_INT8", 1, 896, 1040, False, False, "linear")])
def test_tune_shape(w8, fmt, M, N, K, packed, stream_k, op, tmp_path):
    print(f"[tune] {op} {fmt} M={M} N={N} K={K} packed={packed} stream_k={stream_k}", flush=True)
    w8.clear_config_table()
    best, st = w8.tune_shape(fmt, M, N, K, packed=packed, stream_k=stream_k, op=op, **SMALL)
    print(f"[tune] best {best} stats {st}", flush=True)
    w8.validate_config(fmt, M, N, K, best, op=op)
    assert st["candidates"] > 10 and st["validated"] == st["candidates"] and st["rejected"] == 0
    assert st["best_us_bank2"] > 0 and st["best_gbps"] > 0
    # the default competes on bank 2, so the winner is never slower than it
    assert 0 < st["best_us_bank2"] <= st["default_us_bank2"]
    assert 0 < st["best_us_bank2_min"] <= st["best_us_bank2"] <= st["best_us_bank2_p90"]
    assert w8.lookup_config(fmt, M, N, K, packed=packed, op=op) == best
    assert w8.lookup_config(fmt, M, N, K, packed=not packed, op=op) is None
    cfg, hit = w8.resolve_config(fmt, M, N, K, packed=packed, op=op)
    assert hit and cfg == best
    p = tmp_path / "tuned.tbl"
    w8.save_config_table(str(p))
    w8.clear_config_table()
    w8.load_config_table(str(p))
    assert w8.lookup_config(fmt, M, N, K, packed=packed, op=op) == best
    cs = Case(fmt, M, N, K)
    # resolves the tuned entry
    y = w8.linear(fmt, cs.x, cs.weights(packed), cs.sw, fused=(op == "linear"))
    torch.cuda.synchronize()
    assert_bf16_close(y, cs.Y, f"tuned {op} {fmt}")


def test_tune_linear_picks_quant_launch_where_it_wins(w8):
    """Per-token FP8 at M = 32, K = 7168: every workgroup of the fused kernel
    reads all 32 x 7168 bf16 activations for the row maxima, so a quantize
    launch of its own plus the tuned GEMM is about twice as fast; the linear
    tuner, run after the GEMM's, must pick it, and w8_linear must run it."""
    fmt, M, N, K = "FP8_Dynamic", 32, 512, 7168
    w8.clear_config_table()
    g, _ = w8.tune_shape(fmt, M, N, K, packed=True, op="gemm", **SMALL)
    best, st = w8.tune_shape(fmt, M, N, K, packed=True, op="linear", **SMALL)
    print(f"[tune] linear best {best} stats {st}", flush=True)
    assert best.quant_launch == 1
    gq = w8.Config.make(**{k: v for k, v in g.as_dict().items() if k != "quant_launch"},
                        quant_launch=1)
    assert best in (gq, w8.Config.make(**{k: v for k, v in w8.default_config(
        fmt, M, N, K).as_dict().items() if k != "quant_launch"}, quant_launch=1))
    cs = Case(fmt, M, N, K)
    y = w8.linear(fmt, cs.x, cs.weights(True), cs.sw, fused=True)   # table entry
    torch.cuda.synchronize()
    assert_bf16_close(y, cs.Y, "tuned linear, quant_launch")


def test_tune_rejects_injected_failure(w8):
    w8.clear_config_table()
    best, st = w8.tune_shape("W8A8_INT8", 4, 256, 512, insert=False, fail_candidate=0, **SMALL)
    assert st["rejected"] == 1 and st["validated"] == st["candidates"] - 1
    assert st["best_index"] != 0
    assert w8.config_table_size() == 0                # insert=False


@pytest.mark.parametrize("fmt,M,N,K,op", [("FP8_Dynamic", 8, 1792, 5120, "gemm"),
                                          ("W8A8_INT8", 32, 512, 7168, "gemm"),
                                          ("Block_FP8", 4, 896, 1024, "linear")])
def test_tune_top_n(w8, fmt, M, N, K, op):
    """Tuning only the cost model's top 16 candidates: 16 candidates are
    timed, the winner is one of them (or the default, which competes on bank
    2), it is valid and its output is within the bar of the oracle."""
    print(f"[tune top-16] {op} {fmt} M={M} N={N} K={K}", flush=True)
    w8.clear_config_table()
    top = [c for _, c in w8.rank_configs(fmt, M, N, K, packed=True, op=op,
                                         max_split_k=SMALL["max_split_k"])[:16]]
    best, st = w8.tune_shape(fmt, M, N, K, packed=True, op=op, top_n=16, **SMALL)
    print(f"[tune top-16] best {best} stats {st}", flush=True)
    assert st["candidates"] == len(top) == 16 and st["validated"] == 16
    assert best in top + [w8.default_config(fmt, M, N, K, op=op)]
    assert st["best_us_bank2"] <= st["default_us_bank2"]
    w8.validate_config(fmt, M, N, K, best, op=op)
    cs = Case(fmt, M, N, K)
    y = w8.linear(fmt, cs.x, cs.weights(True), cs.sw, cfg=best, fused=(op == "linear"))
    torch.cuda.synchronize()
    assert_bf16_close(y, cs.Y, f"top-16 tuned {op} {fmt}")


def test_bucket_resolved_configs(w8):
    """Token counts with no table entry of their own (3, 6, 12, 24) on the
    sweep's (N, K): where the shipped table has an entry of the same
    floor(log2 M) bucket, the library resolves it, and the GEMM with that
    config matches the oracle."""
    import synthetic
    pairs = sorted({(N, K) for _, N, K in synthetic.SWEEP})
    hits = 0
    for fmt in ("FP8_Dynamic", "W8A8_INT8", "Block_FP8"):
        for N, K in pairs:
            for M in (3, 6, 12, 24):
                cfg, hit = w8.resolve_config(fmt, M, N, K, packed=True)
                if hit != 2:
                    continue
                hits += 1
                print(f"[bucket] {fmt} M={M} N={N} K={K} {cfg}", flush=True)
                cs = Case(fmt, M, N, K)
                y = w8.linear(fmt, cs.x, cs.weights(True), cs.sw)      # cfg=None: resolved
                torch.cuda.synchronize()
                assert_bf16_close(y, cs.Y, f"bucket {fmt} M={M} {N}x{K}")
    assert hits >= 30


def test_tuners_refuse_under_capture(w8):
    """The tuners allocate and synchronize: while the caller's stream is being
    captured they return W8_E_INVALID and do nothing, and the capture itself
    stays valid (a GEMM captured beside it replays correctly)."""
    cs = Case("FP8_Dynamic", 4, 256, 512)
    xq, sx = cs.gpu_act()
    y = torch.empty((4, 256), dtype=torch.bfloat16, device=xq.device)
    ws = w8.Workspace(xq.device, 1 << 22)
    w8.gemm_w8a8("FP8_Dynamic", xq, sx, cs.wq, cs.sw, y=y, workspace=ws)
    torch.cuda.synchronize()
    ref = y.clone()
    g = torch.cuda.CUDAGraph()
    errs = []
    with torch.cuda.graph(g):
        for call in (lambda: w8.tune_shape("FP8_Dynamic", 4, 256, 512, **SMALL),
                     lambda: w8.profile_configs("FP8_Dynamic", 4, 256, 512,
                                                [w8.default_config("FP8_Dynamic", 4, 256, 512)]),
                     lambda: w8.moe_tune("FP8_Dynamic", 8, 4, 256, 512, 2, **SMALL)):
            try:
                call()
                errs.append(None)
            except w8.W8Error as e:
                errs.append(e.status)
        w8.gemm_w8a8("FP8_Dynamic", xq, sx, cs.wq, cs.sw, y=y, workspace=ws)
    assert errs == [1, 1, 1]                      # W8_E_INVALID, nothing done
    y.zero_()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
