"""The fused linear layer (w8_linear: activation quantization inside the
GEMM) on the GPU.

- bf16 Y bit-identical to the two-launch path (w8_quantize_act, then
  w8_gemm_w8a8) with the same config: the fused staging uses the standalone
  quantizer's rules, so codes, scales and the MFMA sequence all match;
- Y within atol = rtol = 1e-2 of the oracle's fp64 result (oracle codes
  from the same bf16 activations);
- every fused-quantization instance at a ragged shape, whole tiles, split-K
  and stream-K; ragged K (masked tail step); all-zero rows; graph replay.
"""
import itertools

import numpy as np
import pytest
import torch

from tests.gpu_cases import DEV, Case, assert_bf16_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w8():
    import bit_quantized_gemm_token_amd as mod
    return mod


_cases = {}


def case(fmt, M, N, K):
    key = (fmt, M, N, K)
    if key not in _cases:
        _cases.clear()
        _cases[key] = Case(fmt, M, N, K)
    return _cases[key]


def two_launch(w8, cs, cfg, packed):
    xq, sx = w8.quantize_act(cs.fmt, cs.x)
    return w8.gemm_w8a8(cs.fmt, xq, sx, cs.weights(packed), cs.sw, cfg=cfg)


def fused(w8, cs, cfg, packed, x=None):
    return w8.linear(cs.fmt, cs.x if x is None else x, cs.weights(packed), cs.sw, cfg=cfg,
                     fused=True)


def same_bits(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


# (waves_k, waves_n) of the fused instances
FUSED_WAVES = ((1, 1), (2, 1), (4, 1), (1, 2), (1, 4), (1, 8))


@pytest.mark.parametrize("fmt", ["W8A8_INT8", "FP8_Dynamic", "Block_FP8"])
def test_every_fused_instance(w8, fmt):
    """Every fused-quantization instance (tile_n x waves x unroll x swap_ab x
    layout) at M = 17 (two 16-row blocks of M), with whole tiles, split-K and
    stream-K, against the two-launch path bit for bit."""
    M, N, K = 17, 200, 1280
    cs = case(fmt, M, N, K)
    n = 0
    for tn, (wk, wn), u, swap, (s, grid), packed in itertools.product(
            (16, 32, 64), FUSED_WAVES, (1, 2, 4), (0, 1), ((1, 0), (4, 0), (1, 3)), (False, True)):
        if (tn // 16) * u > 4 or (grid and (tn != 16 or u > 2)):
            continue
        cfg = w8.Config.make(tile_n=tn, waves_k=wk, waves_n=wn, unroll=u, split_k=s, grid=grid,
                             swap_ab=swap, x_lds=1)
        y1 = fused(w8, cs, cfg, packed)
        y2 = two_launch(w8, cs, cfg, packed)
        torch.cuda.synchronize()
        assert same_bits(y1, y2), f"{fmt} {cfg} packed={packed}: fused != two-launch"
        n += 1
    assert n == (6 * 6 * 2 * 2 + 2 * 6 * 2) * 2
    assert_bf16_close(y1, cs.Y, f"fused {fmt}")


@pytest.mark.parametrize("fmt,M,N,K", [
    ("W8A8_INT8", 1, 16, 16), ("W8A8_INT8", 5, 200, 208), ("W8A8_INT8", 32, 1000, 1040),
    ("FP8_Dynamic", 1, 16, 16), ("FP8_Dynamic", 31, 77, 336), ("FP8_Dynamic", 32, 1000, 1040),
    ("Block_FP8", 1, 16, 128), ("Block_FP8", 20, 130, 256), ("Block_FP8", 32, 1000, 1024)])
def test_fused_ragged_shapes(w8, fmt, M, N, K):
    """Ragged M, N and K (the masked tail K-step is quantized in the stage),
    default and explicit configs, both weight layouts, against the oracle and
    the two-launch path."""
    cs = case(fmt, M, N, K)
    for packed in (False, True):
        for cfg in (None, w8.Config.make(tile_n=32, waves_k=2, unroll=2, split_k=2, x_lds=1),
                    w8.Config.make(tile_n=16, waves_k=1, waves_n=4, unroll=1, swap_ab=1,
                                   x_lds=1)):
            y = fused(w8, cs, cfg, packed)
            torch.cuda.synchronize()
            assert_bf16_close(y, cs.Y, f"fused ragged {fmt} {cfg} packed={packed}")
            if cfg is not None:
                assert same_bits(y, two_launch(w8, cs, cfg, packed)), f"{fmt} {cfg}"


@pytest.mark.parametrize("fmt,M", [("W8A8_INT8", 1), ("FP8_Dynamic", 8), ("Block_FP8", 32),
                                   ("FP8_Dynamic", 32)])
def test_fused_large(w8, fmt, M):
    """4608 x 7168 (56 or 112 K-steps): per-token row scales over the whole
    K, split-K and stream-K grids, against the oracle and the two-launch
    path."""
    cs = case(fmt, M, 4608, 7168)
    for cfg in (w8.Config.make(tile_n=16, waves_k=1, waves_n=8, unroll=1, split_k=4, x_lds=1),
                w8.Config.make(tile_n=16, waves_k=4, unroll=2, split_k=8, x_lds=1, swap_ab=1),
                w8.Config.make(tile_n=16, waves_k=1, waves_n=2, unroll=1, grid=512, x_lds=1)):
        y = fused(w8, cs, cfg, True)
        torch.cuda.synchronize()
        assert_bf16_close(y, cs.Y, f"fused large {fmt} M={M} {cfg}")
        assert same_bits(y, two_launch(w8, cs, cfg, True)), f"{fmt} M={M} {cfg}"


@pytest.mark.parametrize("fmt", ["W8A8_INT8", "FP8_Dynamic", "Block_FP8"])
def test_fused_zero_rows(w8, fmt):
    """An all-zero row (and, for Block_FP8, all-zero groups) takes scale 1 and
    codes 0 in the stage, like the standalone quantizer."""
    cs = case(fmt, 8, 272, 640 if fmt != "Block_FP8" else 768)
    x = cs.x.clone()
    x[3] = 0
    x[5, :128] = 0
    cfg = w8.Config.make(tile_n=16, waves_k=2, unroll=2, split_k=2, x_lds=1)
    y1 = fused(w8, cs, cfg, True, x=x)
    xq, sx = w8.quantize_act(fmt, x)
    y2 = w8.gemm_w8a8(fmt, xq, sx, cs.weights(True), cs.sw, cfg=cfg)
    torch.cuda.synchronize()
    assert same_bits(y1, y2)
    assert (y1[3].float() == 0).all()


@pytest.mark.parametrize("fmt", ["W8A8_INT8", "FP8_Dynamic", "Block_FP8"])
def test_fused_extreme_magnitudes(w8, fmt):
    """Rows scaled by 2^-124 .. 2^120 with subnormal entries and negative
    zeros: the staged codes and scales equal the standalone quantizer's (its
    own parity with the oracle on these rows is a quantizer test), so Y is
    bit-identical to the two-launch path."""
    import synthetic
    from tests.gpu_cases import to_bf16_tensor
    M, N, K = 14, 272, 1024
    cs = case(fmt, M, N, K)
    x = to_bf16_tensor(synthetic.activations_extreme(fmt, M, K))
    for cfg in (w8.Config.make(tile_n=16, waves_k=2, unroll=2, split_k=2, x_lds=1),
                w8.Config.make(tile_n=32, waves_k=1, waves_n=4, unroll=1, x_lds=1)):
        y1 = fused(w8, cs, cfg, True, x=x)
        xq, sx = w8.quantize_act(fmt, x)
        y2 = w8.gemm_w8a8(fmt, xq, sx, cs.weights(True), cs.sw, cfg=cfg)
        torch.cuda.synchronize()
        assert same_bits(y1, y2), f"{fmt} {cfg}"


def test_fused_graph_replay(w8):
    cs = case("FP8_Dynamic", 4, 4096, 4096)
    cfg = w8.Config.make(tile_n=16, waves_k=4, unroll=2, split_k=8, x_lds=1)
    wp = cs.packed()
    ws = w8.Workspace(DEV, w8.workspace_size("FP8_Dynamic", 4, 4096, 4096, cfg, packed=True,
                                             op="linear"))
    eager = w8.linear("FP8_Dynamic", cs.x, wp, cs.sw, cfg=cfg, workspace=ws, fused=True).clone()
    x_static = cs.x.clone()
    y_static = torch.empty_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        w8.linear("FP8_Dynamic", x_static, wp, cs.sw, cfg=cfg, y=y_static, workspace=ws,
                  fused=True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w8.linear("FP8_Dynamic", x_static, wp, cs.sw, cfg=cfg, y=y_static, workspace=ws,
                  fused=True)
    for i in range(4):
        y_static.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert same_bits(y_static, eager), f"replay {i}"
        junk = torch.randn(512, 512, device=DEV) @ torch.randn(512, 512, device=DEV)
        del junk
    assert_bf16_close(y_static, cs.Y, "fused graph replay")


QL_CFGS = (dict(tile_n=16, waves_k=4, unroll=2, split_k=1),
           dict(tile_n=32, waves_k=16, unroll=1, split_k=8),
           dict(tile_n=16, waves_k=1, waves_n=8, unroll=1, split_k=4, x_lds=1),
           dict(tile_n=64, waves_k=2, unroll=1, split_k=1, swap_ab=1),
           dict(tile_n=16, waves_k=2, unroll=2, grid=300))


@pytest.mark.parametrize("fmt,M,N,K", [("W8A8_INT8", 7, 300, 1040), ("FP8_Dynamic", 32, 1000, 2048),
                                       ("Block_FP8", 17, 520, 1152), ("FP8_Dynamic", 1, 64, 16)])
def test_quant_launch(w8, fmt, M, N, K):
    """quant_launch = 1: w8_linear quantizes in a launch of its own into the
    workspace, then runs the GEMM with the config's GEMM part: Y bit for bit
    the two-call path's, both layouts, split-K, stream-K and x_lds 0/1."""
    cs = case(fmt, M, N, K)
    for kw in QL_CFGS:
        if kw.get("grid", 0) > (N + 15) // 16 * ((K + 127) // 128):
            continue
        g = w8.Config.make(**kw)
        q = w8.Config.make(quant_launch=1, **kw)
        for packed in (False, True):
            y1 = fused(w8, cs, q, packed)
            y2 = two_launch(w8, cs, g, packed)
            torch.cuda.synchronize()
            assert same_bits(y1, y2), f"{fmt} {kw} packed={packed}"
    assert_bf16_close(y1, cs.Y, f"quant_launch {fmt}")


def test_quant_launch_shares_workspace_with_split_k(w8):
    """A workspace used by a quant_launch call and by split-K GEMMs in turn:
    the codes never land on the arrival counters, so every call stays right,
    also under graph replay."""
    fmt, M, N, K = "FP8_Dynamic", 8, 4096, 4096
    cs = case(fmt, M, N, K)
    wp = cs.packed()
    q = w8.Config.make(tile_n=16, waves_k=4, unroll=2, quant_launch=1)            # no split
    sk = w8.Config.make(tile_n=16, waves_k=4, unroll=2, split_k=16)
    qsk = w8.Config.make(tile_n=16, waves_k=4, unroll=2, split_k=16, quant_launch=1)
    ws = w8.Workspace(DEV, max(w8.workspace_size(fmt, M, N, K, c, packed=True, op=op)
                               for c, op in ((q, "linear"), (sk, "gemm"), (qsk, "linear"))))
    xq, sx = w8.quantize_act(fmt, cs.x)
    ref = w8.gemm_w8a8(fmt, xq, sx, wp, cs.sw, cfg=sk, workspace=ws).clone()
    x_static = cs.x.clone()
    y = [torch.empty_like(ref) for _ in range(3)]

    def calls():
        w8.linear(fmt, x_static, wp, cs.sw, cfg=q, y=y[0], workspace=ws, fused=True)
        w8.gemm_w8a8(fmt, xq, sx, wp, cs.sw, cfg=sk, y=y[1], workspace=ws)
        w8.linear(fmt, x_static, wp, cs.sw, cfg=qsk, y=y[2], workspace=ws, fused=True)

    for _ in range(3):
        calls()
        torch.cuda.synchronize()
        for t in y:
            assert same_bits(t, ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for i in range(4):
        for t in y:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for t in y:
            assert same_bits(t, ref), f"replay {i}"
    assert_bf16_close(ref, cs.Y, "shared workspace")


def test_fused_rejects_gemm_config(w8):
    """A GEMM config (no x_lds) is no per-token linear config: refused
    before any launch."""
    cs = case("W8A8_INT8", 4, 64, 256)
    with pytest.raises(w8.W8Error, match="x_lds"):
        fused(w8, cs, w8.Config.make(waves_k=4), False)


@pytest.mark.parametrize("M", [17, 3])
def test_every_block_fp8_k_loop_instance(w8, M):
    """Block_FP8 linear quantizing in the K loop (x_lds = 0: each wave
    quantizes the 1x128 groups it loads): every instance (tile_n x waves_k x
    swap_ab x layout) with whole tiles, split-K and stream-K, at
    M = 17 (two row blocks) and M = 3, bit-identical to the two-launch path
    with the same config, and within the bar of the oracle."""
    fmt, N, K = "Block_FP8", 200, 1280
    cs = case(fmt, M, N, K)
    n = 0
    for tn, wk, swap, (s, grid), packed in itertools.product(
            (16, 32), (2, 4, 8), (0, 1), ((1, 0), (4, 0), (1, 3)), (False, True)):
        if grid and tn != 16:
            continue
        cfg = w8.Config.make(tile_n=tn, waves_k=wk, waves_n=1, unroll=1, split_k=s, grid=grid,
                             swap_ab=swap, x_lds=0)
        y1 = fused(w8, cs, cfg, packed)
        y2 = two_launch(w8, cs, cfg, packed)
        torch.cuda.synchronize()
        assert same_bits(y1, y2), f"{fmt} {cfg} packed={packed}: K-loop != two-launch"
        n += 1
    assert n == (2 * 3 * 2 * 2 + 3 * 2) * 2
    assert_bf16_close(y1, cs.Y, f"K-loop fused {fmt} M={M}")


def test_block_fp8_k_loop_large_and_extreme(w8):
    """The K-loop quantization at 4608 x 7168 (M = 1, 8, 32) and on rows of
    extreme magnitude (subnormal, -0, 2^120 scales): bit-identical to the
    two-launch path."""
    import synthetic
    from tests.gpu_cases import to_bf16_tensor
    fmt = "Block_FP8"
    for M in (1, 8, 32):
        cs = case(fmt, M, 4608, 7168)
        for cfg in (w8.Config.make(tile_n=16, waves_k=4, unroll=1, split_k=1),
                    w8.Config.make(tile_n=32, waves_k=2, unroll=1, split_k=4, swap_ab=1)):
            y1 = fused(w8, cs, cfg, True)
            y2 = two_launch(w8, cs, cfg, True)
            torch.cuda.synchronize()
            assert same_bits(y1, y2), f"M={M} {cfg}"
        assert_bf16_close(y1, cs.Y, f"K-loop fused 4608x7168 M={M}")
    cs = case(fmt, 21, 256, 1024)
    x = to_bf16_tensor(synthetic.activations_extreme(fmt, 21, 1024))
    cfg = w8.Config.make(tile_n=16, waves_k=8, unroll=1, split_k=2)
    xq, sx = w8.quantize_act(fmt, x)
    ref = w8.gemm_w8a8(fmt, xq, sx, cs.weights(True), cs.sw, cfg=cfg)
    y = fused(w8, cs, cfg, True, x=x)
    torch.cuda.synchronize()
    assert same_bits(y, ref)
