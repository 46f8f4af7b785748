"""The K-segmented weight layouts (2, 4, 8 K-steps per MFMA) against the
oracle.

- the packed bytes equal a numpy rendering of the layout's definition;
- every compiled instance (blocks per wave, K-waves, unroll, Swap-AB, one
  or two token groups), whole tiles and split-K: int32 accumulators
  bit-identical to the oracle's exact sums (and to the row-major layout's),
  fp32 accumulators within the summation bound;
- M beyond one launch (two token groups of 16/T rows) runs as consecutive
  launches, ragged N, K and spans reaching past K are masked;
- the whole path (quantize + GEMM, and the linear op with a quantize
  launch or with the quantization fused into the kernel, bit-identical to
  the two calls) within rtol = atol = 1e-2 of the fp64 oracle, also under
  graph replay.
"""
import itertools

import numpy as np
import pytest
import torch

from tests.gpu_cases import DEV, Case, assert_bf16_close, u8

pytestmark = pytest.mark.gpu

LAYOUTS = (2, 4, 8)


@pytest.fixture(scope="module")
def w8():
    import bit_quantized_gemm_token_amd as mod
    return mod


def C(w8, **kw):
    return w8.Config.make(**kw)


_cases = {}


def case(fmt, M, N, K):
    key = (fmt, M, N, K)
    if key not in _cases:
        _cases.clear()
        _cases[key] = Case(fmt, M, N, K)
    return _cases[key]


def packed(w8, cs, T):
    return cs.memo(("seg", T), lambda: w8.pack_weight(cs.fmt, cs.wq, layout=T))


def acc_check(w8, cs, xq, sx, wq, cfg, what):
    acc = w8.gemm_w8a8_acc(cs.fmt, xq, sx, wq, cs.sw, cfg=cfg)
    torch.cuda.synchronize()
    got = acc.cpu().numpy()
    ref = cs.acc_ref()
    if cs.fmt == "W8A8_INT8":
        assert np.array_equal(got.astype(np.int64), ref), f"{what}: int32 accumulators differ"
    else:
        bad = np.argwhere(np.abs(got - ref) > cs.acc_bound())
        assert bad.size == 0, f"{what}: {len(bad)} fp32 accumulators off, first {bad[:3]}"
    return got


def _seg_reference(codes, kstep, T):
    """Layout T written out with numpy from its definition: fragment (block
    of R = 16/T rows, span of T K-steps) of 16 x kstep bytes; in it, load
    instruction jj at jj*1024 and lane l's 16 bytes at 16*l hold row
    R*nb + (l%16)%R, K-step T*sp + (l%16)//R, bytes 64*jj + 16*(l//16) .. +16;
    rows past N and bytes past K are zero."""
    R = 16 // T
    N, K = codes.shape
    nblk = -(-N // R)
    spans = -(-(-(-K // kstep)) // T)
    padded = np.zeros((nblk * R, spans * T * kstep), np.uint8)
    padded[:N, :K] = codes
    out = np.zeros((nblk, spans, kstep // 64, 64, 16), np.uint8)
    for l in range(64):
        p, g = l % 16, l // 16
        r, t = p % R, p // R
        for jj in range(kstep // 64):
            cols = ((np.arange(spans) * T + t) * kstep)[:, None] + 64 * jj + 16 * g + np.arange(16)
            out[:, :, jj, l, :] = padded[np.arange(nblk) * R + r][:, cols]
    return out.reshape(-1)


@pytest.mark.parametrize("fmt,N,K", [("W8A8_INT8", 200, 208), ("FP8_Dynamic", 37, 400),
                                     ("Block_FP8", 130, 384), ("FP8_Dynamic", 512, 7168),
                                     ("W8A8_INT8", 33, 1040)])
@pytest.mark.parametrize("T", LAYOUTS)
def test_pack_segmented_layout(w8, fmt, N, K, T):
    rng = np.random.default_rng(N + K + T)
    codes = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    got = w8.pack_weight(fmt, torch.from_numpy(codes).to(DEV), layout=T).data.cpu().numpy()
    kstep = 64 if fmt == "W8A8_INT8" else 128
    assert got.size == w8.packed_weight_size(fmt, N, K, T)
    assert np.array_equal(got, _seg_reference(codes, kstep, T))


# (blocks per wave, waves_k, unroll) of the compiled K-segmented instances
SEG_TILES = ((1, 1, 1), (1, 1, 2), (1, 1, 4), (1, 2, 1), (1, 2, 2), (1, 4, 1), (1, 4, 2),
             (1, 8, 1), (1, 16, 1), (2, 1, 1), (2, 1, 2), (2, 2, 1), (2, 4, 1))


@pytest.mark.parametrize("fmt", ["W8A8_INT8", "FP8_Dynamic", "Block_FP8"])
@pytest.mark.parametrize("T", LAYOUTS)
def test_every_segmented_instance(w8, fmt, T):
    """Every compiled instance of layout T at a ragged shape: N = 193 leaves
    a partial last block of rows, K a ragged K-step (per-token formats) and
    a last span reaching past K; M = 1 (one partial token group) and
    M = 16/T + 1 (two groups, the second partial); whole tiles and split-K 4."""
    R = 16 // T
    N, K = 193, (1152 if fmt == "Block_FP8" else 1040)
    for M in (1, R + 1):
        cs = case(fmt, M, N, K)
        xq, sx = cs.gpu_act()
        wp = packed(w8, cs, T)
        n = 0
        for (nb, wk, u), swap, s in itertools.product(SEG_TILES, (0, 1), (1, 4)):
            cfg = C(w8, tile_n=nb * R, waves_k=wk, unroll=u, split_k=s, swap_ab=swap)
            w8.validate_config(fmt, M, N, K, cfg, packed=T)
            acc_check(w8, cs, xq, sx, wp, cfg, f"{fmt} T={T} M={M} {cfg}")
            n += 1
        assert n == len(SEG_TILES) * 4


@pytest.mark.parametrize("fmt,M,N,K,T", [
    ("W8A8_INT8", 17, 200, 208, 8), ("FP8_Dynamic", 5, 37, 400, 4), ("FP8_Dynamic", 32, 1000, 1040, 8),
    ("Block_FP8", 9, 130, 384, 2), ("Block_FP8", 32, 512, 1024, 4), ("W8A8_INT8", 3, 16, 16, 8),
    ("FP8_Dynamic", 1, 16, 16, 2), ("Block_FP8", 1, 16, 128, 8)])
def test_segmented_ragged_and_chunked(w8, fmt, M, N, K, T):
    """Ragged M, N and K on the K-segmented layouts, with M up to 32 (several
    launches of 2 x 16/T token rows): the default config, the resolved one
    and explicit ones, accumulators and the whole path against the oracle;
    int8 accumulators equal the row-major layout's bit for bit."""
    cs = case(fmt, M, N, K)
    xq, sx = cs.gpu_act()
    assert np.array_equal(u8(xq), cs.xq_ref)
    R = 16 // T
    wp = packed(w8, cs, T)
    base = w8.gemm_w8a8_acc(fmt, xq, sx, cs.wq, cs.sw).cpu().numpy()
    for cfg in (None, w8.default_config(fmt, M, N, K, packed=T),
                C(w8, tile_n=R, waves_k=2, unroll=1, split_k=2, swap_ab=1),
                C(w8, tile_n=2 * R, waves_k=1, unroll=2, split_k=1, swap_ab=0)):
        try:
            if cfg is not None:
                w8.validate_config(fmt, M, N, K, cfg, packed=T)
        except w8.W8Error:
            continue
        got = acc_check(w8, cs, xq, sx, wp, cfg, f"{fmt} T={T} {cfg}")
        if fmt == "W8A8_INT8":
            assert np.array_equal(got, base)
        y = w8.gemm_w8a8(fmt, xq, sx, wp, cs.sw, cfg=cfg)
        assert_bf16_close(y, cs.Y, f"{fmt} T={T} {cfg}")
        lcfg = None if cfg is None else C(w8, **{**cfg.as_dict(), "quant_launch": 1})
        yl = w8.linear(fmt, cs.x, wp, cs.sw, cfg=lcfg, fused=True)
        torch.cuda.synchronize()
        if cfg is None:                        # the linear op's own resolved config
            assert_bf16_close(yl, cs.Y, f"{fmt} T={T} linear")
        else:                                  # quantize launch + this GEMM config
            assert torch.equal(yl.view(torch.int16), y.view(torch.int16)), f"linear {cfg}"


# (blocks per wave, waves_k, unroll) of the fused-quantization instances
SEG_FUSED = ((1, 1, 1), (1, 1, 2), (1, 2, 1), (1, 2, 2), (1, 4, 1), (2, 1, 1), (2, 2, 1))


@pytest.mark.parametrize("fmt", ["W8A8_INT8", "FP8_Dynamic", "Block_FP8"])
@pytest.mark.parametrize("T", LAYOUTS)
def test_segmented_fused_linear(w8, fmt, T):
    """The linear op with the quantization fused (x_lds 1) on layout T: every
    fused instance, whole tiles and split-K, at the ragged shape of
    test_every_segmented_instance with M = 1 and M = 16/T + 1, and at M = 2 x
    16/T + 3 (two launches plus a third of 3 rows); Y bit-identical to
    quantize_act + gemm_w8a8 with the same tiles (x_lds 0), within the bar
    of the oracle; rows of extreme magnitude too."""
    import synthetic
    from tests.gpu_cases import to_bf16_tensor
    R = 16 // T
    N, K = 193, (1152 if fmt == "Block_FP8" else 1040)
    for M in (1, R + 1, 2 * R + 3):
        cs = case(fmt, M, N, K)
        wp = packed(w8, cs, T)
        n = 0
        for (nb, wk, u), swap, s in itertools.product(SEG_FUSED, (0, 1), (1, 4)):
            if M > R + 1 and (nb, wk, u, s) != (1, 2, 1, 4):
                continue                     # the multi-launch case: one config
            kw = dict(tile_n=nb * R, waves_k=wk, unroll=u, split_k=s, swap_ab=swap)
            cfg = C(w8, **kw, x_lds=1)
            w8.validate_config(fmt, M, N, K, cfg, op="linear", packed=T)
            y1 = w8.linear(fmt, cs.x, wp, cs.sw, cfg=cfg, fused=True)
            xq, sx = w8.quantize_act(fmt, cs.x)
            y2 = w8.gemm_w8a8(fmt, xq, sx, wp, cs.sw, cfg=C(w8, **kw))
            torch.cuda.synchronize()
            assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), f"{fmt} T={T} M={M} {cfg}"
            n += 1
        assert_bf16_close(y1, cs.Y, f"{fmt} T={T} M={M} fused")
        assert n == (len(SEG_FUSED) * 4 if M <= R + 1 else 2)
    x = to_bf16_tensor(synthetic.activations_extreme(fmt, R + 1, K))
    cs = case(fmt, R + 1, N, K)
    wp = packed(w8, cs, T)
    kw = dict(tile_n=R, waves_k=2, unroll=2, split_k=2, swap_ab=1)
    y1 = w8.linear(fmt, x, wp, cs.sw, cfg=C(w8, **kw, x_lds=1), fused=True)
    xq, sx = w8.quantize_act(fmt, x)
    y2 = w8.gemm_w8a8(fmt, xq, sx, wp, cs.sw, cfg=C(w8, **kw))
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), f"{fmt} T={T} extreme rows"


def test_segmented_graph_replay(w8):
    """Split-K on layout 8 with M = 9 (three launches of 4, 4 and 1 token
    rows sharing the workspace) captured once and replayed with eager work
    in between; every replay equals the eager result bit for bit."""
    fmt, M, N, K = "FP8_Dynamic", 9, 512, 7168
    cs = case(fmt, M, N, K)
    wp = packed(w8, cs, 8)
    cfg = C(w8, tile_n=2, waves_k=1, unroll=4, split_k=2, swap_ab=1)
    ws = w8.Workspace(DEV, w8.workspace_size(fmt, M, N, K, cfg, packed=8))
    xq, sx = cs.gpu_act()
    eager = w8.gemm_w8a8(fmt, xq, sx, wp, cs.sw, cfg=cfg, workspace=ws).clone()
    y = torch.empty_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        w8.gemm_w8a8(fmt, xq, sx, wp, cs.sw, cfg=cfg, y=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w8.gemm_w8a8(fmt, xq, sx, wp, cs.sw, cfg=cfg, y=y, workspace=ws)
    for i in range(3):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
        junk = torch.randn(256, 256, device=DEV) @ torch.randn(256, 256, device=DEV)
        del junk
    assert_bf16_close(y, cs.Y, "segmented graph replay")
    # split-K arrival counters: multiples of 256 after every call
    assert (ws.buf[:16384 * 128].view(torch.int32).cpu() % 256 == 0).all()
