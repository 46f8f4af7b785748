"""GPU GEMM against the oracle.

- int32 accumulators (W8A8_INT8) bit-identical to the oracle's exact sums;
- fp32 accumulators (FP8 formats) within the fp32 summation bound of the
  oracle's exact sums;
- bf16 outputs of the whole path (GPU quantize + GPU GEMM, GPU-quantized
  weights) within atol = rtol = 1e-2 of the oracle's fp64 result;
- Standard / Split-K / Swap-AB and every tile choice give the same answer;
- split-K is deterministic, leaves its counters at multiples of 256 and survives graph
  capture and replay.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests.gpu_cases import DEV, Case, assert_bf16_close, u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w8():
    import bit_quantized_gemm_token_amd as mod
    return mod


COUNTERS = 16384 * 128   # workspace arrival-counter region


def C(w8, **kw):
    return w8.Config.make(**kw)


_cases = {}


def case(fmt, M, N, K):
    key = (fmt, M, N, K)
    if key not in _cases:
        _cases.clear()                       # keep one case resident at a time
        _cases[key] = Case(fmt, M, N, K)
    return _cases[key]


def acc_check(w8, cs, xq, sx, cfg, what="", packed=False):
    """Accumulator parity: int32 bit-exact, fp32 within the summation bound."""
    acc = w8.gemm_w8a8_acc(cs.fmt, xq, sx, cs.weights(packed), cs.sw, cfg=cfg)
    torch.cuda.synchronize()
    got = acc.cpu().numpy()
    ref = cs.acc_ref()
    if cs.fmt == "W8A8_INT8":
        assert np.array_equal(got.astype(np.int64), ref), f"{what}: int32 accumulators differ"
    else:
        bad = np.argwhere(np.abs(got - ref) > cs.acc_bound())
        assert bad.size == 0, f"{what}: {len(bad)} fp32 accumulators off, first {bad[:3]}"
    return acc


def full_path(w8, cs, cfg=None, packed=False):
    y = w8.linear(cs.fmt, cs.x, cs.weights(packed), cs.sw, cfg=cfg)
    torch.cuda.synchronize()
    return y


# -------------------------------------------------- the configurations --
def test_int8_standard_16x896x1024(w8):
    """W8A8_INT8, M=16, N=896, K=1024: Standard variant, split_k=1, swap_ab=0."""
    cs = case("W8A8_INT8", 16, 896, 1024)
    cfg = C(w8, tile_n=16, waves_k=4, unroll=2, split_k=1, swap_ab=0)
    xq, sx = cs.gpu_act()
    assert np.array_equal(u8(xq), cs.xq_ref)
    acc_check(w8, cs, xq, sx, cfg, "int8 standard")
    assert_bf16_close(full_path(w8, cs, cfg), cs.Y, "int8 standard")


@pytest.mark.parametrize("M", [1, 4, 16, 32])
def test_fp8_dynamic_4096(w8, M):
    """FP8_Dynamic, N=K=4096: default config, resolved (table) config and a spread of others."""
    cs = case("FP8_Dynamic", M, 4096, 4096)
    xq, sx = cs.gpu_act()
    cfgs = [None, w8.default_config("FP8_Dynamic", M, 4096, 4096),
            C(w8, tile_n=64, waves_k=2, unroll=1, split_k=4, swap_ab=0),
            C(w8, tile_n=32, waves_k=1, unroll=2, split_k=32, swap_ab=1),
            C(w8, tile_n=16, waves_k=8, unroll=4, split_k=1, swap_ab=1)]
    for packed in (False, True):
        for cfg in cfgs:
            acc_check(w8, cs, xq, sx, cfg, f"fp8 M={M} {cfg} packed={packed}", packed)
            assert_bf16_close(full_path(w8, cs, cfg, packed), cs.Y, f"fp8 M={M} {cfg}")


@pytest.mark.parametrize("M", [1, 8, 32])
def test_block_fp8_swap_on_and_off(w8, M):
    """Block_FP8, N=4608, K=7168: swap_ab forced to 0 and 1, both against the
    oracle and against each other."""
    cs = case("Block_FP8", M, 4608, 7168)
    xq, sx = cs.gpu_act()
    assert np.array_equal(u8(xq), cs.xq_ref)
    outs = []
    for swap in (0, 1):
        cfg = C(w8, tile_n=16, waves_k=4, unroll=2, split_k=2, swap_ab=swap)
        acc_check(w8, cs, xq, sx, cfg, f"block swap={swap}")
        acc_check(w8, cs, xq, sx, cfg, f"block swap={swap} packed", packed=True)
        y = full_path(w8, cs, cfg)
        assert_bf16_close(y, cs.Y, f"block M={M} swap={swap}")
        outs.append(y.float().cpu().numpy())
    np.testing.assert_allclose(outs[0], outs[1], rtol=1e-2, atol=1e-2)


@pytest.mark.parametrize("fmt", ["W8A8_INT8", "FP8_Dynamic"])
@pytest.mark.parametrize("M", [1, 2, 4, 8, 16, 32])
def test_split_k_sweep_512x7168(w8, fmt, M):
    """N=512, K=7168: every split_k in 1..256 against the oracle; int8
    accumulators are bit-identical for every setting."""
    cs = case(fmt, M, 512, 7168)
    xq, sx = cs.gpu_act()
    for s in [1 << i for i in range(9)]:
        for swap in (0, 1):
            cfg = C(w8, tile_n=16, waves_k=2, unroll=2, split_k=s, swap_ab=swap)
            acc_check(w8, cs, xq, sx, cfg, f"{fmt} M={M} split_k={s} swap={swap}")
            acc_check(w8, cs, xq, sx, cfg, f"{fmt} M={M} split_k={s} swap={swap} packed", True)
            assert_bf16_close(full_path(w8, cs, cfg), cs.Y, f"{fmt} M={M} split_k={s}")


# (waves_k, waves_n, x_lds)
WAVE_SHAPES = ((1, 1, 0), (2, 1, 0), (4, 1, 0), (8, 1, 0), (16, 1, 0), (1, 1, 1), (2, 1, 1),
               (4, 1, 1), (8, 1, 1), (1, 2, 1), (1, 4, 1), (1, 8, 1))


@pytest.mark.parametrize("fmt", ["W8A8_INT8", "FP8_Dynamic", "Block_FP8"])
def test_every_tile_config(w8, fmt):
    """Every (tile_n, waves_k x waves_n, x_lds, unroll, swap_ab, layout)
    instance at one ragged shape (M = 17 needs both 16-row blocks of M),
    whole tiles and split-K; the stream-K instances (tile_n 16, unroll 1 or
    2) with grids of 3 and 7 workgroups (several tiles and partial tiles per
    workgroup)."""
    M, N, K = (17, 200, 1280)
    cs = case(fmt, M, N, K)
    xq, sx = cs.gpu_act()
    n = 0
    for tn, (wk, wn, xl), u, swap, (s, grid), packed in itertools.product(
            (16, 32, 64), WAVE_SHAPES, (1, 2, 4), (0, 1), ((1, 0), (4, 0), (1, 3), (1, 7)),
            (0, 1)):
        if (tn // 16) * u > 4 or (grid and (tn != 16 or u > 2)):
            continue
        cfg = C(w8, tile_n=tn, waves_k=wk, waves_n=wn, unroll=u, split_k=s, grid=grid,
                swap_ab=swap, x_lds=xl)
        acc_check(w8, cs, xq, sx, cfg, f"{fmt} {cfg} packed={packed}", bool(packed))
        n += 1
    assert n == (6 * 12 * 2 * 2 + 2 * 12 * 2 * 2) * 2


@pytest.mark.parametrize("fmt,M", [("W8A8_INT8", 32), ("FP8_Dynamic", 16), ("Block_FP8", 1),
                                   ("Block_FP8", 32)])
def test_stream_k_and_shared_activations_large(w8, fmt, M):
    """Stream-K grids of 256/512/1024 workgroups, activations staged in LDS
    and waves side by side along N at a large shape (288 row blocks, 56 or
    112 K-steps: tiles shared by up to several workgroups), accumulators
    against the oracle."""
    cs = case(fmt, M, 4608, 7168)
    xq, sx = cs.gpu_act()
    for tn, wk, wn, u, s, grid, swap, xl in (
            (16, 1, 8, 2, 1, 256, 0, 1), (16, 1, 4, 1, 1, 512, 1, 1), (16, 2, 1, 2, 1, 1024, 0, 0),
            (16, 1, 2, 2, 1, 1024, 1, 1), (64, 1, 8, 1, 4, 0, 0, 1), (16, 4, 1, 2, 1, 512, 1, 0),
            (16, 2, 1, 2, 4, 0, 0, 1), (32, 1, 1, 1, 8, 0, 1, 1)):
        cfg = C(w8, tile_n=tn, waves_k=wk, waves_n=wn, unroll=u, split_k=s, grid=grid,
                swap_ab=swap, x_lds=xl)
        acc_check(w8, cs, xq, sx, cfg, f"{fmt} M={M} {cfg} packed", True)
    assert_bf16_close(full_path(w8, cs, cfg, True), cs.Y, f"{fmt} M={M} stream-K path")


@pytest.mark.parametrize("fmt,M,N,K", [
    ("W8A8_INT8", 1, 16, 16), ("W8A8_INT8", 5, 200, 208), ("W8A8_INT8", 32, 1000, 1040),
    ("W8A8_INT8", 17, 33, 80), ("FP8_Dynamic", 1, 16, 16), ("FP8_Dynamic", 5, 200, 208),
    ("FP8_Dynamic", 32, 1000, 1040), ("FP8_Dynamic", 31, 77, 336), ("Block_FP8", 1, 16, 128),
    ("Block_FP8", 5, 200, 384), ("Block_FP8", 32, 1000, 1024), ("Block_FP8", 20, 130, 256)])
def test_ragged_shapes(w8, fmt, M, N, K):
    """Ragged M (tile padding), N (partial tile) and K (masked tail step)."""
    cs = case(fmt, M, N, K)
    xq, sx = cs.gpu_act()
    assert np.array_equal(u8(xq), cs.xq_ref)
    for packed in (False, True):
        for cfg in (None, C(w8, tile_n=32, waves_k=2, unroll=2, split_k=8, swap_ab=0),
                    C(w8, tile_n=64, waves_k=1, unroll=1, split_k=2, swap_ab=1),
                    C(w8, tile_n=16, waves_k=1, waves_n=4, unroll=2,
                      grid=min(5, -(-N // 64) * -(-K // (64 if fmt == "W8A8_INT8" else 128))),
                      swap_ab=0),
                    C(w8, tile_n=16, waves_k=1, waves_n=8, unroll=1, split_k=2, swap_ab=1)):
            acc_check(w8, cs, xq, sx, cfg, f"ragged {cfg} packed={packed}", packed)
            assert_bf16_close(full_path(w8, cs, cfg, packed), cs.Y, f"ragged {fmt} {cfg}")


@pytest.mark.parametrize("fmt", ["W8A8_INT8", "FP8_Dynamic", "Block_FP8"])
@pytest.mark.parametrize("M,N,K", synthetic.SWEEP)
def test_sweep_shapes_resolved_config(w8, fmt, M, N, K):
    """The 24-shape sweep with the config the library resolves (table or
    default), in both weight layouts."""
    cs = case(fmt, M, N, K)
    assert_bf16_close(full_path(w8, cs), cs.Y, f"sweep {fmt} {M}x{N}x{K}")
    assert_bf16_close(full_path(w8, cs, packed=True), cs.Y, f"sweep packed {fmt} {M}x{N}x{K}")


def _pack_reference(codes, kstep):
    """The packed layout written out with numpy: fragment (row block, K-step)
    of 16 x kstep bytes, load instruction jj at jj*1024, lane l's 16 bytes at
    16*l = row 16*nb + l%16, bytes kstep*kk + 64*jj + 16*(l//16) .. +16."""
    N, K = codes.shape
    nblk, ks = -(-N // 16), -(-K // kstep)
    padded = np.zeros((nblk * 16, ks * kstep), np.uint8)
    padded[:N, :K] = codes
    out = np.zeros((nblk, ks, kstep // 64, 64, 16), np.uint8)
    for l in range(64):
        r, g = l % 16, l // 16
        for jj in range(kstep // 64):
            cols = np.arange(ks)[:, None] * kstep + 64 * jj + 16 * g + np.arange(16)[None, :]
            out[:, :, jj, l, :] = padded.reshape(nblk, 16, -1)[:, r, :][:, cols]
    return out.reshape(-1)


@pytest.mark.parametrize("fmt,N,K", [("W8A8_INT8", 200, 208), ("FP8_Dynamic", 37, 400),
                                     ("Block_FP8", 130, 384), ("W8A8_INT8", 512, 7168)])
def test_pack_weight_layout(w8, fmt, N, K):
    rng = np.random.default_rng(N + K)
    codes = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    got = w8.pack_weight(fmt, torch.from_numpy(codes).to(DEV)).data.cpu().numpy()
    kstep = 64 if fmt == "W8A8_INT8" else 128
    assert got.size == w8.packed_weight_size(fmt, N, K)
    assert np.array_equal(got, _pack_reference(codes, kstep))


# ------------------------------------------------ properties of the path --
def test_split_k_deterministic_and_counter_state(w8):
    cs = case("FP8_Dynamic", 8, 1024, 4096)
    xq, sx = cs.gpu_act()
    cfg = C(w8, tile_n=16, waves_k=2, unroll=2, split_k=16, swap_ab=1)
    ws = w8.Workspace(DEV)
    need = w8.workspace_size("FP8_Dynamic", 8, 1024, 4096, cfg)
    ys = [w8.gemm_w8a8("FP8_Dynamic", xq, sx, cs.wq, cs.sw, cfg=cfg, workspace=ws) for _ in range(3)]
    ys += [w8.gemm_w8a8("FP8_Dynamic", xq, sx, cs.packed(), cs.sw, cfg=cfg, workspace=ws)
           for _ in range(2)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16))
    assert need > COUNTERS
    ctr = ws.buf[:COUNTERS].view(torch.int32).cpu().numpy().reshape(-1, 32)
    # split-K: word 0 of each tile's line rises by 256 per call (5 calls here)
    assert (ctr[:64, 0] == 5 * 256).all() and (ctr[64:] == 0).all() and (ctr[:, 1:] == 0).all()
    # stream-K with shared activations: same properties
    cfg = C(w8, tile_n=16, waves_k=1, waves_n=4, unroll=2, grid=96, swap_ab=0)
    ws2 = w8.Workspace(DEV, w8.workspace_size("FP8_Dynamic", 8, 1024, 4096, cfg, packed=True))
    zs = [w8.gemm_w8a8("FP8_Dynamic", xq, sx, cs.packed(), cs.sw, cfg=cfg, workspace=ws2)
          for _ in range(3)]
    torch.cuda.synchronize()
    for z in zs[1:]:
        assert torch.equal(z.view(torch.int16), zs[0].view(torch.int16))
    # stream-K: word 1 of the line, back at zero after every call
    assert (ws2.buf[:COUNTERS].cpu() == 0).all()
    assert_bf16_close(zs[0], cs.Y, "stream-K")


def test_unsupported_m_raises(w8):
    x = torch.zeros((33, 256), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(w8.UnsupportedShape):
        w8.quantize_act("FP8_Dynamic", x)
    xq = torch.zeros((33, 256), dtype=torch.uint8, device=DEV)
    wq = torch.zeros((64, 256), dtype=torch.uint8, device=DEV)
    with pytest.raises(w8.UnsupportedShape):
        w8.gemm_w8a8("FP8_Dynamic", xq, torch.ones(33, device=DEV), wq, torch.ones(64, device=DEV))


@pytest.mark.parametrize("kind", ["split_k", "stream_k"])
def test_graph_capture_replay(w8, kind):
    """quantize + GEMM (split-K, or stream-K with shared activations) captured
    once, replayed with eager work in between; every replay equals the eager
    result bit for bit."""
    cs = case("Block_FP8", 8, 4608, 7168)
    if kind == "split_k":
        cfg = C(w8, tile_n=16, waves_k=4, unroll=2, split_k=8, swap_ab=1)
    else:
        cfg = C(w8, tile_n=16, waves_k=1, waves_n=8, unroll=2, grid=512, swap_ab=1)
    ws = w8.Workspace(DEV, w8.workspace_size("Block_FP8", 8, 4608, 7168, cfg, packed=True))
    wp = cs.packed()
    eager = w8.linear("Block_FP8", cs.x, wp, cs.sw, cfg=cfg, workspace=ws).clone()
    x_static = cs.x.clone()
    y_static = torch.empty_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        w8.linear("Block_FP8", x_static, wp, cs.sw, cfg=cfg, y=y_static, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w8.linear("Block_FP8", x_static, wp, cs.sw, cfg=cfg, y=y_static, workspace=ws)
    for i in range(4):
        y_static.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_static.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
        junk = torch.randn(1024, 1024, device=DEV) @ torch.randn(1024, 1024, device=DEV)
        del junk
    assert_bf16_close(y_static, cs.Y, "graph replay")


@pytest.mark.parametrize("fmt", ["W8A8_INT8", "FP8_Dynamic"])
def test_deepest_k_accumulators(w8, fmt):
    """K = 131072, the deepest K whose all-max int8 sum fits int32 with room
    (131072 x 127^2 = 2 114 060 288 < 2^31 - 1): rows of all +max and all
    -max codes against all-max weight rows give +-K Qmax^2 (E4M3FN: 448^2 K =
    49 x 2^29, a value every partial sum of which fp32 holds exactly), and
    random rows the oracle's exact sums -- under Standard, split-K 16 and
    256, Swap-AB, staged activations with waves along N, and stream-K, with
    unit scales."""
    M, N, K = 4, 48, 131072
    int8 = fmt == "W8A8_INT8"
    g = np.random.Generator(np.random.PCG64(5))
    if int8:
        pos, neg = 0x7F, 0x81                               # +127, -127
        rnd = lambda shape: g.integers(-127, 128, size=shape, dtype=np.int8).view(np.uint8)
        qmax = 127
    else:
        pos, neg = 0x7E, 0xFE                               # +448, -448
        def rnd(shape):
            c = g.integers(0, 256, size=shape, dtype=np.int64).astype(np.uint8)
            c[(c & 0x7F) == 0x7F] = 0x38                     # no NaN codes
            return c
        qmax = 448
    xq = np.empty((M, K), np.uint8)
    xq[0], xq[1] = pos, neg
    xq[2:] = rnd((M - 2, K))
    wq = np.empty((N, K), np.uint8)
    wq[:16] = pos
    wq[16:] = rnd((N - 16, K))
    dt = torch.int8 if int8 else torch.float8_e4m3fn
    xt = torch.from_numpy(xq).to(DEV).view(dt)
    wt = torch.from_numpy(wq).to(DEV).view(dt)
    ones_m = torch.ones(M, dtype=torch.float32, device=DEV)
    ones_n = torch.ones(N, dtype=torch.float32, device=DEV)
    ref = oracle.acc_int8(xq, wq) if int8 else oracle.acc_fp8(xq, wq)
    closed = K * qmax * qmax
    assert np.all(ref[0, :16] == closed) and np.all(ref[1, :16] == -closed)
    if not int8:  # magnitude bound of the E4M3FN accumulation (see Case.acc_bound)
        dec = oracle.e4m3_decode(xq).astype(np.float64)
        decw = oracle.e4m3_decode(wq).astype(np.float64)
        bound = 2.0 ** -14 * (np.abs(dec) @ np.abs(decw).T)
    for kw in (dict(tile_n=16, waves_k=4, unroll=2, split_k=1),
               dict(tile_n=16, waves_k=8, unroll=1, split_k=256),
               dict(tile_n=32, waves_k=2, unroll=2, split_k=16, swap_ab=1),
               dict(tile_n=16, waves_k=1, waves_n=2, unroll=1, split_k=64, x_lds=1),
               dict(tile_n=16, waves_k=4, unroll=1, grid=100)):
        print(f"[deep K] {fmt} {kw}", flush=True)
        acc = w8.gemm_w8a8_acc(fmt, xt, ones_m, wt, ones_n, cfg=C(w8, **kw))
        torch.cuda.synchronize()
        got = acc.cpu().numpy()
        if int8:
            assert np.array_equal(got.astype(np.int64), ref), f"{kw}"
        else:
            assert np.all(np.abs(got.astype(np.float64) - ref) <= bound), f"{kw}"


@pytest.mark.parametrize("fmt,M,N,K", [("W8A8_INT8", 2, (1 << 24) - 7, 16),
                                       ("W8A8_INT8", 3, 16, 1 << 22),
                                       ("FP8_Dynamic", 2, 40, 1 << 22)])
def test_largest_n_and_k(w8, fmt, M, N, K):
    """The largest N (2^24, here with a ragged last tile) and K (2^22) the
    library accepts, with random codes and unit scales: the default config
    and an explicit one, accumulators against the oracle's exact sums (all
    of them, or for the 2^24 columns a sample with the ragged tail)."""
    g = np.random.Generator(np.random.PCG64(K + N))
    int8 = fmt == "W8A8_INT8"
    def rnd(shape):
        if int8:
            return g.integers(-127, 128, size=shape, dtype=np.int8).view(np.uint8)
        c = g.integers(0, 256, size=shape, dtype=np.int64).astype(np.uint8)
        c[(c & 0x7F) == 0x7F] = 0x38
        return c
    xq, wq = rnd((M, K)), rnd((N, K))
    dt = torch.int8 if int8 else torch.float8_e4m3fn
    xt = torch.from_numpy(xq).to(DEV).view(dt)
    wt = torch.from_numpy(wq).to(DEV).view(dt)
    ones_m = torch.ones(M, dtype=torch.float32, device=DEV)
    ones_n = torch.ones(N, dtype=torch.float32, device=DEV)
    cols = np.arange(N) if N <= 4096 else np.unique(np.r_[g.integers(0, N, 4096),
                                                          np.arange(N - 80, N)])
    if int8:
        ref = oracle.acc_int8(xq, wq[cols])
    else:
        ref = oracle.acc_fp8(xq, wq[cols])
        dec = np.abs(oracle.e4m3_decode(xq)).astype(np.float32)  # a bound: fp32 suffices
        decw = np.abs(oracle.e4m3_decode(wq[cols])).astype(np.float32)
        bound = 2.0 ** -14 * (dec @ decw.T).astype(np.float64) * 1.001
    for cfg in (None, C(w8, tile_n=64, waves_k=1, unroll=1, split_k=1),
                C(w8, tile_n=16, waves_k=8, unroll=1, split_k=1)):
        print(f"[largest] {fmt} M={M} N={N} K={K} {cfg}", flush=True)
        acc = w8.gemm_w8a8_acc(fmt, xt, ones_m, wt, ones_n, cfg=cfg)
        torch.cuda.synchronize()
        got = acc[:, torch.from_numpy(cols).to(DEV)].cpu().numpy()
        if int8:
            assert np.array_equal(got.astype(np.int64), ref), f"{cfg}"
        else:
            assert np.all(np.abs(got.astype(np.float64) - ref) <= bound), f"{cfg}"


@pytest.mark.parametrize("M", [5, 20])
def test_block_fp8_long_segments(w8, M):
    """Block_FP8 at a K longer than the sweep's (16384: 128 groups, each
    K-step's products scaled by its own pair of group scales): split_k 1, 2
    and 4, one and four K-waves, both Swap-AB settings, one and two 16-row
    blocks of M, row-major and packed weights; accumulators against the
    oracle within the fp32 summation bound."""
    cs = case("Block_FP8", M, 160, 16384)
    xq, sx = cs.gpu_act()
    for s, wk, swap, packed in itertools.product((1, 2, 4), (1, 4), (0, 1), (0, 1)):
        cfg = C(w8, tile_n=16, waves_k=wk, unroll=2, split_k=s, swap_ab=swap)
        acc_check(w8, cs, xq, sx, cfg, f"Block_FP8 M={M} K=16384 {cfg} packed={packed}",
                  bool(packed))
