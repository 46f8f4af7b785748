"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, rejects bad arguments before touching the device, and its
config table parses, saves, reloads and falls back as documented."""
import ctypes
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w8gemm.h")


@pytest.fixture(scope="module")
def w8():
    import bit_quantized_gemm_token_amd as mod
    return mod


@pytest.fixture(scope="module")
def lib(w8):
    return w8._lib


@pytest.fixture(autouse=True)
def _clean_table(w8):
    w8.clear_config_table()
    yield
    w8.clear_config_table()


def test_exports_every_declared_symbol(lib):
    text = open(HEADER).read()
    declared = sorted(set(re.findall(r"\b(w8_[a-z0-9_]+)\s*\(", text)))
    assert len(declared) >= 20
    from bit_quantized_gemm_token_amd import _capi
    assert sorted(_capi.EXPORTS) == declared
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _capi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(set(re.findall(r" T (\w+)", out)))
    assert exported == declared          # nothing else leaks out of the library


def test_abi_and_status_strings(lib):
    assert lib.w8_abi_version() == 5
    assert lib.w8_status_string(2) == b"W8_E_UNSUPPORTED"
    assert lib.w8_status_string(99) == b"W8_E_UNKNOWN"


def test_pages_constants_match_library(w8):
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_constants.json")))
    assert list(w8.FORMATS) == g["formats"]["value"]
    assert w8.MAX_M == g["max_tokens"]["value"]
    allowed = [s for s in range(1, 513)
               if _valid(w8, "W8A8_INT8", 16, 512, 1024, w8.Config.make(split_k=s))]
    assert allowed == g["split_k_values"]["value"]
    # M window: 32 accepted, 33 refused as unsupported (caller falls back)
    w8.default_config("FP8_Dynamic", g["max_tokens"]["value"], 256, 256)
    with pytest.raises(w8.UnsupportedShape):
        w8.default_config("FP8_Dynamic", g["max_tokens"]["value"] + 1, 256, 256)


def _valid(w8, fmt, M, N, K, cfg):
    try:
        w8.validate_config(fmt, M, N, K, cfg)
        return True
    except w8.W8Error:
        return False


@pytest.mark.parametrize("field,value", [("tile_n", 8), ("tile_n", 128), ("waves_k", 3),
                                         ("waves_k", 32), ("unroll", 3), ("split_k", 0),
                                         ("split_k", 3), ("split_k", 512), ("swap_ab", 2)])
def test_config_rejects(w8, field, value):
    cfg = w8.Config.make()
    setattr(cfg, field, value)
    assert not _valid(w8, "FP8_Dynamic", 4, 512, 1024, cfg)


def test_config_rejects_abi_and_reserved(w8):
    cfg = w8.Config.make()
    cfg.abi_version = 1
    assert not _valid(w8, "FP8_Dynamic", 4, 512, 1024, cfg)
    cfg = w8.Config.make()
    cfg.reserved[0] = 7
    assert not _valid(w8, "FP8_Dynamic", 4, 512, 1024, cfg)
    cfg = w8.Config.make(tile_n=64, unroll=2)    # 4 row blocks x unroll 2 > 4 registers sets
    assert not _valid(w8, "FP8_Dynamic", 4, 512, 1024, cfg)
    cfg = w8.Config.make(tile_n=32, unroll=4)
    assert not _valid(w8, "FP8_Dynamic", 4, 512, 1024, cfg)
    assert _valid(w8, "FP8_Dynamic", 4, 512, 1024, w8.Config.make(tile_n=64, unroll=1, waves_k=16))


def test_config_rejects_wave_shapes_and_grids(w8):
    M, N, K = 4, 512, 1024                       # FP8: 8 K-steps
    ok = w8.Config.make(tile_n=16, waves_k=1, waves_n=8, unroll=2)
    assert _valid(w8, "FP8_Dynamic", M, N, K, ok)
    for kw in (dict(waves_n=3), dict(waves_n=16), dict(waves_n=0),
               dict(waves_n=2, waves_k=2),       # waves split either K or N
               dict(grid=-1), dict(grid=256, split_k=2),
               dict(waves_n=2, x_lds=0),         # side by side along N shares through LDS
               dict(waves_k=16, x_lds=1), dict(x_lds=2)):
        cfg = w8.Config.make(**dict(dict(tile_n=16, waves_k=1, unroll=2), **kw))
        assert not _valid(w8, "FP8_Dynamic", M, N, K, cfg), kw
    # stream-K: at most one workgroup per (tile, K-step) iteration
    iters = (N // (16 * 4)) * (K // 128)         # 8 tiles of 4 waves x 8 K-steps = 64
    assert _valid(w8, "FP8_Dynamic", M, N, K, w8.Config.make(tile_n=16, waves_k=1, waves_n=4,
                                                              grid=iters))
    assert not _valid(w8, "FP8_Dynamic", M, N, K, w8.Config.make(tile_n=16, waves_k=1,
                                                                  waves_n=4, grid=iters + 1))
    # stream-K is compiled for tile_n 16 with unroll 1 or 2 only
    for kw in (dict(tile_n=32, unroll=1), dict(tile_n=64, unroll=1), dict(tile_n=16, unroll=4)):
        assert not _valid(w8, "FP8_Dynamic", M, N, K,
                          w8.Config.make(**dict(dict(waves_k=1, grid=8), **kw))), kw
    # x_lds: the workgroup's K range of activations must fit in 64 KiB
    # (ceil(M/16) x K-steps x K-step/64 chunks of 1 KiB)
    K2 = 7168                                    # FP8: 56 K-steps, 2 chunks each
    assert _valid(w8, "FP8_Dynamic", 16, N, K2, w8.Config.make(waves_k=1, x_lds=1, split_k=2))
    assert not _valid(w8, "FP8_Dynamic", 16, N, K2, w8.Config.make(waves_k=1, x_lds=1))
    assert not _valid(w8, "FP8_Dynamic", 32, N, K2, w8.Config.make(waves_k=1, x_lds=1,
                                                                   split_k=2))
    assert _valid(w8, "FP8_Dynamic", 32, N, K2, w8.Config.make(waves_k=1, x_lds=1, split_k=4))


def _max_contributors(I, G, KS, T):
    # by definition: workgroup g owns iterations [g*I//G, (g+1)*I//G)
    starts = [g * I // G for g in range(G + 1)]
    most = 0
    for t in range(T):
        lo, hi = t * KS, (t + 1) * KS
        most = max(most, sum(1 for g in range(G) if starts[g] < hi and starts[g + 1] > lo))
    return most


@pytest.mark.parametrize("N,K,grid", [(512, 7168, 256), (4608, 7168, 256), (4608, 7168, 1024),
                                      (896, 1024, 256), (896, 1024, 448), (5120, 640, 512),
                                      (272, 640, 7), (80, 256, 3)])
def test_stream_k_workspace_covers_every_tile(w8, N, K, grid):
    cfg = w8.Config.make(tile_n=16, waves_k=1, waves_n=1, unroll=1, grid=grid)
    KS = K // 64                                 # W8A8_INT8 K-steps
    T = -(-N // 16)
    need = w8.workspace_size("W8A8_INT8", 20, N, K, cfg)
    slots = (need - COUNTERS) // (T * 1 * 2 * 1024)  # 1 row block per tile, 2 blocks of M
    assert need == COUNTERS + T * slots * 1 * 2 * 1024
    assert slots >= _max_contributors(T * KS, grid, KS, T)


def test_config_rejects_grid_overflow(w8):
    # 16384 tiles x 256 splits x 16 waves x 64 lanes = 2^32 threads: one more
    # than a launch can hold; half the waves fit
    big = w8.Config.make(tile_n=64, unroll=1, waves_k=16, split_k=256)
    with pytest.raises(w8.W8Error, match="2\\^32"):
        w8.validate_config("FP8_Dynamic", 1, 16384 * 64, 1 << 20, big)
    assert _valid(w8, "FP8_Dynamic", 1, 16384 * 64, 1 << 20,
                  w8.Config.make(tile_n=64, unroll=1, waves_k=8, split_k=256))


def test_default_config_is_valid_everywhere(w8):
    import synthetic
    for fmt in w8.FORMATS:
        for (M, N, K) in synthetic.SWEEP + ((2, 512, 7168), (32, 4096, 4096), (32, 5120, 8192)):
            c = w8.default_config(fmt, M, N, K)
            w8.validate_config(fmt, M, N, K, c)
            assert c.swap_ab == (1 if M < 32 else 0)
            cl = w8.default_config(fmt, M, N, K, op="linear")
            w8.validate_config(fmt, M, N, K, cl, op="linear")
            assert cl.x_lds == 1
            # the GEMM default (no x_lds, unroll 2) is no linear config
            assert not _valid_op(w8, fmt, M, N, K, c, "linear")


def _valid_op(w8, fmt, M, N, K, cfg, op):
    try:
        w8.validate_config(fmt, M, N, K, cfg, op=op)
        return True
    except w8.W8Error:
        return False


def test_linear_config_rules(w8):
    ok = w8.Config.make(waves_k=4, x_lds=1, split_k=2)
    assert _valid_op(w8, "FP8_Dynamic", 4, 512, 1024, ok, "linear")
    assert not _valid_op(w8, "FP8_Dynamic", 4, 512, 1024, w8.Config.make(waves_k=8, x_lds=1),
                         "linear")                                   # waves_k <= 4
    assert _valid_op(w8, "FP8_Dynamic", 4, 512, 1024,
                     w8.Config.make(waves_k=1, waves_n=8, x_lds=1), "linear")
    with pytest.raises(ValueError):
        w8.validate_config("FP8_Dynamic", 4, 512, 1024, ok, op="fused")
    # Block_FP8 linear may quantize in the K loop (x_lds 0): waves along K
    # only, at most 8 of them, unroll <= 2; not the per-token formats (their
    # row scale needs the whole row), not the grouped op
    inloop = w8.Config.make(waves_k=8, unroll=1, x_lds=0, split_k=2)
    assert _valid_op(w8, "Block_FP8", 4, 512, 1024, inloop, "linear")
    assert not _valid_op(w8, "FP8_Dynamic", 4, 512, 1024, inloop, "linear")
    assert not _valid_op(w8, "W8A8_INT8", 4, 512, 1024, inloop, "linear")
    for bad in (w8.Config.make(waves_k=8, unroll=2, tile_n=16, x_lds=0),
                w8.Config.make(waves_k=16, unroll=1, x_lds=0),
                w8.Config.make(waves_k=1, unroll=1, x_lds=0),
                w8.Config.make(waves_k=4, unroll=1, tile_n=64, x_lds=0)):
        assert not _valid_op(w8, "Block_FP8", 4, 512, 1024, bad, "linear")
    assert not _valid_op(w8, "Block_FP8", 4, 512, 1024, inloop, "moe_linear")


def test_quant_launch_rules_and_workspace(w8):
    """quant_launch = 1: the linear op quantizes in a launch of its own into
    the workspace and runs the GEMM under the GEMM's rules."""
    g = w8.Config.make(waves_k=8, split_k=4)                         # a GEMM config, no x_lds
    ql = w8.Config.make(waves_k=8, split_k=4, quant_launch=1)
    assert not _valid_op(w8, "FP8_Dynamic", 4, 512, 1024, g, "linear")
    assert _valid_op(w8, "FP8_Dynamic", 4, 512, 1024, ql, "linear")
    assert not _valid_op(w8, "FP8_Dynamic", 4, 512, 1024, ql, "gemm")  # linear only
    bad = w8.Config.make(waves_k=8, quant_launch=2)
    assert not _valid_op(w8, "FP8_Dynamic", 4, 512, 1024, bad, "linear")
    assert not _valid_op(w8, "FP8_Dynamic", 4, 512, 1024,
                         w8.Config.make(waves_k=16, x_lds=1, quant_launch=1), "linear")

    def r256(b):
        return (b + 255) // 256 * 256

    for fmt, M, N, K in (("FP8_Dynamic", 4, 512, 1024), ("Block_FP8", 17, 300, 1152),
                         ("W8A8_INT8", 32, 64, 208)):
        gemm_ws = w8.workspace_size(fmt, M, N, K, g)
        nsx = M * (K // 128) if fmt == "Block_FP8" else M
        assert gemm_ws > COUNTERS
        want = r256(gemm_ws) + r256(M * ((K + 15) // 16 * 16)) + r256(4 * nsx)
        assert w8.workspace_size(fmt, M, N, K, ql, op="linear") == want
        # no shared tiles: the codes still start past the counter region
        one = w8.Config.make(waves_k=8, quant_launch=1)
        assert w8.workspace_size(fmt, M, N, K, one, op="linear") == \
            COUNTERS + r256(M * ((K + 15) // 16 * 16)) + r256(4 * nsx)
        assert w8.workspace_size(fmt, M, N, K, w8.Config.make(waves_k=8)) == 0


FAKE = ctypes.c_void_p(0x100000)   # 16-byte aligned, never dereferenced
COUNTERS = 16384 * 128              # workspace arrival-counter region


def _gemm(lib, fmt=0, M=4, N=64, K=256, xq=FAKE, ldq=256, sx=FAKE, wq=FAKE, ldw=256, sw=FAKE,
          y=FAKE, ldy=64, cfg=None, ws=None, wsb=0):
    return lib.w8_gemm_w8a8(fmt, M, N, K, xq, ldq, sx, wq, ldw, sw, y, ldy, cfg, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=0), 1), (dict(M=33), 2), (dict(N=0), 1), (dict(K=0), 1), (dict(K=200), 1),
    (dict(fmt=2, K=272, ldq=272, ldw=272), 1), (dict(fmt=7), 1),
    (dict(xq=None), 1), (dict(sw=None), 1), (dict(y=None), 1),
    (dict(xq=ctypes.c_void_p(0x100008)), 1), (dict(ldq=255), 1), (dict(ldw=248), 1),
    (dict(ldw=-16), 1), (dict(wq=ctypes.c_void_p(0x100004), ldw=0), 1),
    (dict(ldy=63), 1), (dict(sx=ctypes.c_void_p(0x100002)), 1)])
def test_gemm_argument_errors(lib, kw, status):
    assert _gemm(lib, **kw) == status
    assert lib.w8_last_error() != b""


def test_gemm_workspace_errors(w8, lib):
    cfg = w8.Config.make(split_k=8)
    need = w8.workspace_size("FP8_Dynamic", 4, 64, 1024, cfg)
    assert need > 0
    assert _gemm(lib, K=1024, ldq=1024, ldw=1024, cfg=ctypes.byref(cfg)) == 3
    assert _gemm(lib, K=1024, ldq=1024, ldw=1024, cfg=ctypes.byref(cfg), ws=FAKE, wsb=need - 1) == 3
    assert b"workspace" in lib.w8_last_error()
    assert w8.workspace_size("FP8_Dynamic", 4, 64, 1024, w8.Config.make(split_k=1)) == 0
    # counters (one per 128-byte line, 16384 tiles: 2 MiB) + one 1 KiB fragment
    # per (tile, split, row block, M block)
    assert need == COUNTERS + 4 * 8 * 1 * 1 * 1024
    assert w8.workspace_size("FP8_Dynamic", 20, 64, 1024, w8.Config.make(tile_n=32, unroll=2,
                                                                         split_k=8)) == \
        COUNTERS + 2 * 8 * 2 * 2 * 1024


def test_pack_argument_errors(w8, lib):
    # every call here fails validation before anything touches a device
    p = lib.w8_pack_weight
    assert p(0, 64, 256, FAKE, 248, FAKE, 1, None) == 1            # ldw < K
    assert p(0, 64, 200, FAKE, 256, FAKE, 1, None) == 1            # K % 16
    assert p(2, 64, 192, FAKE, 256, FAKE, 1, None) == 1            # Block_FP8 K % 128
    assert p(0, 64, 256, None, 256, FAKE, 1, None) == 1
    assert p(0, 64, 256, FAKE, 256, ctypes.c_void_p(0x100008), 1, None) == 1
    for bad_layout in (0, 3, 16, -1):
        assert p(0, 64, 256, FAKE, 256, FAKE, bad_layout, None) == 1
    # 16-row blocks x K-steps x (16 x K-step) bytes, zero padded
    assert w8.packed_weight_size("W8A8_INT8", 17, 80) == 2 * 2 * 16 * 64
    assert w8.packed_weight_size("FP8_Dynamic", 200, 208) == 13 * 2 * 16 * 128
    assert w8.packed_weight_size("Block_FP8", 4608, 7168) == 4608 * 7168
    # K-segmented: (16/T)-row blocks x spans of T K-steps x (16 x K-step) bytes
    assert w8.packed_weight_size("FP8_Dynamic", 200, 208, layout=2) == 25 * 1 * 16 * 128
    assert w8.packed_weight_size("FP8_Dynamic", 200, 1040, layout=8) == 100 * 2 * 16 * 128
    assert w8.packed_weight_size("W8A8_INT8", 17, 80, layout="seg4") == 5 * 1 * 16 * 64
    assert w8.packed_weight_size("Block_FP8", 4608, 7168, layout=8) == 4608 * 7168
    with pytest.raises(w8.W8Error):
        w8.packed_weight_size("FP8_Dynamic", 64, 256, layout=0)
    with pytest.raises(ValueError):
        w8.packed_weight_size("FP8_Dynamic", 64, 256, layout=3)


def test_linear_argument_errors(w8, lib):
    # every call here fails validation before anything touches a device
    L = lib.w8_linear
    cfg = w8.Config.make(waves_k=4, x_lds=1)
    c = ctypes.byref(cfg)
    assert L(0, 33, 64, 256, FAKE, 256, FAKE, 256, FAKE, FAKE, 64, c, None, 0, None) == 2
    assert L(0, 4, 64, 200, FAKE, 256, FAKE, 256, FAKE, FAKE, 64, c, None, 0, None) == 1
    assert L(0, 4, 64, 256, None, 256, FAKE, 256, FAKE, FAKE, 64, c, None, 0, None) == 1
    assert L(0, 4, 64, 256, ctypes.c_void_p(0x100008), 256, FAKE, 256, FAKE, FAKE, 64, c, None, 0,
             None) == 1                                              # x not 16-byte aligned
    assert L(0, 4, 64, 256, FAKE, 252, FAKE, 256, FAKE, FAKE, 64, c, None, 0, None) == 1
    assert L(0, 4, 64, 256, FAKE, 256, FAKE, 248, FAKE, FAKE, 64, c, None, 0, None) == 1
    assert L(0, 4, 64, 256, FAKE, 256, FAKE, 256, FAKE, FAKE, 63, c, None, 0, None) == 1
    gemm_cfg = w8.Config.make(waves_k=4)                            # no x_lds
    assert L(0, 4, 64, 256, FAKE, 256, FAKE, 256, FAKE, FAKE, 64, ctypes.byref(gemm_cfg), None,
             0, None) == 1
    assert b"x_lds" in lib.w8_last_error()
    sk = w8.Config.make(waves_k=4, x_lds=1, split_k=2)
    assert L(0, 4, 64, 256, FAKE, 256, FAKE, 256, FAKE, FAKE, 64, ctypes.byref(sk), None, 0,
             None) == 3                                              # workspace missing
    ql = w8.Config.make(waves_k=4, quant_launch=1)                    # codes live in the workspace
    assert L(0, 4, 64, 256, FAKE, 256, FAKE, 256, FAKE, FAKE, 64, ctypes.byref(ql), None, 0,
             None) == 3
    assert L(0, 4, 64, 256, FAKE, 256, FAKE, 256, FAKE, FAKE, 64, ctypes.byref(ql), FAKE,
             COUNTERS + 1279, None) == 3                             # counters, codes, scales - 1


def test_quantize_argument_errors(lib):
    q = lib.w8_quantize_act
    assert q(0, 33, 256, FAKE, 256, FAKE, 256, FAKE, None) == 2
    assert q(0, 4, 100, FAKE, 256, FAKE, 256, FAKE, None) == 1
    assert q(2, 4, 192, FAKE, 256, FAKE, 256, FAKE, None) == 1
    assert q(0, 4, 256, FAKE, 252, FAKE, 256, FAKE, None) == 1
    assert q(0, 4, 256, FAKE, 256, FAKE, 264, FAKE, None) == 1
    assert q(0, 4, 256, None, 256, FAKE, 256, FAKE, None) == 1
    w = lib.w8_quantize_weight
    assert w(1, 4, 256, FAKE, 256, FAKE, 256, FAKE, None) == 1   # int8 weights are given
    assert w(0, 0, 256, FAKE, 256, FAKE, 256, FAKE, None) == 1


def test_table_roundtrip_and_lookup(w8, tmp_path):
    c1 = w8.Config.make(tile_n=32, waves_k=2, unroll=2, split_k=16, swap_ab=1)
    c2 = w8.Config.make(tile_n=16, waves_k=8, unroll=1, split_k=1, swap_ab=0)
    w8.set_config("FP8_Dynamic", 4, 4096, 4096, c1, 3.25)
    w8.set_config("Block_FP8", 32, 4608, 7168, c2, 5.5, packed=True)
    assert w8.config_table_size() == 2
    assert w8.lookup_config("FP8_Dynamic", 4, 4096, 4096) == c1
    assert w8.lookup_config("FP8_Dynamic", 4, 4096, 4096, op="linear") is None
    assert w8.lookup_config("FP8_Dynamic", 4, 4096, 4096, packed=True) is None
    assert w8.lookup_config("FP8_Dynamic", 5, 4096, 4096) is None
    assert w8.lookup_config("Block_FP8", 32, 4608, 7168, packed=True, with_time=True) == (c2, 5.5)
    got, hit = w8.resolve_config("Block_FP8", 32, 4608, 7168, packed=True)
    assert hit and got == c2
    got, hit = w8.resolve_config("Block_FP8", 32, 4608, 7168)       # other layout -> model
    assert hit == 0 and got == w8.model_config("Block_FP8", 32, 4608, 7168)
    got, hit = w8.resolve_config("Block_FP8", 16, 4608, 7168)       # other bucket -> model
    assert hit == 0 and got == w8.model_config("Block_FP8", 16, 4608, 7168)
    assert w8.best_layout("Block_FP8", 32, 4608, 7168) == 1
    assert w8.best_layout("FP8_Dynamic", 4, 4096, 4096) == 0
    # the fused linear op has entries of its own
    c3 = w8.Config.make(tile_n=16, waves_k=1, waves_n=8, unroll=1, split_k=4, x_lds=1)
    w8.set_config("Block_FP8", 32, 4608, 7168, c3, 7.5, packed=True, op="linear")
    assert w8.lookup_config("Block_FP8", 32, 4608, 7168, packed=True, op="linear") == c3
    assert w8.lookup_config("Block_FP8", 32, 4608, 7168, packed=True) == c2
    got, hit = w8.resolve_config("Block_FP8", 32, 4608, 7168, packed=True, op="linear")
    assert hit == 1 and got == c3
    got, hit = w8.resolve_config("Block_FP8", 32, 4608, 7168, op="linear")
    assert hit == 0 and got == w8.model_config("Block_FP8", 32, 4608, 7168, op="linear")
    with pytest.raises(w8.W8Error):                                  # a GEMM config is no linear one
        w8.set_config("Block_FP8", 32, 4608, 7168, w8.Config.make(tile_n=16, waves_k=16, unroll=1),
                      5.5, packed=True, op="linear")
    p = tmp_path / "t.tbl"
    w8.save_config_table(str(p))
    assert " linear packed 32 4608 7168 " in p.read_text()
    w8.clear_config_table()
    assert w8.config_table_size() == 0
    w8.load_config_table(str(p))
    assert w8.config_table_size() == 3
    assert w8.lookup_config("FP8_Dynamic", 4, 4096, 4096) == c1
    assert w8.lookup_config("Block_FP8", 32, 4608, 7168, packed=True) == c2
    assert w8.lookup_config("Block_FP8", 32, 4608, 7168, packed=True, op="linear") == c3


def test_m_bucket_fallback(w8):
    """A miss takes the entry of the nearest M in the same floor(log2 M)
    bucket (the larger on a tie) if its config is valid for this M, else the
    cost model's pick."""
    N, K = 4096, 4096
    c4 = w8.Config.make(tile_n=32, waves_k=2, unroll=2, split_k=4, swap_ab=1)
    c6 = w8.Config.make(tile_n=16, waves_k=8, unroll=1, split_k=2)
    c16 = w8.Config.make(tile_n=16, waves_k=1, waves_n=8, unroll=1, split_k=2, x_lds=1)
    w8.set_config("FP8_Dynamic", 4, N, K, c4, 3.0)
    w8.set_config("FP8_Dynamic", 6, N, K, c6, 3.0)
    w8.set_config("FP8_Dynamic", 16, N, K, c16, 3.0)
    assert w8.resolve_config("FP8_Dynamic", 5, N, K) == (c6, 2)    # 5: 4 and 6 tie, larger wins
    assert w8.resolve_config("FP8_Dynamic", 7, N, K) == (c6, 2)
    assert w8.resolve_config("FP8_Dynamic", 4, N, K) == (c4, 1)
    assert w8.resolve_config("FP8_Dynamic", 31, N, K) == (c16, 2)  # bucket 16..31
    assert w8.resolve_config("FP8_Dynamic", 8, N, K) == (w8.model_config("FP8_Dynamic", 8, N, K), 0)
    assert w8.resolve_config("FP8_Dynamic", 32, N, K)[1] == 0      # 32 is a bucket of its own
    assert w8.resolve_config("FP8_Dynamic", 5, N, K, packed=True)[1] == 0
    assert w8.resolve_config("FP8_Dynamic", 5, N, K, op="linear")[1] == 0
    # an entry whose config does not fit this M is skipped: x_lds with the
    # whole K = 4096 of one 16-row block (64 KiB) in LDS fits M = 16; two
    # blocks (M = 17) do not
    big = w8.Config.make(tile_n=16, waves_k=1, waves_n=2, unroll=1, split_k=1, x_lds=1)
    w8.set_config("W8A8_INT8", 16, 512, 4096, big, 2.0)
    w8.validate_config("W8A8_INT8", 16, 512, 4096, big)
    assert not _valid(w8, "W8A8_INT8", 17, 512, 4096, big)
    assert w8.resolve_config("W8A8_INT8", 17, 512, 4096)[1] == 0


def test_model_ranking(w8):
    """The ranked list is the tuner's candidate set, sorted by predicted
    time; its head is the model's pick; every entry is valid; top_n prunes."""
    for fmt, M, N, K, op in (("FP8_Dynamic", 1, 4096, 4096, "gemm"),
                             ("Block_FP8", 32, 4608, 7168, "gemm"),
                             ("W8A8_INT8", 16, 896, 1024, "linear")):
        r = w8.rank_configs(fmt, M, N, K, op=op)
        assert len(r) > 20
        us = [u for u, _ in r]
        assert us == sorted(us) and us[0] > 0
        for _, c in r[:50]:
            w8.validate_config(fmt, M, N, K, c, op=op)
        assert r[0][1] == w8.model_config(fmt, M, N, K, op=op)
        if op == "linear":
            assert any(c.quant_launch == 1 for _, c in r)
            assert any(c.quant_launch == 0 for _, c in r)
        else:
            assert all(c.quant_launch == 0 for _, c in r)


def test_table_malformed_keeps_old_table(w8, tmp_path):
    w8.set_config("W8A8_INT8", 16, 896, 1024, w8.Config.make(), 1.0)
    bad_files = [
        "gfx950 5 W8A8_INT8 gemm row 16 896 1024 16 4 1 2 1 0 0 0 1.0\n",          # too few fields
        "gfx950 5 INT4 gemm row 16 896 1024 16 4 1 2 1 0 0 0 0 1.0\n",               # unknown format
        "gfx950 5 W8A8_INT8 gemm tiled 16 896 1024 16 4 1 2 1 0 0 0 0 1.0\n",        # unknown layout
        "gfx950 5 W8A8_INT8 gemm row 16 896 1024 16 4 1 2 3 0 0 0 0 1.0\n",          # split_k 3
        "gfx950 5 W8A8_INT8 gemm row 40 896 1024 16 4 1 2 1 0 0 0 0 1.0\n",          # M above 32
        "gfx950 5 W8A8_INT8 gemm row 16 896 1024 16 4 1 x 1 0 0 0 0 1.0\n",          # not an integer
        "gfx950 5 W8A8_INT8 gemm row 16 896 1024 16 4 1 2 1 0 0 0 0 fast\n",         # bad time
        "gfx950 5 W8A8_INT8 gemm row 16 896 1024 64 4 1 2 1 0 0 0 0 1.0\n",          # tile 64 x unroll 2
        "gfx950 5 W8A8_INT8 gemm row 16 896 1024 16 2 2 2 1 0 0 0 0 1.0\n",          # waves_k and waves_n
        "gfx950 5 W8A8_INT8 gemm row 16 896 1024 16 1 1 2 2 256 0 0 0 1.0\n",        # grid with split_k
        "gfx950 5 W8A8_INT8 gemm row 16 896 1024 16 1 1 2 1 100000 0 0 0 1.0\n",     # grid > iterations
        "gfx950 5 W8A8_INT8 gemm row 16 896 1024 16 16 1 2 1 0 0 1 0 1.0\n",        # x_lds, 16 waves
        "gfx950 5 W8A8_INT8 fused row 16 896 1024 16 4 1 2 1 0 0 1 0 1.0\n",       # unknown op
        "gfx950 5 W8A8_INT8 linear row 16 896 1024 16 4 1 2 1 0 0 0 0 1.0\n",      # linear without x_lds
        "gfx950 5 W8A8_INT8 linear row 16 896 1024 16 8 1 2 1 0 0 1 0 1.0\n",      # linear, 8 waves_k
        "gfx950 5 W8A8_INT8 linear row 16 896 1024 16 8 1 2 1 0 0 1 2 1.0\n",      # quant_launch 2
        "gfx950 5 W8A8_INT8 gemm row 16 896 1024 16 4 1 2 1 0 0 0 1 1.0\n",        # gemm, quant_launch
    ]
    for i, text in enumerate(bad_files):
        p = tmp_path / f"bad{i}.tbl"
        p.write_text("# header\n" + text)
        with pytest.raises(w8.W8Error) as e:
            w8.load_config_table(str(p))
        assert e.value.status == 4 and "line 2" in str(e.value)
        assert w8.config_table_size() == 1          # old table kept
    with pytest.raises(w8.W8Error) as e:
        w8.load_config_table(str(tmp_path / "missing.tbl"))
    assert e.value.status == 5


def test_table_foreign_entries_ignored_and_kept(w8, tmp_path):
    p = tmp_path / "mixed.tbl"
    p.write_text("gfx942 2 FP8_Dynamic gemm row 4 4096 4096 64 2 1 4 1 0 1 0 2.0\n"
                 "gfx950 9 FP8_Dynamic row 4 4096 4096 64 2 1 4 1 0 1 2.0\n"
                 "gfx950 1 FP8_Dynamic row 4 4096 4096 32 2 2 4 0 2.5\n"
                 "gfx950 2 FP8_Dynamic gemm row 4 4096 4096 32 2 1 2 4 0 0 0 2.5\n"
                 "gfx950 3 FP8_Dynamic gemm row 4 4096 4096 64 2 1 1 4 0 0 0 0 2.5\n"
                 "gfx950 5 FP8_Dynamic gemm row 4 4096 4096 32 2 1 2 4 0 0 0 0 2.5  # native\n")
    w8.load_config_table(str(p))
    assert w8.config_table_size() == 1 and w8.config_table_foreign() == 5
    assert w8.lookup_config("FP8_Dynamic", 4, 4096, 4096) == \
        w8.Config.make(tile_n=32, waves_k=2, unroll=2, split_k=4, swap_ab=0)
    q = tmp_path / "out.tbl"
    w8.save_config_table(str(q))
    text = q.read_text()
    assert "gfx942 2 FP8_Dynamic gemm row" in text and "gfx950 9 FP8_Dynamic row" in text
    assert "gfx950 1 FP8_Dynamic row 4 4096 4096 32 2 2 4 0 2.5" in text   # older ABI, kept
    assert "gfx950 3 FP8_Dynamic gemm row 4 4096 4096 64 2 1 1 4" in text


def test_table_from_environment(tmp_path):
    p = tmp_path / "env.tbl"
    p.write_text("gfx950 5 W8A8_INT8 gemm row 16 896 1024 32 2 1 2 8 0 1 0 0 0.5\n")
    code = ("import bit_quantized_gemm_token_amd as w8;"
            "c = w8.lookup_config('W8A8_INT8', 16, 896, 1024);"
            "print(c.as_dict() if c else None)")
    env = dict(os.environ, W8_CONFIG_TABLE=str(p))
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                         text=True, check=True).stdout
    # the shipped default table is loaded at import and replaces the env table,
    # unless there is none
    from bit_quantized_gemm_token_amd import DEFAULT_TABLE
    if not os.path.exists(DEFAULT_TABLE):
        assert "'split_k': 8" in out and "'tile_n': 32" in out


def test_env_table_loaded_by_the_c_library_alone(tmp_path):
    p = tmp_path / "env.tbl"
    p.write_text("gfx950 5 W8A8_INT8 gemm row 16 896 1024 32 2 1 2 8 0 1 0 0 0.5\n")
    from bit_quantized_gemm_token_amd import _capi
    # load _capi.py on its own (the package __init__ would load the shipped table)
    code = (
        "import ctypes, importlib.util\n"
        f"spec = importlib.util.spec_from_file_location('capi', {os.path.join(ROOT, 'bit_quantized_gemm_token_amd', '_capi.py')!r})\n"
        "_capi = importlib.util.module_from_spec(spec)\n"
        "spec.loader.exec_module(_capi)\n"
        "lib = _capi.load()\n"
        "c = _capi.Config()\n"
        "print(lib.w8_lookup_config(1, 0, 16, 896, 1024, 0, ctypes.byref(c), None), c.split_k, c.tile_n)\n")
    env = dict(os.environ, W8_CONFIG_TABLE=str(p))
    out = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                         check=True).stdout.split()
    assert out == ["0", "8", "32"]


def test_model_fit_uses_library_model(w8):
    """The fitter evaluates the library's own model (w8_predict_us): with its
    starting constants it reproduces the tuner's ranking predictions, so
    those constants are the compiled ones, on every layout; a change of one
    constant moves the prediction; bad rows are refused."""
    from bit_quantized_gemm_token_amd import fit_model as fm
    for fmt, M, N, K, op, lay in (("FP8_Dynamic", 1, 4096, 4096, "gemm", 1),
                                  ("W8A8_INT8", 32, 896, 1040, "gemm", 0),
                                  ("Block_FP8", 17, 4608, 7168, "linear", 1),
                                  ("FP8_Dynamic", 8, 512, 7168, "linear", 0),
                                  ("FP8_Dynamic", 1, 512, 7168, "gemm", 8),
                                  ("W8A8_INT8", 4, 896, 1040, "gemm", 4),
                                  ("Block_FP8", 12, 1792, 5120, "linear", 2)):
        ranked = w8.rank_configs(fmt, M, N, K, op=op, packed=lay, stream_k=True)
        assert ranked, (fmt, M, N, K, op, lay)
        batch = w8.PredictBatch([(fmt, op, lay, M, N, K, c) for _, c in ranked])
        got = batch.run(fm.CURRENT)
        for (us, c), want in zip(ranked, got):
            assert abs(us - want) <= 1e-9 * want, (fmt, M, N, K, op, lay, c, us, want)
        assert list(batch.run()) == [u for u, _ in ranked]
        slower = list(fm.CURRENT)
        slower[0] += 1.0                                   # t0, the fixed launch cost
        assert all(abs(a - b - 1.0) < 1e-9 for a, b in zip(batch.run(slower), got))
    with pytest.raises(w8.W8Error):
        w8.predict_us([("FP8_Dynamic", "gemm", 1, 1, 512, 7168, w8.Config.make(split_k=0))])
    with pytest.raises(w8.W8Error):
        w8.predict_us([("FP8_Dynamic", "gemm", 1, 1, 512, 7168, w8.Config.make())],
                      params=fm.CURRENT[:12])

def test_moe_argument_errors(w8, lib):
    """Validation of the MoE entry point before anything touches a device."""
    L = lib.w8_moe_gemm
    cfg = w8.Config.make(waves_k=4, unroll=1)
    c = ctypes.byref(cfg)

    def call(fmt=0, E=8, T=16, N=64, K=256, max_m=32, xq=FAKE, ldq=256, ldw=256,
             w_stride=64 * 256, sw_stride=64, cfgp=c, ws=None, wsb=0, n_rows=64):
        return L(fmt, E, T, N, K, max_m, xq, ldq, FAKE, FAKE, FAKE, n_rows, FAKE, ldw, w_stride,
                 FAKE, sw_stride, FAKE, 64, cfgp, ws, wsb, None)

    assert call(max_m=33) == 2                       # outside the small-M window
    assert call(E=0) == 1 and call(T=0) == 1
    assert call(xq=None) == 1
    assert call(n_rows=-1) == 1
    assert call(ldq=250) == 1
    assert call(w_stride=64 * 256 - 16) == 1         # experts overlap
    assert call(ldw=0, w_stride=100) == 1            # packed: below one expert's packed size
    assert call(sw_stride=63) == 1
    assert call(fmt=2, sw_stride=1) == 1             # Block_FP8: ceil(N/128) x K/128 = 2
    bad = w8.Config.make(waves_k=16, unroll=1)       # no grouped instance with 16 waves
    assert call(cfgp=ctypes.byref(bad)) == 1 and b"grouped" in lib.w8_last_error()
    sk = w8.Config.make(waves_k=4, unroll=1, split_k=4)
    assert call(cfgp=ctypes.byref(sk)) == 3          # workspace missing
    with pytest.raises(w8.W8Error):
        w8.moe_workspace_size("FP8_Dynamic", 8, 16, 16384 * 16 + 16, 256, 32,
                              w8.Config.make(waves_k=4, unroll=1, split_k=2))


def test_moe_workspace_and_default(w8):
    sk = w8.Config.make(tile_n=16, waves_k=4, unroll=1, split_k=4)
    E, N, K = 8, 300, 1024
    per = (N + 15) // 16 * 4 * 1 * 2 * 1024          # tiles x slots x N blocks x M blocks x 1 KiB
    assert w8.moe_workspace_size("FP8_Dynamic", E, 16, N, K, 32, sk) == \
        COUNTERS + E * ((per + 255) // 256 * 256)
    assert w8.moe_workspace_size("FP8_Dynamic", E, 16, N, K, 32,
                                 w8.Config.make(waves_k=4, unroll=1)) == 0
    for fmt in w8.FORMATS:
        for (E, T, N, K, m) in ((128, 16, 1536, 2048, 32), (8, 1, 4096, 4096, 1),
                                (64, 32, 2048, 768, 16)):
            c, hit = w8.moe_config(fmt, E, T, N, K, m, packed=True)
            assert lib_ok(w8, fmt, E, N, K, m, c) and hit in (0, 1)


def lib_ok(w8, fmt, E, N, K, m, c):
    st = w8._lib.w8_moe_validate_config(w8.FORMATS[fmt], E, N, K, m, 1, ctypes.byref(c))
    return st == 0


def test_moe_table_entries(w8, tmp_path):
    """A "moe" entry keyed by the token count T is what moe_config returns
    when the grouped kernel runs it; otherwise the fallback is used."""
    fmt, E, T, N, K = "FP8_Dynamic", 128, 4, 1536, 2048
    base, hit = w8.moe_config(fmt, E, T, N, K, T, packed=True)
    assert hit == 0
    c = w8.Config.make(tile_n=16, waves_k=4, unroll=2, split_k=1)
    assert c != base
    w8.set_config(fmt, T, N, K, c, 9.5, packed=True, op="moe")
    assert w8.lookup_config(fmt, T, N, K, packed=True, op="moe") == c
    assert w8.lookup_config(fmt, T, N, K, packed=True) is None        # not a GEMM entry
    got, hit = w8.moe_config(fmt, E, T, N, K, T, packed=True)
    assert hit == 1 and got == c
    assert w8.moe_config(fmt, E, T, N, K, T, packed=False)[1] == 0     # other layout
    assert w8.moe_config(fmt, E, 8, N, K, 8, packed=True)[1] == 0      # other T: exact keys only
    # an entry the grouped kernel does not compile (waves_k 16) is passed over
    bad = w8.Config.make(tile_n=16, waves_k=16, unroll=1, split_k=1)
    w8.set_config(fmt, T, N, K, bad, 9.0, packed=True, op="moe")
    got, hit = w8.moe_config(fmt, E, T, N, K, T, packed=True)
    assert hit == 0 and got == base
    w8.set_config(fmt, T, N, K, c, 9.5, packed=True, op="moe")
    p = tmp_path / "m.tbl"
    w8.save_config_table(str(p))
    assert " moe packed 4 1536 2048 " in p.read_text()
    w8.clear_config_table()
    w8.load_config_table(str(p))
    assert w8.moe_config(fmt, E, T, N, K, T, packed=True) == (c, 1)
    with pytest.raises(w8.W8Error):   # grouped configs are checked by the grouped rules
        w8.validate_config(fmt, T, N, K, c, op="moe")
    assert w8._lib.w8_moe_validate_config(w8.FORMATS[fmt], E, N, K, T, 1, ctypes.byref(c)) == 0


def test_moe_tune_argument_errors(w8, lib):
    best, stats = w8.Config(), w8._capi.TuneStats()
    t = lib.w8_moe_tune
    assert t(0, 0, 4, 1536, 2048, 1, None, ctypes.byref(best), ctypes.byref(stats)) == 1   # E
    assert t(0, 8, 4, 1536, 2048, 9, None, ctypes.byref(best), ctypes.byref(stats)) == 1   # topk > E
    assert t(0, 8, 4, 1536, 2048, 0, None, ctypes.byref(best), ctypes.byref(stats)) == 1   # topk
    assert t(0, 8, 33, 1536, 2048, 2, None, ctypes.byref(best), ctypes.byref(stats)) != 0  # T > 32
    assert t(0, 8, 4, 1536, 2048, 2, None, None, ctypes.byref(stats)) == 1                # best


def test_moe_linear_argument_errors_and_config(w8, lib):
    """w8_moe_linear validates its bf16 activations and takes only configs of
    the fused grouped kernel; its default config is valid for every format at
    the benchmark's MoE layers and at a deep K that needs split-K to stage."""
    L = lib.w8_moe_linear
    cfg = w8.Config.make(waves_k=1, waves_n=4, unroll=1, x_lds=1)

    def call(fmt=0, E=8, T=16, N=64, K=256, max_m=32, x=FAKE, ldx=256, cfgp=ctypes.byref(cfg),
             ws=None, wsb=0):
        return L(fmt, E, T, N, K, max_m, x, ldx, FAKE, FAKE, 64, FAKE, 256, 64 * 256, FAKE, 64,
                 FAKE, 64, cfgp, ws, wsb, None)

    assert call(max_m=33) == 2
    assert call(x=None) == 1
    assert call(ldx=250) == 1                        # ldx % 8
    assert call(ldx=248) == 1                        # ldx < K
    for bad in (w8.Config.make(waves_k=1, unroll=1, x_lds=0),     # x_lds 0
                w8.Config.make(waves_k=8, unroll=1, x_lds=1),     # fused: waves_k <= 4
                w8.Config.make(waves_k=2, unroll=1, x_lds=1),     # fused: waves along N only
                # quantize launch: the unfused grouped kernel stages activations
                # only with waves along N
                w8.Config.make(waves_k=2, unroll=1, x_lds=1, quant_launch=1)):
        assert call(cfgp=ctypes.byref(bad)) == 1
    ql = w8.Config.make(waves_k=2, unroll=1, quant_launch=1)
    assert call(cfgp=ctypes.byref(ql)) == 3          # the codes need a workspace
    with pytest.raises(w8.W8Error):                  # quant_launch is no moe_gemm config
        w8.moe_workspace_size("FP8_Dynamic", 8, 16, 64, 256, 32,
                              w8.Config.make(waves_k=2, unroll=1, quant_launch=1, x_lds=2))
    sk = w8.Config.make(waves_k=1, waves_n=4, unroll=1, x_lds=1, split_k=4)
    assert call(cfgp=ctypes.byref(sk)) == 3          # workspace missing
    # workspace sizing accepts a config of either grouped op
    assert w8.moe_workspace_size("FP8_Dynamic", 8, 16, 64, 256, 32, sk) > 0
    for fmt in w8.FORMATS:
        for (E, T, N, K, m) in ((128, 1, 1536, 2048, 1), (128, 32, 2048, 768, 32),
                                (64, 8, 512, 16384, 8)):
            # no table entry: quantize launch + the grouped kernel's own default
            c, hit = w8.moe_linear_config(fmt, E, T, N, K, m, packed=True)
            d, _ = w8.moe_config(fmt, E, T, N, K, m, packed=True)
            assert hit == 0 and c.quant_launch == 1 and c == w8.Config.make(
                **dict(d.as_dict(), quant_launch=1))
            # its workspace holds the T tokens' codes and scales past the counters
            ws = w8.moe_workspace_size(fmt, E, T, N, K, m, c, packed=True)
            ldq = (K + 15) // 16 * 16
            nsx = T * (K // 128) if fmt == "Block_FP8" else T
            r256 = lambda b: (b + 255) // 256 * 256
            shared = w8.moe_workspace_size(fmt, E, T, N, K, m, d, packed=True)
            assert ws == r256(max(shared, COUNTERS)) + r256(T * ldq) + r256(4 * nsx)
    # moe_linear table entries: their own key, the fused rules
    fmt, E, T, N, K = "W8A8_INT8", 128, 4, 1536, 2048
    good = w8.Config.make(tile_n=32, waves_k=1, waves_n=4, unroll=1, x_lds=1)
    w8.set_config(fmt, T, N, K, good, 7.0, packed=True, op="moe_linear")
    assert w8.moe_linear_config(fmt, E, T, N, K, T, packed=True) == (good, 1)
    assert w8.moe_config(fmt, E, T, N, K, T, packed=True)[1] == 0
    with pytest.raises(w8.W8Error):                  # fused entries need x_lds = 1
        w8.set_config(fmt, T, N, K, w8.Config.make(waves_k=2, unroll=1), 7.0, packed=True,
                      op="moe_linear")


def test_segmented_rules(w8):
    """What the K-segmented layouts refuse: staged activation codes, waves
    along N, stream-K, tiles that are not 1, 2 or 4 blocks of 16/T rows, a
    linear op neither fused into LDS nor with a quantize launch, and the
    grouped GEMM."""
    ok = w8.Config.make(tile_n=2, waves_k=2, unroll=2, split_k=1, swap_ab=1)
    w8.validate_config("FP8_Dynamic", 1, 512, 7168, ok, packed=8)
    for bad in (dict(x_lds=1), dict(waves_n=2, x_lds=1, waves_k=1), dict(grid=64, split_k=1),
                dict(tile_n=16), dict(tile_n=3), dict(tile_n=16 * 4)):
        c = w8.Config.make(**{**ok.as_dict(), **bad})
        with pytest.raises(w8.W8Error):
            w8.validate_config("FP8_Dynamic", 1, 512, 7168, c, packed=8)
    with pytest.raises(w8.W8Error):    # fused linear: the activations quantized into LDS
        w8.validate_config("FP8_Dynamic", 1, 512, 7168, ok, op="linear", packed=8)
    w8.validate_config("FP8_Dynamic", 1, 512, 7168, w8.Config.make(**{**ok.as_dict(), "x_lds": 1}),
                       op="linear", packed=8)
    with pytest.raises(w8.W8Error):    # ... with at most 4 K-waves
        w8.validate_config("FP8_Dynamic", 1, 512, 7168,
                           w8.Config.make(**{**ok.as_dict(), "x_lds": 1, "waves_k": 8}),
                           op="linear", packed=8)
    w8.validate_config("FP8_Dynamic", 1, 512, 7168, w8.Config.make(**{**ok.as_dict(), "quant_launch": 1}),
                       op="linear", packed=8)
    with pytest.raises(w8.W8Error):    # a quantize launch's GEMM loads its codes
        w8.validate_config("FP8_Dynamic", 1, 512, 7168,
                           w8.Config.make(**{**ok.as_dict(), "quant_launch": 1, "x_lds": 1}),
                           op="linear", packed=8)
    with pytest.raises(w8.W8Error):
        w8.validate_config("FP8_Dynamic", 4, 512, 7168, ok, op="moe", packed=8)


def test_segmented_defaults_models_and_table(w8, tmp_path):
    """On every K-segmented layout: the default config and the cost model's
    pick are valid configs of the layout at every sweep shape and M up to 32
    (several launches), their workspaces are sized for one launch's token
    groups, entries round-trip through the table file under their layout
    names, and the layout's entries never answer a lookup for another."""
    import synthetic
    for T in (2, 4, 8):
        R = 16 // T
        for fmt in w8.FORMATS:
            for (M, N, K) in synthetic.SWEEP[:6] + ((32, 512, 7168), (3, 530, 1040)):
                if fmt == "Block_FP8" and K % 128:
                    continue
                for op in ("gemm", "linear"):
                    c = w8.default_config(fmt, M, N, K, op=op, packed=T)
                    w8.validate_config(fmt, M, N, K, c, op=op, packed=T)
                    assert c.tile_n == R and c.x_lds == 0 and c.quant_launch == (op == "linear")
                    m = w8.model_config(fmt, M, N, K, packed=T, op=op)
                    w8.validate_config(fmt, M, N, K, m, op=op, packed=T)
                    assert m.tile_n % R == 0 and m.waves_n == 1 and m.grid == 0
        # a split-K config's workspace: counters, then one 1 KiB fragment per
        # (tile, split, block of rows, token group of one launch)
        cfg = w8.Config.make(tile_n=2 * R, waves_k=1, unroll=2, split_k=4, swap_ab=1)
        tiles = -(-512 // (2 * R))
        assert w8.workspace_size("FP8_Dynamic", 32, 512, 7168, cfg, packed=T) == \
            16384 * 128 + tiles * 4 * 2 * 2 * 1024
        assert w8.workspace_size("FP8_Dynamic", 1, 512, 7168, cfg, packed=T) == \
            16384 * 128 + tiles * 4 * 2 * 1 * 1024
    w8.clear_config_table()
    try:
        c8 = w8.Config.make(tile_n=2, waves_k=1, unroll=4, split_k=1, swap_ab=1)
        c2 = w8.Config.make(tile_n=8, waves_k=8, unroll=1, split_k=1, swap_ab=1)
        w8.set_config("FP8_Dynamic", 1, 512, 7168, c8, 2.8, packed=8)
        w8.set_config("FP8_Dynamic", 8, 896, 5120, c2, 4.3, packed="seg2")
        w8.set_config("FP8_Dynamic", 1, 512, 7168, w8.Config.make(split_k=8), 4.1, packed=True)
        with pytest.raises(w8.W8Error):            # a plain config is no layout-8 config
            w8.set_config("FP8_Dynamic", 1, 512, 7168, w8.Config.make(split_k=8), 4.1, packed=8)
        p = tmp_path / "seg.tbl"
        w8.save_config_table(str(p))
        text = p.read_text()
        assert " FP8_Dynamic gemm seg8 1 512 7168 2 1 1 4 1 0 1 0 0 " in text
        assert " FP8_Dynamic gemm seg2 8 896 5120 8 8 1 1 1 0 1 0 0 " in text
        w8.clear_config_table()
        w8.load_config_table(str(p))
        assert w8.lookup_config("FP8_Dynamic", 1, 512, 7168, packed=8) == c8
        assert w8.lookup_config("FP8_Dynamic", 8, 896, 5120, packed=2) == c2
        assert w8.lookup_config("FP8_Dynamic", 8, 896, 5120, packed=4) is None
        assert w8.resolve_config("FP8_Dynamic", 1, 512, 7168, packed=8) == (c8, 1)
        assert w8.best_layout("FP8_Dynamic", 1, 512, 7168) == 8
        bad = tmp_path / "bad.tbl"
        bad.write_text("gfx950 5 FP8_Dynamic gemm seg8 1 512 7168 2 1 1 4 1 0 1 1 0 1.0\n")
        with pytest.raises(w8.W8Error):             # x_lds on a K-segmented layout
            w8.load_config_table(str(bad))
        bad.write_text("gfx950 5 FP8_Dynamic gemm seg3 1 512 7168 2 1 1 4 1 0 1 0 0 1.0\n")
        with pytest.raises(w8.W8Error):
            w8.load_config_table(str(bad))
        assert w8.lookup_config("FP8_Dynamic", 1, 512, 7168, packed=8) == c8   # old table kept
    finally:
        w8.clear_config_table()
        w8.load_default_table()
