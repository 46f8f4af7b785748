"""w8_gemm_w8a8_noalloc, through the C-ABI: the same output as w8_gemm_w8a8
with a caller workspace, bit for bit, for two calls in a row (the second
smaller, so it runs on what the first left in the library's scratch array),
with configs that share output tiles (split-K, stream-K: the scratch is used)
and the table's config; a config that needs more scratch than the array
holds is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from tests.gpu_cases import DEV, Case, assert_bf16_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w8():
    import bit_quantized_gemm_token_amd as mod
    return mod


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def noalloc(w8, fmt, xq, sx, wq, sw, cfg):
    M, K = xq.shape
    if isinstance(wq, w8.PackedWeight):
        N, ldw, wt = wq.N, 0, wq.data
    else:
        N, ldw, wt = wq.shape[0], wq.stride(0), wq
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    st = w8._lib.w8_gemm_w8a8_noalloc(
        w8.FORMATS[fmt], M, N, K, _p(xq), xq.stride(0), _p(sx), _p(wt), ldw, _p(sw), _p(y), N,
        ctypes.byref(cfg) if cfg is not None else None,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, w8._lib.w8_last_error().decode()
    return y


CASES = [
    # (fmt, M, N, K, config of the first call) then a smaller second call
    ("FP8_Dynamic", 16, 512, 7168, dict(tile_n=16, waves_k=1, unroll=4, split_k=8)),
    ("W8A8_INT8", 32, 896, 5120, dict(tile_n=16, waves_k=2, unroll=2, split_k=16, swap_ab=1)),
    ("Block_FP8", 8, 1792, 5120, dict(tile_n=16, waves_k=1, waves_n=4, unroll=2, grid=300)),
]
SECOND = [("FP8_Dynamic", 3, 256, 2048, dict(tile_n=16, waves_k=2, unroll=2, split_k=4)),
          ("W8A8_INT8", 5, 272, 640, dict(tile_n=16, waves_k=1, unroll=1, split_k=2)),
          ("Block_FP8", 1, 384, 1024, None)]


@pytest.mark.parametrize("i", range(len(CASES)))
def test_noalloc_matches_workspace_entry(w8, i):
    for fmt, M, N, K, kw in (CASES[i], SECOND[i]):
        print(f"[noalloc] {fmt} M={M} N={N} K={K} {kw}", flush=True)
        cs = Case(fmt, M, N, K)
        xq, sx = cs.gpu_act()
        cfg = w8.Config.make(**kw) if kw is not None else None
        for packed in (False, True):
            wq = cs.weights(packed)
            ref = w8.gemm_w8a8(fmt, xq, sx, wq, cs.sw, cfg=cfg)
            got = noalloc(w8, fmt, xq, sx, wq, cs.sw, cfg)
            again = noalloc(w8, fmt, xq, sx, wq, cs.sw, cfg)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"{fmt} {kw}"
            assert torch.equal(again.view(torch.int16), ref.view(torch.int16)), f"{fmt} {kw}"
        assert_bf16_close(got, cs.Y, f"noalloc {fmt} {M}x{N}x{K}")


def test_noalloc_refuses_what_does_not_fit(w8):
    M, N, K = 4, 1 << 16, 4096
    cfg = w8.Config.make(tile_n=16, waves_k=1, unroll=1, split_k=256)
    need = w8.workspace_size("FP8_Dynamic", M, N, K, cfg)
    assert need > 16 << 20
    z = torch.zeros(16, dtype=torch.uint8, device=DEV)
    st = w8._lib.w8_gemm_w8a8_noalloc(0, M, N, K, _p(z), K, _p(z), _p(z), K, _p(z), _p(z), N,
                                      ctypes.byref(cfg), None)
    assert st == 3                                   # W8_E_WORKSPACE, nothing launched
    assert b"no-allocation" in w8._lib.w8_last_error()
