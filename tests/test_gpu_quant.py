"""GPU quantizers against the oracle: codes and scales byte-identical.

Includes a dense check of the hardware E4M3FN conversion (rounding ties,
subnormals, signed zero) and of int8 rounding ties on gfx950.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests.gpu_cases import DEV, to_bf16_tensor, u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w8():
    import bit_quantized_gemm_token_amd as mod
    return mod


TOKEN_SHAPES = [(1, 16), (1, 1024), (5, 208), (16, 1024), (32, 8192), (3, 9008), (32, 7168),
                (4, 640), (2, 4096)]
BLOCK_SHAPES = [(1, 128), (5, 384), (8, 7168), (32, 7168), (32, 8192), (3, 10240)]


def _act_case(w8, fmt, M, K, bits=None):
    print(f"[quant] {fmt} M={M} K={K}", flush=True)
    if bits is None:
        bits = synthetic.activations(fmt, M, 1, K)
    xq, sx = w8.quantize_act(fmt, to_bf16_tensor(bits))
    torch.cuda.synchronize()
    xq_ref, sx_ref = oracle.quantize_act(fmt, bits)
    assert np.array_equal(u8(xq), xq_ref), f"codes differ at {np.argwhere(u8(xq) != xq_ref)[:5]}"
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), sx_ref.view(np.uint32))


@pytest.mark.parametrize("fmt", ["FP8_Dynamic", "W8A8_INT8"])
@pytest.mark.parametrize("M,K", TOKEN_SHAPES)
def test_quantize_act_token_formats(w8, fmt, M, K):
    _act_case(w8, fmt, M, K)


@pytest.mark.parametrize("M,K", BLOCK_SHAPES)
def test_quantize_act_block(w8, M, K):
    _act_case(w8, "Block_FP8", M, K)


@pytest.mark.parametrize("fmt", ["FP8_Dynamic", "W8A8_INT8", "Block_FP8"])
def test_quantize_act_zero_rows_and_groups(w8, fmt):
    bits = synthetic.activations(fmt, 6, 1, 512)
    bits[2] = 0
    bits[4, 128:256] = 0           # one all-zero group in a nonzero row
    bits[5, :] = 0x8000            # -0.0 everywhere
    _act_case(w8, fmt, 6, 512, bits)


@pytest.mark.parametrize("fmt", ["FP8_Dynamic", "W8A8_INT8", "Block_FP8"])
def test_quantize_act_extreme_magnitudes(w8, fmt):
    """Rows scaled by 2^-124 .. 2^120, with subnormal entries and negative
    zeros: scales below 2^-100 (divided), just above it (reciprocal with an
    FMA correction, subnormal x), and near the top of the bf16 range."""
    M, K = 21, 1024
    _act_case(w8, fmt, M, K, synthetic.activations_extreme(fmt, M, K))


def test_int8_round_ties(w8):
    # amax 127 gives s = 1, so x / s = x: every k + 0.5 is an exact tie
    vals = np.concatenate([[127.0], np.arange(-126.5, 127.0, 1.0), [-0.0, 0.5, -0.5]])
    K = (len(vals) + 15) // 16 * 16
    row = np.zeros(K, np.float32)
    row[:len(vals)] = vals
    bits = synthetic.fp32_to_bf16_bits(row[None, :])
    assert np.array_equal(synthetic.bf16_bits_to_fp32(bits)[0], row)   # all exact in bf16
    _act_case(w8, "W8A8_INT8", 1, K, bits)


def _e4m3_dense_values():
    t = torch.arange(0x7F, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    vals = t.to(torch.float64).numpy()
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    pts = np.concatenate([vals.astype(np.float32), mids])
    pts = np.concatenate([pts, np.nextafter(pts, np.float32(0)), np.nextafter(pts, np.float32(500))])
    rng = np.random.default_rng(99)
    rnd = (2.0 ** rng.uniform(-13, np.log2(448), 1_500_000)).astype(np.float32)
    sub = rng.uniform(0, 2 ** -6, 200_000).astype(np.float32)
    pos = np.concatenate([pts, rnd, sub])
    pos = pos[(pos >= 0) & (pos <= 448)]
    return np.concatenate([pos, -pos, np.array([0.0, -0.0], np.float32)])


def test_e4m3_conversion_dense(w8):
    """Hardware fp32 -> E4M3FN conversion vs the oracle encoder on ~3.4M values.

    Rows of the FP8_Dynamic weight quantizer whose amax is 448 have s = 1, so
    their codes are the encodings of the fp32 values themselves."""
    v = _e4m3_dense_values()
    C = 8192
    R = (len(v) + C - 2) // (C - 1)
    w = np.zeros((R, C), np.float32)
    w[:, 0] = 448.0
    flat = np.zeros(R * (C - 1), np.float32)
    flat[:len(v)] = v
    w[:, 1:] = flat.reshape(R, C - 1)
    print(f"[quant] dense e4m3 conversion: {len(v)} values", flush=True)
    wq, sw = w8.quantize_weight("FP8_Dynamic", torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    assert (sw.cpu().numpy() == 1.0).all()
    got = u8(wq)
    want = oracle.e4m3_encode(w)
    bad = np.argwhere(got != want)
    assert bad.size == 0, [(float(w[tuple(i)]), hex(got[tuple(i)]), hex(want[tuple(i)]))
                           for i in bad[:10]]


@pytest.mark.parametrize("fmt,N,K", [("FP8_Dynamic", 4096, 4096), ("FP8_Dynamic", 37, 200),
                                     ("Block_FP8", 4608, 7168), ("Block_FP8", 130, 200),
                                     ("Block_FP8", 512, 7168)])
def test_quantize_weight(w8, fmt, N, K):
    print(f"[quant] weight {fmt} N={N} K={K}", flush=True)
    w = synthetic.fp32_weights(fmt, 1, N, K)
    wq, sw = w8.quantize_weight(fmt, torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    wq_ref, sw_ref = oracle.quantize_weight(fmt, w)
    assert np.array_equal(u8(wq), wq_ref)
    assert np.array_equal(sw.cpu().numpy().view(np.uint32), sw_ref.view(np.uint32))


def test_quantize_act_strided(w8):
    # x and xq with row strides larger than K
    bits = synthetic.activations("FP8_Dynamic", 4, 1, 512)
    xbig = torch.zeros((4, 640), dtype=torch.bfloat16, device=DEV)
    xbig[:, :512] = to_bf16_tensor(bits)
    xq = torch.zeros((4, 528), dtype=torch.uint8, device=DEV)
    _, sx = w8.quantize_act("FP8_Dynamic", xbig[:, :512], xq=xq[:, :512])
    torch.cuda.synchronize()
    xq_ref, sx_ref = oracle.quantize_act("FP8_Dynamic", bits)
    assert np.array_equal(xq[:, :512].cpu().numpy(), xq_ref)
    assert (xq[:, 512:].cpu().numpy() == 0).all()          # nothing written past K
    assert np.array_equal(sx.cpu().numpy(), sx_ref)
