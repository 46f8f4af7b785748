"""Pins for the oracle's GEMM (CPU only).

Pinned against numpy integer / float64 matmul (exact at these magnitudes),
an exact Fraction triple loop, closed forms (all-ones, all-max, identity,
permutation and one-hot operands) and invariants (scale linearity, Block_FP8
with uniform scales reducing to the per-token result, K-range additivity).
"""
from fractions import Fraction

import numpy as np
import pytest

import synthetic
from tests import exact


def _rand_e4m3(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3C                      # replace NaN codes
    return c


def test_acc_int8_matches_numpy(oracle_mod):
    rng = np.random.default_rng(0)
    x = rng.integers(-127, 128, size=(5, 300), dtype=np.int8)
    w = rng.integers(-127, 128, size=(37, 300), dtype=np.int8)
    C = oracle_mod.acc_int8(x, w)
    assert (C == x.astype(np.int64) @ w.astype(np.int64).T).all()
    C2 = oracle_mod.acc_int8(x, w, 64, 200)
    assert (C2 == x[:, 64:200].astype(np.int64) @ w[:, 64:200].astype(np.int64).T).all()


def test_acc_fp8_matches_numpy_float64(oracle_mod):
    # every partial sum is a multiple of 2^-18 below 2^31: float64 matmul is exact
    rng = np.random.default_rng(1)
    x = _rand_e4m3(rng, (6, 512))
    w = _rand_e4m3(rng, (19, 512))
    D = oracle_mod.acc_fp8(x, w)
    t = exact.torch_e4m3_table()
    ref = t[x] @ t[w].T
    assert (D == ref).all()


def test_acc_fp8_rejects_nan_codes(oracle_mod):
    x = np.full((1, 16), 0x38, dtype=np.uint8)
    w = np.full((1, 16), 0x38, dtype=np.uint8)
    w[0, 3] = 0x7F
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.acc_fp8(x, w)


def _fraction_gemm(fmt, xq, sx, wq, sw):
    t = exact.torch_e4m3_table()
    M, K = xq.shape
    N = wq.shape[0]
    dec_x = (lambda c: Fraction(int(np.int8(np.uint8(c).view(np.int8))))) if fmt == "W8A8_INT8" \
        else (lambda c: Fraction(float(t[c])))
    out = np.zeros((M, N), dtype=object)
    mag = np.zeros((M, N), dtype=object)             # sum of |group terms| (rounding scale)
    for m in range(M):
        for n in range(N):
            if fmt == "Block_FP8":
                tot = Fraction(0)
                absum = Fraction(0)
                for g in range(K // 128):
                    d = sum(dec_x(xq[m, k]) * dec_x(wq[n, k]) for k in range(128 * g, 128 * g + 128))
                    term = Fraction(float(sx[m, g])) * Fraction(float(sw[n // 128, g])) * d
                    tot += term
                    absum += abs(term)
                out[m, n] = tot
                mag[m, n] = absum
            else:
                d = sum(dec_x(xq[m, k]) * dec_x(wq[n, k]) for k in range(K))
                out[m, n] = d * Fraction(float(sx[m])) * Fraction(float(sw[n]))
                mag[m, n] = abs(out[m, n])
    return out, mag


@pytest.mark.parametrize("fmt", ["W8A8_INT8", "FP8_Dynamic", "Block_FP8"])
def test_gemm_fraction_brute_force(oracle_mod, fmt):
    M, N, K = 3, 4, 256
    x = synthetic.activations(fmt, M, N, K)
    xq, sx = oracle_mod.quantize_act(fmt, x)
    if fmt == "W8A8_INT8":
        wq, sw = synthetic.int8_weights(fmt, M, N, K)
        wq = wq.view(np.uint8)
    else:
        wq, sw = oracle_mod.quantize_weight(fmt, synthetic.fp32_weights(fmt, M, N, K))
    Y = oracle_mod.gemm(fmt, xq, sx, wq, sw)
    ref, mag = _fraction_gemm(fmt, xq, sx, wq, sw)
    # fp64 scale products and group sums: a few roundings of 2^-53 each, relative
    # to the sum of the magnitudes of the terms
    for m in range(M):
        for n in range(N):
            r = float(ref[m, n])
            assert abs(Y[m, n] - r) <= 1e-15 * float(mag[m, n]) + 1e-300, (m, n, Y[m, n], r)


@pytest.mark.parametrize("fmt,one,big,qmax", [("W8A8_INT8", 1, 127, 127),
                                              ("FP8_Dynamic", 0x38, 0x7E, 448)])
def test_gemm_closed_form_all_ones_all_max(oracle_mod, fmt, one, big, qmax):
    M, N, K = 4, 8, 8192
    rng = np.random.default_rng(2)
    sx = rng.uniform(0.01, 1, M).astype(np.float32)
    sw = rng.uniform(0.001, 0.01, N).astype(np.float32)
    xq = np.full((M, K), one, dtype=np.uint8)
    wq = np.full((N, K), one, dtype=np.uint8)
    Y = oracle_mod.gemm(fmt, xq, sx, wq, sw)
    assert (Y == K * sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]).all()
    xq[:] = big
    wq[:] = big
    wq[1::2] = big | 0x80 if fmt != "W8A8_INT8" else np.uint8(np.int8(-127).view(np.uint8))
    Y = oracle_mod.gemm(fmt, xq, sx, wq, sw)
    sign = np.where(np.arange(N) % 2 == 1, -1.0, 1.0)
    want = K * qmax * qmax * sx.astype(np.float64)[:, None] * (sign * sw.astype(np.float64))[None, :]
    assert (Y == want).all()
    # K * 448^2 = 49 * 2^25 at K = 8192: exactly representable even in fp32
    assert float(np.float32(K * qmax * qmax)) == K * qmax * qmax


def test_gemm_identity_and_permutation_int8(oracle_mod):
    M, K = 5, 64
    x = synthetic.activations("W8A8_INT8", M, K, K)
    xq, sx = oracle_mod.quantize_act("W8A8_INT8", x)
    eye = np.eye(K, dtype=np.int8).view(np.uint8)
    Y = oracle_mod.gemm("W8A8_INT8", xq, sx, eye, np.ones(K, np.float32))
    assert (Y == xq.view(np.int8).astype(np.float64) * sx.astype(np.float64)[:, None]).all()
    perm = np.random.default_rng(3).permutation(K)
    P = np.zeros((K, K), dtype=np.int8)
    P[np.arange(K), perm] = 1                        # output column n picks input column perm[n]
    Yp = oracle_mod.gemm("W8A8_INT8", xq, sx, P.view(np.uint8), np.ones(K, np.float32))
    assert (Yp == Y[:, perm]).all()


def test_gemm_identity_blocks_block_fp8(oracle_mod):
    # identity weight codes (1.0 = 0x38) with unit block scales return dequant(Xq)
    M, K = 3, 256
    x = synthetic.activations("Block_FP8", M, K, K)
    xq, sx = oracle_mod.quantize_act("Block_FP8", x)
    wq = np.where(np.eye(K, dtype=bool), 0x38, 0x00).astype(np.uint8)
    sw = np.ones((2, 2), np.float32)
    Y = oracle_mod.gemm("Block_FP8", xq, sx, wq, sw)
    deq = oracle_mod.e4m3_decode(xq) * np.repeat(sx.astype(np.float64), 128, axis=1)
    assert (Y == deq).all()


def test_gemm_one_hot_places_single_value(oracle_mod):
    # one-hot rows and columns: only Y[m0, n0] is nonzero (orientation check)
    M, N, K = 7, 9, 128
    for fmt, code in (("W8A8_INT8", 3), ("FP8_Dynamic", 0x40), ("Block_FP8", 0x40)):
        xq = np.zeros((M, K), np.uint8)
        wq = np.zeros((N, K), np.uint8)
        xq[5, 77] = code
        wq[2, 77] = code
        sx = np.ones((M, 1) if fmt == "Block_FP8" else (M,), np.float32)
        sw = np.ones((1, 1) if fmt == "Block_FP8" else (N,), np.float32)
        Y = oracle_mod.gemm(fmt, xq, sx, wq, sw)
        want = 9.0 if fmt == "W8A8_INT8" else 4.0
        assert Y[5, 2] == want
        Y[5, 2] = 0
        assert (Y == 0).all()


def test_gemm_scale_linearity(oracle_mod):
    M, N, K = 4, 6, 256
    for fmt in ("W8A8_INT8", "FP8_Dynamic", "Block_FP8"):
        x = synthetic.activations(fmt, M, N, K)
        xq, sx = oracle_mod.quantize_act(fmt, x)
        if fmt == "W8A8_INT8":
            wq, sw = synthetic.int8_weights(fmt, M, N, K)
            wq = wq.view(np.uint8)
        else:
            wq, sw = oracle_mod.quantize_weight(fmt, synthetic.fp32_weights(fmt, M, N, K))
        Y = oracle_mod.gemm(fmt, xq, sx, wq, sw)
        Y2 = oracle_mod.gemm(fmt, xq, sx, wq, sw * np.float32(2))
        assert (Y2 == 2 * Y).all()


def test_block_fp8_uniform_scales_reduce_to_token_format(oracle_mod):
    M, N, K = 4, 130, 512
    rng = np.random.default_rng(9)
    xq = _rand_e4m3(rng, (M, K))
    wq = _rand_e4m3(rng, (N, K))
    sx_tok = rng.uniform(0.01, 1, M).astype(np.float32)
    c = np.float32(0.0037)
    Yb = oracle_mod.gemm("Block_FP8", xq, np.repeat(sx_tok[:, None], K // 128, axis=1),
                         wq, np.full((2, K // 128), c, np.float32))
    Yt = oracle_mod.gemm("FP8_Dynamic", xq, sx_tok, wq, np.full(N, c, np.float32))
    np.testing.assert_allclose(Yb, Yt, rtol=1e-13, atol=0)


def test_k_range_additivity(oracle_mod):
    # split-K partial sums over any partition of K add up to the whole (exactly)
    rng = np.random.default_rng(4)
    xi = rng.integers(-127, 128, size=(3, 448), dtype=np.int8)
    wi = rng.integers(-127, 128, size=(5, 448), dtype=np.int8)
    cuts = [0, 64, 65, 300, 448]
    parts = sum(oracle_mod.acc_int8(xi, wi, a, b) for a, b in zip(cuts[:-1], cuts[1:]))
    assert (parts == oracle_mod.acc_int8(xi, wi)).all()
    xf = _rand_e4m3(rng, (3, 448))
    wf = _rand_e4m3(rng, (5, 448))
    parts = sum(oracle_mod.acc_fp8(xf, wf, a, b) for a, b in zip(cuts[:-1], cuts[1:]))
    assert (parts == oracle_mod.acc_fp8(xf, wf)).all()


def test_int8_accumulator_range_guard(oracle_mod):
    # the int32 bound holds for every K the library accepts at full magnitude
    K = 8192
    assert K * 127 * 127 < 2 ** 31
    xq = np.full((1, K), 127, np.uint8)
    Y = oracle_mod.gemm("W8A8_INT8", xq, np.ones(1, np.float32), xq, np.ones(1, np.float32))
    assert Y[0, 0] == K * 127 * 127
